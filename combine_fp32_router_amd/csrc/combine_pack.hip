// Combine of one chunk and dispatch pack of the next, in one launch.
//
// What it computes: exactly what moe_combine does for chunk A followed by
// moe_dispatch_pack for chunk B (both are defined in combine.hip and
// dispatch_pack.hip); the two touch disjoint buffers, so their order does
// not matter.  The batch is processed in chunks and the work of neighbouring
// chunks overlaps (ThunderEP write-up s2.2): here the combine of chunk c and
// the pack of chunk c+1 share one grid.
//
// gfx950 design.  Blocks [0, Tc) run the combine body of tokens 0..Tc-1 and
// blocks [Tc, Tc+Tp) the pack body of tokens 0..Tp-1, the same per-token
// code as the standalone kernels, so results are bit for bit those of the
// two separate launches.  Workgroups are dispatched in index order: the pack
// blocks start as the combine blocks drain, so the combine's tail and the
// pack's ramp-up overlap instead of each launch paying its own (dsv3 bf16,
// 8 chunks: 4% less time per step than 16 separate launches).  Two other
// orders measured slower: alternating the kinds block by block (their reads
// and writes then contend for the whole launch) and packing first (the
// combine's reads then queue behind the pack's write stream).
//
// With streaming send stores (ST, MOE_PACK_STREAM: the rows are not kept in
// the last-level cache, nor is anything this launch reads), combine block b
// also loads the hidden row of pack token b into the caches (prefetch_row in
// combine_rows.hpp; no extra HBM bytes, the pack half reads the same row),
// so the pack blocks find it there rather than waiting on HBM before their
// k stores: the merged launch of the T=16384, H=7168 step went from 95.3 to
// 92.0 us (bf16) and from 104.5 to 100.9 us (int8) when its combine reads
// rows packed a step earlier (int4 unchanged).  Without ST the cache holds
// the send rows the combine is about to read, and nothing is prefetched.
#include "combine_rows.hpp"
#include "launch.hpp"
#include "pack_rows.hpp"

namespace moe {
namespace {

template <int VPT, bool ST>
__global__ __launch_bounds__(1024) void combine_pack_bf16_kernel(
    const u32x4 *__restrict__ ret, const int32_t *__restrict__ cpos, const float *__restrict__ w,
    int64_t Tc, u32x4 *__restrict__ out, const u32x4 *__restrict__ x,
    const int32_t *__restrict__ ppos, u32x4 *__restrict__ send, int HV, int k)
{
    const int64_t b = blockIdx.x;
    const int64_t Tp = static_cast<int64_t>(gridDim.x) - Tc;
    if (b < Tc)  // ST: prefetch the hidden row of pack token b (none when Tp == 0)
        combine_bf16_row<VPT, ST>(b, ret, cpos, w, HV, k, out,
                                  Tp > 0 ? x + (b < Tp ? b : Tp - 1) * HV : x,
                                  Tp > 0 ? HV * 16 : 0);
    else
        pack_bf16_row<VPT, ST>(b - Tc, x, HV, k, ppos, send);
}

template <int VPT, bool FP8, bool ST>
__global__ __launch_bounds__(1024) void combine_pack_byte_kernel(
    const u32x4 *__restrict__ ret, const float *__restrict__ rscales,
    const int32_t *__restrict__ cpos, const float *__restrict__ w, int64_t Tc,
    u32x4 *__restrict__ out, const u32x4 *__restrict__ x, const int32_t *__restrict__ ppos,
    u32x4 *__restrict__ send, float *__restrict__ sscales, int G, int k)
{
    const int64_t b = blockIdx.x;
    const int64_t Tp = static_cast<int64_t>(gridDim.x) - Tc;
    if (b < Tc)
        combine_byte_row<VPT, FP8, ST>(b, ret, rscales, cpos, w, G, k, out,
                                       Tp > 0 ? x + (b < Tp ? b : Tp - 1) * 2 * G : x,
                                       Tp > 0 ? G * 32 : 0);
    else
        pack_byte_row<VPT, FP8, ST>(b - Tc, x, G, k, ppos, send, sscales);
}

// int4: combine and pack both take 16 elements per thread, so the pack half
// uses every thread of the combine's block.
template <int VPT, bool ST>
__global__ __launch_bounds__(1024) void combine_pack_int4_kernel(
    const u32x2 *__restrict__ ret, const float *__restrict__ rscales,
    const int32_t *__restrict__ cpos, const float *__restrict__ w, int64_t Tc,
    u32x4 *__restrict__ out, const u32x4 *__restrict__ x, const int32_t *__restrict__ ppos,
    u32x2 *__restrict__ send, float *__restrict__ sscales, int G, int k)
{
    const int64_t b = blockIdx.x;
    const int64_t Tp = static_cast<int64_t>(gridDim.x) - Tc;
    if (b < Tc)
        combine_int4_row<VPT, ST>(b, ret, rscales, cpos, w, G, k, out,
                                  Tp > 0 ? x + (b < Tp ? b : Tp - 1) * 2 * G : x,
                                  Tp > 0 ? G * 32 : 0);
    else
        pack_int4_row<VPT, ST>(b - Tc, x, G, k, ppos, send, sscales);
}

template <bool ST>
hipError_t combine_pack_launch(const void *recv, const float *rscales, const int32_t *pos_c,
                               const float *w, int64_t Tc, void *out, const void *x,
                               const int32_t *pos_p, int64_t Tp, void *send, float *sscales,
                               int H, int k, int quant, hipStream_t stream)
{
    const dim3 grid(static_cast<unsigned>(Tc + Tp));
    u32x4 *ov = static_cast<u32x4 *>(out);
    const u32x4 *xv = static_cast<const u32x4 *>(x);
    u32x4 *sv = static_cast<u32x4 *>(send);
    if (quant == 0) {
        const int HV = H / 8;
        const RowTiling rt = row_tiling(HV);
        const dim3 block(rt.threads);
        const u32x4 *rv = static_cast<const u32x4 *>(recv);
#define MOE_CP_BF16(V)                                                                         \
    combine_pack_bf16_kernel<V, ST><<<grid, block, 0, stream>>>(rv, pos_c, w, Tc, ov, xv, pos_p, \
                                                                sv, HV, k)
        switch (rt.vpt) {
        case 1: MOE_CP_BF16(1); break;
        case 2: MOE_CP_BF16(2); break;
        case 4: MOE_CP_BF16(4); break;
        default: MOE_CP_BF16(8); break;
        }
#undef MOE_CP_BF16
    } else if (quant == 2) {
        const int G = H / 16;
        const RowTiling ct = row_tiling(G);
        const dim3 block(ct.threads);
        const u32x2 *rv = static_cast<const u32x2 *>(recv);
        u32x2 *s2 = static_cast<u32x2 *>(send);
#define MOE_CP_INT4(V)                                                                         \
    combine_pack_int4_kernel<V, ST><<<grid, block, 0, stream>>>(rv, rscales, pos_c, w, Tc, ov,  \
                                                                xv, pos_p, s2, sscales, G, k)
        switch (ct.vpt) {
        case 1: MOE_CP_INT4(1); break;
        case 2: MOE_CP_INT4(2); break;
        default: MOE_CP_INT4(4); break;
        }
#undef MOE_CP_INT4
    } else {
        const int G = H / 16;
        const RowTiling gt = row_tiling(G);
        const dim3 block(gt.threads);
        const u32x4 *rv = static_cast<const u32x4 *>(recv);
#define MOE_CP_BYTE(V, F)                                                                      \
    combine_pack_byte_kernel<V, F, ST><<<grid, block, 0, stream>>>(rv, rscales, pos_c, w, Tc, ov, \
                                                                   xv, pos_p, sv, sscales, G, k)
        if (quant == 1) {
            switch (gt.vpt) {
            case 1: MOE_CP_BYTE(1, false); break;
            case 2: MOE_CP_BYTE(2, false); break;
            default: MOE_CP_BYTE(4, false); break;
            }
        } else {
            switch (gt.vpt) {
            case 1: MOE_CP_BYTE(1, true); break;
            case 2: MOE_CP_BYTE(2, true); break;
            default: MOE_CP_BYTE(4, true); break;
            }
        }
#undef MOE_CP_BYTE
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_combine_pack(const void *recv, const float *rscales, const int32_t *pos_c,
                               const float *w, int64_t Tc, void *out, const void *x,
                               const int32_t *pos_p, int64_t Tp, void *send, float *sscales,
                               int H, int k, int quant, bool stream_stores, hipStream_t stream)
{
    if (Tc == 0)
        return Tp == 0 ? hipSuccess
                       : launch_dispatch_pack(x, Tp, H, k, pos_p, quant, stream_stores, send,
                                              sscales, stream);
    if (Tp == 0)
        return launch_combine(recv, rscales, quant, pos_c, w, Tc, H, k, out, stream);
    return stream_stores
               ? combine_pack_launch<true>(recv, rscales, pos_c, w, Tc, out, x, pos_p, Tp, send,
                                           sscales, H, k, quant, stream)
               : combine_pack_launch<false>(recv, rscales, pos_c, w, Tc, out, x, pos_p, Tp, send,
                                            sscales, H, k, quant, stream);
}

}  // namespace moe
