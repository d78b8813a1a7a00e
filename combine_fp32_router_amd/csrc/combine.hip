// Combine: gather each token's returned rows, dequantise (bf16, int8, int4
// or fp8 records), and form the gate-weighted sum back in token order.
//
// What it computes (ThunderEP write-up s1.3: expert results go back to the
// token's GPU, which takes the weighted sum over the token's k experts):
//   out[t,h] = bf16_rne( sum_{j<k, pos[t,j] >= 0} w[t,j] * deq(ret[pos[t,j]])[h] )
// with fp32 accumulation in slot order j = 0..k-1, starting from -0 (the
// IEEE identity of addition, so one kept term passes through bit for bit).
// Dropped slots add nothing, the remaining weights are not renormalised, and
// a token with every slot dropped gets +0.
//
// gfx950 design.  One block per token, each thread owning `VPT` 16-byte
// output vectors (8 elements).  The token's k rows and weights arrive with
// one vector load each (lane j holds slot j's) and are read back with
// v_readlane rather than as a chain of dependent scalar loads before each
// group of row gathers (measured the same); the (int8 / int4 / fp8) scales
// are block-uniform scalar loads from the scale array.  Rows are fetched in groups
// of kLoadsPerLane/VPT slots whose loads are issued before the first FMA.
// Few loads per lane keep VGPRs low, so many waves (896-thread blocks at
// H=7168) stay resident and the CU as a whole keeps the read stream full;
// on MI355X two bf16 loads per lane measured faster than four or eight,
// while the int8 / fp8 rows (half the bytes per load) do best with all
// eight of a token's rows in flight and int4 with four.  The read stream is
// what bounds the kernel (HBM).  Output rows are written with nontemporal
// stores: device-scope and default-policy stores measured 2-26% slower for
// the T=16384, H=7168 step, with or without the rows in the cache.
#include "combine_rows.hpp"
#include "launch.hpp"

namespace moe {
namespace {

template <int VPT>
__global__ __launch_bounds__(1024) void combine_bf16_kernel(const u32x4 *__restrict__ ret,
                                                            const int32_t *__restrict__ pos,
                                                            const float *__restrict__ w, int HV,
                                                            int k, u32x4 *__restrict__ out)
{
    combine_bf16_row<VPT>(blockIdx.x, ret, pos, w, HV, k, out);
}

template <int VPT, bool FP8>
__global__ __launch_bounds__(1024) void combine_byte_kernel(const u32x4 *__restrict__ ret,
                                                            const float *__restrict__ scales,
                                                            const int32_t *__restrict__ pos,
                                                            const float *__restrict__ w, int G,
                                                            int k, u32x4 *__restrict__ out)
{
    combine_byte_row<VPT, FP8>(blockIdx.x, ret, scales, pos, w, G, k, out);
}

template <int VPT>
__global__ __launch_bounds__(1024) void combine_int4_kernel(const u32x2 *__restrict__ ret,
                                                            const float *__restrict__ scales,
                                                            const int32_t *__restrict__ pos,
                                                            const float *__restrict__ w, int G,
                                                            int k, u32x4 *__restrict__ out)
{
    combine_int4_row<VPT>(blockIdx.x, ret, scales, pos, w, G, k, out);
}

}  // namespace

hipError_t launch_combine(const void *recv, const float *scales, int quant, const int32_t *pos,
                          const float *w, int64_t T, int H, int k, void *out,
                          hipStream_t stream)
{
    const int HV = H / 8;
    const RowTiling rt = row_tiling(HV);
    const dim3 grid(static_cast<unsigned>(T));
    const dim3 block(rt.threads);
    u32x4 *ov = static_cast<u32x4 *>(out);
    if (quant == 0) {
        const u32x4 *rv = static_cast<const u32x4 *>(recv);
        switch (rt.vpt) {
        case 1: combine_bf16_kernel<1><<<grid, block, 0, stream>>>(rv, pos, w, HV, k, ov); break;
        case 2: combine_bf16_kernel<2><<<grid, block, 0, stream>>>(rv, pos, w, HV, k, ov); break;
        case 4: combine_bf16_kernel<4><<<grid, block, 0, stream>>>(rv, pos, w, HV, k, ov); break;
        default: combine_bf16_kernel<8><<<grid, block, 0, stream>>>(rv, pos, w, HV, k, ov); break;
        }
        return hipGetLastError();
    }
    const int G = H / 16;
    const RowTiling gt = row_tiling(G);
    const dim3 gblock(gt.threads);
    if (quant == 2) {
        const u32x2 *rv = static_cast<const u32x2 *>(recv);
#define MOE_COMB_INT4(V)                                                                       \
    combine_int4_kernel<V><<<grid, gblock, 0, stream>>>(rv, scales, pos, w, G, k, ov)
        switch (gt.vpt) {
        case 1: MOE_COMB_INT4(1); break;
        case 2: MOE_COMB_INT4(2); break;
        default: MOE_COMB_INT4(4); break;
        }
#undef MOE_COMB_INT4
    } else {
        const u32x4 *rv = static_cast<const u32x4 *>(recv);
#define MOE_COMB_BYTE(V, F)                                                                    \
    combine_byte_kernel<V, F><<<grid, gblock, 0, stream>>>(rv, scales, pos, w, G, k, ov)
        if (quant == 1) {
            switch (gt.vpt) {
            case 1: MOE_COMB_BYTE(1, false); break;
            case 2: MOE_COMB_BYTE(2, false); break;
            default: MOE_COMB_BYTE(4, false); break;
            }
        } else {
            switch (gt.vpt) {
            case 1: MOE_COMB_BYTE(1, true); break;
            case 2: MOE_COMB_BYTE(2, true); break;
            default: MOE_COMB_BYTE(4, true); break;
            }
        }
#undef MOE_COMB_BYTE
    }
    return hipGetLastError();
}

}  // namespace moe
