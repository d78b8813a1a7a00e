// Dispatch pack: stable scatter of hidden rows into the send buffer, plain
// bf16 or per-token dynamic int8 / int4.
//
// What it computes (aggregation by destination into one contiguous buffer,
// ThunderEP write-up s2.1; per-token dynamic int8 with one run-time scale per
// token, s2.3): for each slot s with pos[s] >= 0, row pos[s] = token s/k's
// row, copied bit for bit (bf16) or as H int8 codes (scale = max|x|/127,
// code = rne(x/scale) clamped to +-127; fp8 the same with scale =
// max|x|/448 and an OCP E4M3 code, the NCCL EP article's FP8 communication,
// s6.3), or as H/2 bytes of 4-bit codes (int4, the write-up's 4-bit
// follow-up, s5.2; scale = max|x|/7, codes clamped to +-7, element 2i in the
// low nibble of byte i); a quantised row's fp32 scale goes to entry pos[s]
// of the scale array.
//
// gfx950 design.  One block per token; the row is read from HBM once, kept in
// VGPRs (each thread owns `VPT` 16-byte vectors, strided by the block size so
// every wave instruction moves 1 KiB of contiguous memory) and written to
// the token's k rows.  The k row numbers arrive with one vector load (lane j
// holds slot j's row) issued beside the row load and are read back with
// v_readlane, instead of k dependent scalar loads in the store loop (which
// the resident waves already hid: the two forms measured the same).
// Stores are not nontemporal: when one chunk's send buffer fits the 256 MB
// Infinity Cache, its consumer (the exchange, or combine on one device)
// reads it from there; measured neutral when it does not fit, and 11%
// faster for pack + combine at 8 chunks of the T=16384, H=7168, k=8 batch.
// They are device-scope buffer stores (store_row<false>): written through the
// XCD's L2 rather than left dirty in it, which took the bf16 step of that
// batch from 0.620 to 0.614 ms and the int4 step from 0.258 to 0.252 (int8
// and fp8 within 0.3%).  When nothing reads the send rows back from this
// GPU's cache soon (their consumer is another GPU, or runs after other
// traffic), the caller asks for streaming stores (store_row<true>,
// MOE_PACK_STREAM): kept dirty in the last-level cache, the rows would have
// to be evicted and written back in the middle of later kernels.  With
// combine reading rows written a step earlier and new inputs every step,
// the two policies time alike for the T=16384, H=7168 bf16 step (0.778
// against 0.787 ms), and only with streaming stores does the merged launch
// prefetch its pack rows (combine_pack.hip: 0.757 ms); where the rows are
// re-read from the cache, streaming stores cost 17% (0.617 against 0.72
// ms).  The same policy on combine's output was much worse (int8 step
// 0.378 -> 0.496 ms), so combine keeps nontemporal stores.
// The int8 variant gives each thread 16 elements, reduces max|x| over the
// block (wave shuffles + LDS), quantises in registers and stores 16 codes
// per lane (one 16-byte store per row); thread 0 writes the scale.  Keeping
// the scale out of the row keeps every row a whole number of 128-byte lines
// (H = 7168: 56), so no line is shared by two rows written from different
// blocks and every wave's 1 KiB access covers 8 lines, not 9; with the scale
// in a 16-byte slot after the codes (7184-byte rows) the T=16384, H=7168
// int8 step took 0.420 ms against 0.383 ms (int4 0.326 against 0.301).
// Nothing here is a contraction: the kernel is bound by HBM write bandwidth
// (k row writes per row read).
#include "pack_rows.hpp"
#include "launch.hpp"

namespace moe {
namespace {

template <int VPT, bool ST>
__global__ __launch_bounds__(1024) void pack_bf16_kernel(const u32x4 *__restrict__ x, int HV,
                                                         int k, const int32_t *__restrict__ pos,
                                                         u32x4 *__restrict__ send)
{
    pack_bf16_row<VPT, ST>(blockIdx.x, x, HV, k, pos, send);
}

template <int VPT, bool FP8, bool ST>
__global__ __launch_bounds__(1024) void pack_byte_kernel(const u32x4 *__restrict__ x, int G,
                                                         int k, const int32_t *__restrict__ pos,
                                                         u32x4 *__restrict__ send,
                                                         float *__restrict__ scales)
{
    pack_byte_row<VPT, FP8, ST>(blockIdx.x, x, G, k, pos, send, scales);
}

template <int VPT, bool ST>
__global__ __launch_bounds__(1024) void pack_int4_kernel(const u32x4 *__restrict__ x, int G,
                                                         int k, const int32_t *__restrict__ pos,
                                                         u32x2 *__restrict__ send,
                                                         float *__restrict__ scales)
{
    pack_int4_row<VPT, ST>(blockIdx.x, x, G, k, pos, send, scales);
}

template <bool ST>
hipError_t pack_launch(const void *x, int64_t T, int H, int k, const int32_t *pos, int quant,
                       void *send, float *scales, hipStream_t stream)
{
    const int HV = H / 8;
    const RowTiling rt = row_tiling(HV);
    const dim3 grid(static_cast<unsigned>(T));
    const dim3 block(rt.threads);
    const u32x4 *xv = static_cast<const u32x4 *>(x);
    u32x4 *sv = static_cast<u32x4 *>(send);
    if (quant == 0) {
        switch (rt.vpt) {
        case 1: pack_bf16_kernel<1, ST><<<grid, block, 0, stream>>>(xv, HV, k, pos, sv); break;
        case 2: pack_bf16_kernel<2, ST><<<grid, block, 0, stream>>>(xv, HV, k, pos, sv); break;
        case 4: pack_bf16_kernel<4, ST><<<grid, block, 0, stream>>>(xv, HV, k, pos, sv); break;
        default: pack_bf16_kernel<8, ST><<<grid, block, 0, stream>>>(xv, HV, k, pos, sv); break;
        }
    } else if (quant == 1 || quant == 3) {
        const int G = H / 16;
        const RowTiling gt = row_tiling(G);
        const dim3 gblock(gt.threads);
#define MOE_PACK_BYTE(V, F)                                                                    \
    pack_byte_kernel<V, F, ST><<<grid, gblock, 0, stream>>>(xv, G, k, pos, sv, scales)
        if (quant == 1) {
            switch (gt.vpt) {
            case 1: MOE_PACK_BYTE(1, false); break;
            case 2: MOE_PACK_BYTE(2, false); break;
            default: MOE_PACK_BYTE(4, false); break;
            }
        } else {
            switch (gt.vpt) {
            case 1: MOE_PACK_BYTE(1, true); break;
            case 2: MOE_PACK_BYTE(2, true); break;
            default: MOE_PACK_BYTE(4, true); break;
            }
        }
#undef MOE_PACK_BYTE
    } else {
        const int G = H / 16;
        const RowTiling gt = row_tiling(G);
        const dim3 gblock(gt.threads);
        u32x2 *s2 = static_cast<u32x2 *>(send);
#define MOE_PACK_INT4(V)                                                                       \
    pack_int4_kernel<V, ST><<<grid, gblock, 0, stream>>>(xv, G, k, pos, s2, scales)
        switch (gt.vpt) {
        case 1: MOE_PACK_INT4(1); break;
        case 2: MOE_PACK_INT4(2); break;
        default: MOE_PACK_INT4(4); break;
        }
#undef MOE_PACK_INT4
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_dispatch_pack(const void *x, int64_t T, int H, int k, const int32_t *pos,
                                int quant, bool stream_stores, void *send, float *scales,
                                hipStream_t stream)
{
    return stream_stores ? pack_launch<true>(x, T, H, k, pos, quant, send, scales, stream)
                         : pack_launch<false>(x, T, H, k, pos, quant, send, scales, stream);
}

}  // namespace moe
