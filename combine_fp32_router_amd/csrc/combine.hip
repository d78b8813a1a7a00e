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
// group of row gathers (measured the same); the (int8 / int4) scales are
// block-uniform scalar loads.  Rows are fetched in groups
// of kLoadsPerLane/VPT slots whose loads are issued before the first FMA.
// Few loads per lane keep VGPRs low, so many waves (896-thread blocks at
// H=7168) stay resident and the CU as a whole keeps the read stream full;
// on MI355X two loads per lane measured faster than four or eight.  The read
// stream is what bounds the kernel (HBM).
#include "common.hpp"
#include "launch.hpp"

namespace moe {
namespace {

// row-vector loads each lane issues before accumulating (VPT * slots/group)
constexpr int kLoadsPerLane = 2;

template <int VPT>
__global__ __launch_bounds__(1024) void combine_bf16_kernel(const u32x4 *__restrict__ ret,
                                                            const int32_t *__restrict__ pos,
                                                            const float *__restrict__ w, int HV,
                                                            int k, u32x4 *__restrict__ out)
{
    const int64_t t = blockIdx.x;
    const int nthr = blockDim.x;
    float acc[VPT][8];
#pragma unroll
    for (int i = 0; i < VPT; ++i)
#pragma unroll
        for (int q = 0; q < 8; ++q)
            acc[i][q] = -0.0f;  // IEEE identity of +: one kept term passes unchanged

    constexpr int kGroup = kLoadsPerLane / VPT > 0 ? kLoadsPerLane / VPT : 1;
    const int32_t rows = load_per_lane(pos + t * k, k);  // lane j: row of slot j
    const float wts = load_per_lane(w + t * k, k);        // lane j: gate weight of slot j
    int kept = 0;
    for (int j0 = 0; j0 < k; j0 += kGroup) {
        u32x4 v[kGroup][VPT];
        float wj[kGroup];
#pragma unroll
        for (int g = 0; g < kGroup; ++g) {
            const int j = j0 + g;
            const int32_t p = (j < k) ? lane_value(rows, j) : -1;
            wj[g] = (p >= 0) ? lane_value(wts, j) : -0.0f;  // fma(-0, 0, acc) == acc
            kept += (p >= 0);
            const u32x4 *src = ret + static_cast<int64_t>(p < 0 ? 0 : p) * HV;
#pragma unroll
            for (int i = 0; i < VPT; ++i) {
                const int c = threadIdx.x + i * nthr;
                v[g][i] = (p >= 0 && c < HV) ? __builtin_nontemporal_load(src + c)
                                             : u32x4{0, 0, 0, 0};
            }
        }
#pragma unroll
        for (int g = 0; g < kGroup; ++g) {
#pragma unroll
            for (int i = 0; i < VPT; ++i) {
                float f[8];
                unpack8(v[g][i], f);
#pragma unroll
                for (int q = 0; q < 8; ++q)
                    acc[i][q] = fmaf(wj[g], f[q], acc[i][q]);
            }
        }
    }
    if (kept == 0)  // every slot dropped: +0
#pragma unroll
        for (int i = 0; i < VPT; ++i)
#pragma unroll
            for (int q = 0; q < 8; ++q)
                acc[i][q] = 0.0f;
    u32x4 *ot = out + t * HV;
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
        const int c = threadIdx.x + i * nthr;
        if (c < HV)
            __builtin_nontemporal_store(pack8(acc[i]), ot + c);
    }
}

// int8 / fp8 (FP8 = true): each thread owns VPT groups of 16 elements: one
// 16-byte load of 16 one-byte codes per row, 16 fp32 accumulators, two
// 16-byte bf16 stores.
template <int VPT, bool FP8>
__global__ __launch_bounds__(1024) void combine_byte_kernel(const uint8_t *__restrict__ ret,
                                                            int64_t stride,
                                                            const int32_t *__restrict__ pos,
                                                            const float *__restrict__ w, int G,
                                                            int k, u32x4 *__restrict__ out)
{
    const int64_t t = blockIdx.x;
    const int nthr = blockDim.x;
    const int H = G * 16;
    float acc[VPT][16];
#pragma unroll
    for (int i = 0; i < VPT; ++i)
#pragma unroll
        for (int q = 0; q < 16; ++q)
            acc[i][q] = -0.0f;  // IEEE identity of +: one kept term passes unchanged

    constexpr int kGroup = kLoadsPerLane / VPT > 0 ? kLoadsPerLane / VPT : 1;
    int kept = 0;
    const int32_t rows = load_per_lane(pos + t * k, k);  // lane j: row of slot j
    const float wts = load_per_lane(w + t * k, k);        // lane j: gate weight of slot j
    for (int j0 = 0; j0 < k; j0 += kGroup) {
        u32x4 v[kGroup][VPT];
        float wj[kGroup], sj[kGroup];
#pragma unroll
        for (int gg = 0; gg < kGroup; ++gg) {
            const int j = j0 + gg;
            const int32_t p = (j < k) ? lane_value(rows, j) : -1;
            const uint8_t *rec = ret + static_cast<int64_t>(p < 0 ? 0 : p) * stride;
            wj[gg] = (p >= 0) ? lane_value(wts, j) : -0.0f;  // fma(-0, 0, acc) == acc
            kept += (p >= 0);
            sj[gg] = (p >= 0) ? *reinterpret_cast<const float *>(rec + H) : 0.0f;
            const u32x4 *src = reinterpret_cast<const u32x4 *>(rec);
#pragma unroll
            for (int i = 0; i < VPT; ++i) {
                const int g = threadIdx.x + i * nthr;
                v[gg][i] = (p >= 0 && g < G) ? __builtin_nontemporal_load(src + g)
                                             : u32x4{0, 0, 0, 0};
            }
        }
#pragma unroll
        for (int gg = 0; gg < kGroup; ++gg) {
#pragma unroll
            for (int i = 0; i < VPT; ++i) {
                float f[16];
                if (FP8) {
                    dequant_fp8x8(u32x2{v[gg][i].x, v[gg][i].y}, sj[gg], f);
                    dequant_fp8x8(u32x2{v[gg][i].z, v[gg][i].w}, sj[gg], f + 8);
                } else {
                    dequant8(u32x2{v[gg][i].x, v[gg][i].y}, sj[gg], f);
                    dequant8(u32x2{v[gg][i].z, v[gg][i].w}, sj[gg], f + 8);
                }
#pragma unroll
                for (int q = 0; q < 16; ++q)
                    acc[i][q] = fmaf(wj[gg], f[q], acc[i][q]);
            }
        }
    }
    if (kept == 0)  // every slot dropped: +0
#pragma unroll
        for (int i = 0; i < VPT; ++i)
#pragma unroll
            for (int q = 0; q < 16; ++q)
                acc[i][q] = 0.0f;
    u32x4 *ot = out + t * 2 * G;
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
        const int g = threadIdx.x + i * nthr;
        if (g < G) {
            __builtin_nontemporal_store(pack8(acc[i]), ot + 2 * g);
            __builtin_nontemporal_store(pack8(acc[i] + 8), ot + 2 * g + 1);
        }
    }
}

// int4: each thread owns VPT groups of 16 elements: one 8-byte load of 16
// codes per row, 16 fp32 accumulators, two 16-byte bf16 stores.  The
// record's scale follows its H/2 code bytes.  The weight and the scale of a
// row are folded once, so each element costs a bit-field extract, a convert
// and one FMA: acc += code * (w * scale).  (The exact product w * (code *
// scale) differs by fp32 rounding only, ~1e-7 relative, far below the
// tolerance the output is held to; for int8 the same fold measured slower.)
// Sixteen elements per thread keep the VGPR count near the int8 kernel's
// (39 against 101 with 32), so enough waves stay resident.
template <int VPT>
__global__ __launch_bounds__(1024) void combine_int4_kernel(const uint8_t *__restrict__ ret,
                                                            int64_t stride,
                                                            const int32_t *__restrict__ pos,
                                                            const float *__restrict__ w, int G,
                                                            int k, u32x4 *__restrict__ out)
{
    const int64_t t = blockIdx.x;
    const int nthr = blockDim.x;
    const int H = G * 16;
    float acc[VPT][16];
#pragma unroll
    for (int i = 0; i < VPT; ++i)
#pragma unroll
        for (int q = 0; q < 16; ++q)
            acc[i][q] = -0.0f;  // IEEE identity of +: one kept term passes unchanged

    // 8-byte code loads: twice the rows per group keeps the same bytes in
    // flight per lane as the 16-byte kernels (measured ~4% faster than 2)
    constexpr int kGroup = 2 * kLoadsPerLane / VPT > 0 ? 2 * kLoadsPerLane / VPT : 1;
    int kept = 0;
    const int32_t rows = load_per_lane(pos + t * k, k);  // lane j: row of slot j
    const float wts = load_per_lane(w + t * k, k);        // lane j: gate weight of slot j
    for (int j0 = 0; j0 < k; j0 += kGroup) {
        u32x2 v[kGroup][VPT];
        float ws[kGroup];
#pragma unroll
        for (int gg = 0; gg < kGroup; ++gg) {
            const int j = j0 + gg;
            const int32_t p = (j < k) ? lane_value(rows, j) : -1;
            const uint8_t *rec = ret + static_cast<int64_t>(p < 0 ? 0 : p) * stride;
            kept += (p >= 0);
            // dropped: codes load as +0 and fma(+0, -0, acc) == acc
            ws[gg] = (p >= 0) ? lane_value(wts, j) * *reinterpret_cast<const float *>(rec + H / 2) : -0.0f;
            const u32x2 *src = reinterpret_cast<const u32x2 *>(rec);
#pragma unroll
            for (int i = 0; i < VPT; ++i) {
                const int g = threadIdx.x + i * nthr;
                v[gg][i] = (p >= 0 && g < G) ? __builtin_nontemporal_load(src + g)
                                             : u32x2{0, 0};
            }
        }
#pragma unroll
        for (int gg = 0; gg < kGroup; ++gg) {
#pragma unroll
            for (int i = 0; i < VPT; ++i) {
                float f[16];
                codes4x8(v[gg][i].x, f);
                codes4x8(v[gg][i].y, f + 8);
#pragma unroll
                for (int q = 0; q < 16; ++q)
                    acc[i][q] = fmaf(f[q], ws[gg], acc[i][q]);
            }
        }
    }
    if (kept == 0)  // every slot dropped: +0
#pragma unroll
        for (int i = 0; i < VPT; ++i)
#pragma unroll
            for (int q = 0; q < 16; ++q)
                acc[i][q] = 0.0f;
    u32x4 *ot = out + t * 2 * G;
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
        const int g = threadIdx.x + i * nthr;
        if (g < G) {
            __builtin_nontemporal_store(pack8(acc[i]), ot + 2 * g);
            __builtin_nontemporal_store(pack8(acc[i] + 8), ot + 2 * g + 1);
        }
    }
}

}  // namespace

hipError_t launch_combine(const void *recv, int quant, const int32_t *pos, const float *w,
                          int64_t T, int H, int k, void *out, hipStream_t stream)
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
    } else if (quant == 2) {
        const uint8_t *rb = static_cast<const uint8_t *>(recv);
        const int64_t stride = record_bytes(H, 2);
        const int G = H / 16;
        const RowTiling gt = row_tiling(G);
        const dim3 gblock(gt.threads);
        switch (gt.vpt) {
        case 1: combine_int4_kernel<1><<<grid, gblock, 0, stream>>>(rb, stride, pos, w, G, k, ov); break;
        case 2: combine_int4_kernel<2><<<grid, gblock, 0, stream>>>(rb, stride, pos, w, G, k, ov); break;
        case 4: combine_int4_kernel<4><<<grid, gblock, 0, stream>>>(rb, stride, pos, w, G, k, ov); break;
        default: combine_int4_kernel<8><<<grid, gblock, 0, stream>>>(rb, stride, pos, w, G, k, ov); break;
        }
    } else {
        const uint8_t *rb = static_cast<const uint8_t *>(recv);
        const int64_t stride = record_bytes(H, quant);
        const int G = H / 16;
        const RowTiling gt = row_tiling(G);
        const dim3 gblock(gt.threads);
        if (quant == 1) {
            switch (gt.vpt) {
            case 1: combine_byte_kernel<1, false><<<grid, gblock, 0, stream>>>(rb, stride, pos, w, G, k, ov); break;
            case 2: combine_byte_kernel<2, false><<<grid, gblock, 0, stream>>>(rb, stride, pos, w, G, k, ov); break;
            case 4: combine_byte_kernel<4, false><<<grid, gblock, 0, stream>>>(rb, stride, pos, w, G, k, ov); break;
            default: combine_byte_kernel<8, false><<<grid, gblock, 0, stream>>>(rb, stride, pos, w, G, k, ov); break;
            }
        } else {
            switch (gt.vpt) {
            case 1: combine_byte_kernel<1, true><<<grid, gblock, 0, stream>>>(rb, stride, pos, w, G, k, ov); break;
            case 2: combine_byte_kernel<2, true><<<grid, gblock, 0, stream>>>(rb, stride, pos, w, G, k, ov); break;
            case 4: combine_byte_kernel<4, true><<<grid, gblock, 0, stream>>>(rb, stride, pos, w, G, k, ov); break;
            default: combine_byte_kernel<8, true><<<grid, gblock, 0, stream>>>(rb, stride, pos, w, G, k, ov); break;
            }
        }
    }
    return hipGetLastError();
}

}  // namespace moe
