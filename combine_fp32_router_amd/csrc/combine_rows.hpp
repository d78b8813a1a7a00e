// Per-token bodies of the combine kernels (one block per token), shared by
// the standalone combine launch and the combine+pack launch.  The operation
// and the gfx950 design are described in combine.hip.
#pragma once

#include "common.hpp"

namespace moe {
namespace {

// row-vector loads each lane issues before accumulating (VPT * slots/group):
// two for the bf16 rows; eight for the int8 / fp8 rows, whose loads carry
// half the bytes (at k = 8 every row of the token is in flight at once:
// the T=16384, H=7168 int8 step 0.388 -> 0.379 ms and fp8 0.385 -> 0.377;
// with rows read a step after they were written, 0-2% faster; bf16 lost 1%
// that way)
constexpr int kLoadsPerLane = 2;
constexpr int kByteLoadsPerLane = 8;

// Prefetch for a merged launch with streaming send stores (combine_pack.hip):
// the combine body for token t first loads, with the default cache policy,
// the hidden row that the pack half will read for its token t, so that the
// pack finds it in the last-level cache instead of waiting on HBM before its
// k stores.  The loads are issued after the slot tables' and before the
// rows', so the only wait they add is folded into the first row wait; the
// values are only kept live (an empty asm that uses them, placed after the
// combine's stores), never used.  PF = false compiles none of it.
template <bool PF, int N>
__device__ __forceinline__ void prefetch_row(const u32x4 *row, int bytes, u32x4 (&pf)[N])
{
    if constexpr (PF) {
        const __amdgpu_buffer_rsrc_t r = row_rsrc(const_cast<u32x4 *>(row), bytes);
#pragma unroll
        for (int i = 0; i < N; ++i)
            pf[i] = load_cached(r, (threadIdx.x + i * blockDim.x) * 16);  // zeros past the row
    }
}
template <bool PF, int N>
__device__ __forceinline__ void keep_prefetch(const u32x4 (&pf)[N])
{
    if constexpr (PF) {
#pragma unroll
        for (int i = 0; i < N; ++i)
            asm volatile("" ::"v"(pf[i].x), "v"(pf[i].y), "v"(pf[i].z), "v"(pf[i].w) : "memory");
    }
}

template <int VPT, bool PF = false>
__device__ __forceinline__ void combine_bf16_row(int64_t t, const u32x4 *__restrict__ ret,
                                                 const int32_t *__restrict__ pos,
                                                 const float *__restrict__ w, int HV,
                                                 int k, u32x4 *__restrict__ out,
                                                 const u32x4 *pf_row = nullptr, int pf_bytes = 0)
{
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
    u32x4 pf[VPT];  // PF: the pack partner's hidden row (VPT vectors per thread)
    prefetch_row<PF>(pf_row, pf_bytes, pf);
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
    keep_prefetch<PF>(pf);
}

// int8 / fp8 (FP8 = true): each thread owns VPT groups of 16 elements: one
// 16-byte load of 16 one-byte codes per row, 16 fp32 accumulators, two
// 16-byte bf16 stores.  The row's scale is a block-uniform load from the
// scale array.  As in the int4 kernel below, the row's weight and scale are
// folded once: acc += code * (w * scale), a convert and one FMA per element.
template <int VPT, bool FP8, bool PF = false>
__device__ __forceinline__ void combine_byte_row(int64_t t, const u32x4 *__restrict__ ret,
                                                 const float *__restrict__ scales,
                                                 const int32_t *__restrict__ pos,
                                                 const float *__restrict__ w, int G,
                                                 int k, u32x4 *__restrict__ out,
                                                 const u32x4 *pf_row = nullptr, int pf_bytes = 0)
{
    const int nthr = blockDim.x;
    float acc[VPT][16];
#pragma unroll
    for (int i = 0; i < VPT; ++i)
#pragma unroll
        for (int q = 0; q < 16; ++q)
            acc[i][q] = -0.0f;  // IEEE identity of +: one kept term passes unchanged

    constexpr int kGroup = kByteLoadsPerLane / VPT > 0 ? kByteLoadsPerLane / VPT : 1;
    int kept = 0;
    const int32_t rows = load_per_lane(pos + t * k, k);  // lane j: row of slot j
    const float wts = load_per_lane(w + t * k, k);        // lane j: gate weight of slot j
    u32x4 pf[2 * VPT];  // PF: the pack partner's hidden row (2 VPT vectors per thread)
    prefetch_row<PF>(pf_row, pf_bytes, pf);
    for (int j0 = 0; j0 < k; j0 += kGroup) {
        u32x4 v[kGroup][VPT];
        float wj[kGroup], sj[kGroup];
#pragma unroll
        for (int gg = 0; gg < kGroup; ++gg) {
            const int j = j0 + gg;
            const int32_t p = (j < k) ? lane_value(rows, j) : -1;
            const int64_t pr = p < 0 ? 0 : p;
            wj[gg] = (p >= 0) ? lane_value(wts, j) : -0.0f;  // fma(-0, 0, acc) == acc
            kept += (p >= 0);
            sj[gg] = (p >= 0) ? scales[pr] : 0.0f;
            const u32x4 *src = ret + pr * G;
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
                const float ws = wj[gg] * sj[gg];
                if (FP8) {
                    dequant_fp8x8(u32x2{v[gg][i].x, v[gg][i].y}, 1.0f, f);
                    dequant_fp8x8(u32x2{v[gg][i].z, v[gg][i].w}, 1.0f, f + 8);
                } else {
                    dequant8(u32x2{v[gg][i].x, v[gg][i].y}, 1.0f, f);
                    dequant8(u32x2{v[gg][i].z, v[gg][i].w}, 1.0f, f + 8);
                }
#pragma unroll
                for (int q = 0; q < 16; ++q)
                    acc[i][q] = fmaf(f[q], ws, acc[i][q]);
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
    keep_prefetch<PF>(pf);
}

// int4: each thread owns VPT groups of 16 elements: one 8-byte load of 16
// codes per row, 16 fp32 accumulators, two 16-byte bf16 stores.  The row's
// scale is a block-uniform load from the scale array.  The weight and the
// scale of a row are folded once, so each element costs a sign-extending byte convert
// (codes4x8_x16, 16 * code) and one FMA: acc += (16 * code) * (w * scale /
// 16), the same product as code * (w * scale).  (The exact product
// w * (code * scale) differs by fp32 rounding only, ~1e-7 relative, far
// below the tolerance the output is held to.)
// Sixteen elements per thread keep the VGPR count near the int8 kernel's
// (39 against 101 with 32), so enough waves stay resident.
template <int VPT, bool PF = false>
__device__ __forceinline__ void combine_int4_row(int64_t t, const u32x2 *__restrict__ ret,
                                                 const float *__restrict__ scales,
                                                 const int32_t *__restrict__ pos,
                                                 const float *__restrict__ w, int G,
                                                 int k, u32x4 *__restrict__ out,
                                                 const u32x4 *pf_row = nullptr, int pf_bytes = 0)
{
    const int nthr = blockDim.x;
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
    u32x4 pf[2 * VPT];  // PF: the pack partner's hidden row (2 VPT vectors per thread)
    prefetch_row<PF>(pf_row, pf_bytes, pf);
    for (int j0 = 0; j0 < k; j0 += kGroup) {
        u32x2 v[kGroup][VPT];
        float ws[kGroup];
#pragma unroll
        for (int gg = 0; gg < kGroup; ++gg) {
            const int j = j0 + gg;
            const int32_t p = (j < k) ? lane_value(rows, j) : -1;
            const int64_t pr = p < 0 ? 0 : p;
            kept += (p >= 0);
            // dropped: codes load as +0 and fma(+0, -0, acc) == acc
            // w * scale / 16: the codes arrive as 16 * code (codes4x8_x16);
            // the power-of-two factor is exact
            ws[gg] = (p >= 0) ? lane_value(wts, j) * scales[pr] * 0.0625f : -0.0f;
            // G 8-byte groups of 16 codes; a buffer descriptor per row keeps
            // the address arithmetic scalar (one byte offset per thread for
            // all rows), which this ALU-bound kernel feels: 0.257 -> 0.253 ms
            // for the T=16384, H=7168 int4 step (the int8 / fp8 combines,
            // less ALU-bound, lost 0.7% the same way and keep global loads)
            const __amdgpu_buffer_rsrc_t src =
                row_rsrc(const_cast<u32x2 *>(ret) + pr * G, p < 0 ? 0 : G * 8);
#pragma unroll
            for (int i = 0; i < VPT; ++i)
                v[gg][i] = load_stream8(src, (threadIdx.x + i * nthr) * 8);
        }
#pragma unroll
        for (int gg = 0; gg < kGroup; ++gg) {
#pragma unroll
            for (int i = 0; i < VPT; ++i) {
                float f[16];
                codes4x8_x16(v[gg][i].x, f);
                codes4x8_x16(v[gg][i].y, f + 8);
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
    keep_prefetch<PF>(pf);
}

}  // namespace
}  // namespace moe
