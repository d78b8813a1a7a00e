// Per-token bodies of the dispatch pack kernels (one block per token), shared
// by the standalone pack launch and the combine+pack launch.  The operation
// and the gfx950 design are described in dispatch_pack.hip.  STREAM selects
// the send rows' store policy (store_row in common.hpp).
#pragma once

#include "common.hpp"

namespace moe {
namespace {

template <int VPT, bool STREAM>
__device__ __forceinline__ void pack_bf16_row(int64_t t, const u32x4 *__restrict__ x, int HV,
                                              int k, const int32_t *__restrict__ pos,
                                              u32x4 *__restrict__ send)
{
    const int nthr = blockDim.x;
    const __amdgpu_buffer_rsrc_t xr = row_rsrc(const_cast<u32x4 *>(x) + t * HV, HV * 16);
    const int32_t rows = load_per_lane(pos + t * k, k);  // lane j: row of slot j
    u32x4 v[VPT];
#pragma unroll
    for (int i = 0; i < VPT; ++i)
        v[i] = load_cached(xr, (threadIdx.x + i * nthr) * 16);  // zeros past the row
    for (int j = 0; j < k; ++j) {
        const int32_t p = lane_value(rows, j);
        if (p < 0)
            continue;
        const __amdgpu_buffer_rsrc_t dst = row_rsrc(send + static_cast<int64_t>(p) * HV, HV * 16);
#pragma unroll
        for (int i = 0; i < VPT; ++i) {
            const int c = threadIdx.x + i * nthr;
            if (c < HV)
                store_row<STREAM>(dst, c * 16, v[i]);
        }
    }
}

// int8 / fp8 (FP8 = true): each thread owns VPT groups of 16 elements (two
// 16-byte bf16 loads, one 16-byte store of 16 one-byte codes per row),
// strided by the block size.  Thread 0 writes the row's scale to
// scales[p].
template <int VPT, bool FP8, bool STREAM>
__device__ __forceinline__ void pack_byte_row(int64_t t, const u32x4 *__restrict__ x, int G,
                                              int k, const int32_t *__restrict__ pos,
                                              u32x4 *__restrict__ send,
                                              float *__restrict__ scales)
{
    __shared__ float red[16];
    const int nthr = blockDim.x;
    const __amdgpu_buffer_rsrc_t xr = row_rsrc(const_cast<u32x4 *>(x) + t * 2 * G, G * 32);
    const int32_t rows = load_per_lane(pos + t * k, k);  // lane j: row of slot j
    float f[VPT][16];
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
        const int g = threadIdx.x + i * nthr;
        const u32x4 a = load_cached(xr, g * 32);  // zeros past the row
        const u32x4 b = load_cached(xr, g * 32 + 16);
        unpack8(a, f[i]);
        unpack8(b, f[i] + 8);
#pragma unroll
        for (int q = 0; q < 16; ++q)
            amax = fmaxf(amax, fabsf(f[i][q]));
    }
    amax = block_max_nonneg(amax, red);
    const bool zero = (amax == 0.0f);
    const float scale = zero ? 0.0f : amax / (FP8 ? 448.0f : 127.0f);
    u32x4 codes[VPT];
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
        if (FP8) {
            codes[i] = u32x4{fp8x4(f[i], scale, zero), fp8x4(f[i] + 4, scale, zero),
                             fp8x4(f[i] + 8, scale, zero), fp8x4(f[i] + 12, scale, zero)};
        } else {
            const u32x2 lo = quant8(f[i], scale, zero);
            const u32x2 hi = quant8(f[i] + 8, scale, zero);
            codes[i] = u32x4{lo.x, lo.y, hi.x, hi.y};
        }
    }

    for (int j = 0; j < k; ++j) {
        const int32_t p = lane_value(rows, j);
        if (p < 0)
            continue;
        const __amdgpu_buffer_rsrc_t dst = row_rsrc(send + static_cast<int64_t>(p) * G, G * 16);
#pragma unroll
        for (int i = 0; i < VPT; ++i) {
            const int g = threadIdx.x + i * nthr;
            if (g < G)
                store_row<STREAM>(dst, g * 16, codes[i]);
        }
        if (threadIdx.x == 0)
            scales[p] = scale;
    }
}

// int4: each thread owns VPT groups of 16 elements (two 16-byte bf16 loads,
// one 8-byte store of 16 codes per row), strided by the block size, the
// same split of the row as the int8 pack.  Thread 0 writes the row's scale
// to scales[p].  With 32 elements per thread and 16-byte stores the pack
// issued half the store instructions but each thread ran 32 IEEE
// divisions, and in the merged launch (the combine's block size) half of
// the pack block's threads idled: the T=16384, H=7168 int4 step took 0.294
// ms against 0.270 with 16 (a one-chunk T=4096 step, standalone launches
// only, 2.9% less).
template <int VPT, bool STREAM>
__device__ __forceinline__ void pack_int4_row(int64_t t, const u32x4 *__restrict__ x, int G,
                                              int k, const int32_t *__restrict__ pos,
                                              u32x2 *__restrict__ send,
                                              float *__restrict__ scales)
{
    __shared__ float red[16];
    const int nthr = blockDim.x;
    const __amdgpu_buffer_rsrc_t xr = row_rsrc(const_cast<u32x4 *>(x) + t * 2 * G, G * 32);
    const int32_t rows = load_per_lane(pos + t * k, k);  // lane j: row of slot j
    float f[VPT][16];
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
        const int g = threadIdx.x + i * nthr;
        const u32x4 a = load_cached(xr, g * 32);  // zeros past the row
        const u32x4 b = load_cached(xr, g * 32 + 16);
        unpack8(a, f[i]);
        unpack8(b, f[i] + 8);
#pragma unroll
        for (int q = 0; q < 16; ++q)
            amax = fmaxf(amax, fabsf(f[i][q]));
    }
    amax = block_max_nonneg(amax, red);
    const bool zero = (amax == 0.0f);
    const float scale = zero ? 0.0f : amax / 7.0f;
    u32x2 codes[VPT];
#pragma unroll
    for (int i = 0; i < VPT; ++i)
        codes[i] = u32x2{quant4x8(f[i], scale, zero), quant4x8(f[i] + 8, scale, zero)};

    for (int j = 0; j < k; ++j) {
        const int32_t p = lane_value(rows, j);
        if (p < 0)
            continue;
        const __amdgpu_buffer_rsrc_t dst = row_rsrc(send + static_cast<int64_t>(p) * G, G * 8);
#pragma unroll
        for (int i = 0; i < VPT; ++i) {
            const int g = threadIdx.x + i * nthr;
            if (g < G)
                store_row<STREAM>(dst, g * 8, codes[i]);
        }
        if (threadIdx.x == 0)
            scales[p] = scale;
    }
}

}  // namespace
}  // namespace moe
