// Router top-k with renormalised gate weights, one wavefront per token.
//
// What it computes (sparse-communication article, intelliparadigm.com,
// s2.1: softmax over the router logits, keep the top-k; weights are the
// selected probabilities renormalised to sum to one):
//   idx[t, 0..k-1]  the k largest logits of row t, descending, equal values
//                   to the lower expert id;
//   w[t, j]         exp(l_j - l_max) / sum_i exp(l_i - l_max) over the k.
//
// gfx950 mapping.  A 64-lane wave owns one token; lane l holds experts
// l, l+64, l+128, ... as 64-bit keys (order-preserving image of the fp32
// value << 32 | ~expert id), so "larger value, then lower id" is a single
// unsigned max.  k rounds of a wave max pick the experts in output order;
// the winner's lane retires that key.  The wave max runs in the VALU: DPP
// row reductions (quad_perm / row_half_mirror / row_mirror) and four
// v_readlane of the row results, so the round's winner is a scalar and no
// LDS round trip sits on the dependency chain.  The k-way softmax is
// evaluated in double by lanes 0..k-1 (k <= 16: one DPP row sum); it is ~0.4%
// of the path's bytes and makes the fp32 weights correctly rounded up to one
// double rounding.
#include "common.hpp"
#include "launch.hpp"

namespace moe {
namespace {

__device__ __forceinline__ uint64_t make_key(float v, int e)
{
    uint32_t u = __float_as_uint(v);
    if (u == 0x80000000u)  // -0 ties with +0
        u = 0;
    const uint32_t ord = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
    return (static_cast<uint64_t>(ord) << 32) | static_cast<uint32_t>(~static_cast<uint32_t>(e));
}

__device__ __forceinline__ float key_value(uint64_t key)
{
    const uint32_t ord = static_cast<uint32_t>(key >> 32);
    const uint32_t u = (ord & 0x80000000u) ? (ord & 0x7fffffffu) : ~ord;
    return __uint_as_float(u);
}

__device__ __forceinline__ int key_expert(uint64_t key)
{
    return static_cast<int>(~static_cast<uint32_t>(key));
}

// NE = keys per lane = ceil(E / 64).  Absent experts hold key 0, below every
// finite logit (the smallest finite key is 0x00800000 << 32).
template <int NE>
__global__ __launch_bounds__(256) void route_topk_kernel(const float *__restrict__ logits,
                                                         int64_t T, int E, int k,
                                                         int32_t *__restrict__ idx,
                                                         float *__restrict__ w)
{
    const int lane = lane_id();
    const int64_t t = static_cast<int64_t>(blockIdx.x) * 4 + uniform(threadIdx.x / kWave);
    if (t >= T)
        return;
    const float *row = logits + t * E;

    uint64_t key[NE];
#pragma unroll
    for (int i = 0; i < NE; ++i) {
        const int e = i * kWave + lane;
        key[i] = (e < E) ? make_key(__builtin_nontemporal_load(row + e), e) : 0ull;
    }

    uint64_t mine = 0;   // lane j keeps the j-th selected key
    uint64_t first = 0;  // the largest key (wave-uniform)
    for (int r = 0; r < k; ++r) {
        uint64_t best = key[0];
#pragma unroll
        for (int i = 1; i < NE; ++i)
            best = umax64(key[i], best);
        const uint64_t top = wave_max_u64_dpp(best);  // scalar
        if (r == 0)
            first = top;
#pragma unroll
        for (int i = 0; i < NE; ++i)
            key[i] = (key[i] == top) ? 0ull : key[i];  // ids are distinct: one match
        if (lane == r)
            mine = top;
    }

    // k <= 16: the selected keys live in lanes 0..k-1 of the first row
    const double lmax = static_cast<double>(key_value(first));
    const double a = (lane < k) ? exp(static_cast<double>(key_value(mine)) - lmax) : 0.0;
    const double s = row_sum_f64(a);
    if (lane < k) {
        idx[t * k + lane] = key_expert(mine);
        w[t * k + lane] = static_cast<float>(a / s);
    }
}

}  // namespace

hipError_t launch_route_topk(const float *logits, int64_t T, int E, int k,
                             int32_t *idx, float *w, hipStream_t stream)
{
    const dim3 block(256);
    const dim3 grid(static_cast<unsigned>((T + 3) / 4));
    if (E <= 64)
        route_topk_kernel<1><<<grid, block, 0, stream>>>(logits, T, E, k, idx, w);
    else if (E <= 128)
        route_topk_kernel<2><<<grid, block, 0, stream>>>(logits, T, E, k, idx, w);
    else if (E <= 256)
        route_topk_kernel<4><<<grid, block, 0, stream>>>(logits, T, E, k, idx, w);
    else if (E <= 512)
        route_topk_kernel<8><<<grid, block, 0, stream>>>(logits, T, E, k, idx, w);
    else
        route_topk_kernel<16><<<grid, block, 0, stream>>>(logits, T, E, k, idx, w);
    return hipGetLastError();
}

}  // namespace moe
