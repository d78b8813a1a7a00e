// Router top-k with renormalised gate weights.
//
// What it computes (sparse-communication article, intelliparadigm.com,
// s2.1: softmax over the router logits, keep the top-k; weights are the
// selected probabilities renormalised to sum to one):
//   idx[t, 0..k-1]  the k largest logits of row t, descending, equal values
//                   to the lower expert id;
//   w[t, j]         exp(l_j - l_max) / sum_i exp(l_i - l_max) over the k.
//
// gfx950 mapping.  A group of L lanes owns one token (a 16-lane DPP row for
// E <= 256, so four tokens per wave; the whole wave for larger E); lane l of
// the group holds experts l, l+L, l+2L, ... as 64-bit keys (order-preserving
// image of the fp32 value << 32 | ~expert id), so "larger value, then lower
// id" is a single unsigned max.  k rounds of a group max pick the experts in
// output order; the winner's lane retires that key.  The max runs in the
// VALU: DPP row reductions (quad_perm / row_half_mirror / row_mirror), plus
// four v_readlane of the row results when a token spans the wave, so no LDS
// round trip sits on the dependency chain.  The k-way softmax is evaluated
// in double by lanes 0..k-1 of the group (k <= 16: one DPP row sum); it is
// ~0.4% of the path's bytes and makes the fp32 weights correctly rounded up
// to one double rounding.
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

// Top-k of token t by the group of L lanes this lane belongs to (L = 16:
// four tokens per wave, for E <= 256; L = 64: one token per wave).  NE =
// keys per lane = ceil(E / L).  Absent experts hold key 0, below every finite
// logit (the smallest finite key is 0x00800000 << 32).  With L = 16 every
// reduction stays inside a 16-lane DPP row, so there is no cross-row step.
// Lanes sub < k of a valid token write idx/w and return the expert they
// hold; every other lane returns -1.  All lanes of the wave must call it.
template <int NE, int L>
__device__ __forceinline__ int route_token(const float *__restrict__ logits, int64_t t, bool ok,
                                           int E, int k, int32_t *__restrict__ idx,
                                           float *__restrict__ w)
{
    const int sub = lane_id() % L;
    const float *row = logits + (ok ? t : 0) * E;

    uint64_t key[NE];
#pragma unroll
    for (int i = 0; i < NE; ++i) {
        const int e = i * L + sub;
        key[i] = (ok && e < E) ? make_key(row[e], e) : 0ull;
    }

    uint64_t mine = 0;   // lane sub = j keeps the token's j-th selected key
    uint64_t first = 0;  // the token's largest key
    for (int r = 0; r < k; ++r) {
        uint64_t best = key[0];
#pragma unroll
        for (int i = 1; i < NE; ++i)
            best = umax64(key[i], best);
        const uint64_t top = (L == kWave) ? wave_max_u64_dpp(best) : row_max_u64(best);
        if (r == 0)
            first = top;
#pragma unroll
        for (int i = 0; i < NE; ++i)
            key[i] = (key[i] == top) ? 0ull : key[i];  // ids are distinct: one match
        if (sub == r)
            mine = top;
    }

    // k <= 16: the selected keys live in lanes 0..k-1 of the token's first row
    const bool sel = ok && sub < k;
    const double lmax = static_cast<double>(key_value(first));
    const double a = sel ? exp(static_cast<double>(key_value(mine)) - lmax) : 0.0;
    const double s = row_sum_f64(a);
    if (!sel)
        return -1;
    const int e = key_expert(mine);
    idx[t * k + sub] = e;
    w[t * k + sub] = static_cast<float>(a / s);
    return e;
}

template <int NE, int L>
__global__ __launch_bounds__(256) void route_topk_kernel(const float *__restrict__ logits,
                                                         int64_t T, int E, int k,
                                                         int32_t *__restrict__ idx,
                                                         float *__restrict__ w)
{
    constexpr int kTokensPerWave = kWave / L;
    const int64_t wave = static_cast<int64_t>(blockIdx.x) * 4 + uniform(threadIdx.x / kWave);
    if (wave * kTokensPerWave >= T)
        return;  // whole wave past the end
    const int64_t t = wave * kTokensPerWave + lane_id() / L;
    route_token<NE, L>(logits, t, t < T, E, k, idx, w);
}

// Routing fused with the first pass of the dispatch layout: block (g, c)
// routes group g of chunk c (kGroupTokens consecutive tokens of the chunk,
// the last group possibly shorter) and writes the group's expert histogram
// as row g of chunk c's histogram matrix, hist[c][g][E], so the layout does
// not read the expert ids a second time to count them.
template <int NE, int L>
__global__ __launch_bounds__(256) void route_hist_kernel(const float *__restrict__ logits,
                                                         int64_t T, int64_t chunk_tokens, int E,
                                                         int k, int hrows,
                                                         int32_t *__restrict__ idx,
                                                         float *__restrict__ w,
                                                         int32_t *__restrict__ hist)
{
    extern __shared__ int32_t h[];
    constexpr int kTokensPerWave = kWave / L;
    constexpr int kGroupTokens = 4 * kTokensPerWave;
    for (int e = threadIdx.x; e < E; e += blockDim.x)
        h[e] = 0;
    __syncthreads();
    const int64_t c0 = static_cast<int64_t>(blockIdx.y) * chunk_tokens;
    const int64_t c1 = min(T, c0 + chunk_tokens);
    const int64_t t = c0 + static_cast<int64_t>(blockIdx.x) * kGroupTokens +
                      uniform(threadIdx.x / kWave) * kTokensPerWave + lane_id() / L;
    const int e = route_token<NE, L>(logits, t, t < c1, E, k, idx, w);
    if (e >= 0)
        atomicAdd(&h[e], 1);
    __syncthreads();
    int32_t *row = hist + (static_cast<int64_t>(blockIdx.y) * hrows + blockIdx.x) * E;
    for (int x = threadIdx.x; x < E; x += blockDim.x)
        row[x] = h[x];
}

}  // namespace

hipError_t launch_route_topk(const float *logits, int64_t T, int E, int k,
                             int32_t *idx, float *w, hipStream_t stream)
{
    const dim3 block(256);
    if (E <= 256) {  // 16 lanes per token, 16 tokens per block
        const dim3 grid(static_cast<unsigned>((T + 15) / 16));
        if (E <= 16)
            route_topk_kernel<1, 16><<<grid, block, 0, stream>>>(logits, T, E, k, idx, w);
        else if (E <= 32)
            route_topk_kernel<2, 16><<<grid, block, 0, stream>>>(logits, T, E, k, idx, w);
        else if (E <= 64)
            route_topk_kernel<4, 16><<<grid, block, 0, stream>>>(logits, T, E, k, idx, w);
        else if (E <= 128)
            route_topk_kernel<8, 16><<<grid, block, 0, stream>>>(logits, T, E, k, idx, w);
        else
            route_topk_kernel<16, 16><<<grid, block, 0, stream>>>(logits, T, E, k, idx, w);
    } else {  // one wave per token
        const dim3 grid(static_cast<unsigned>((T + 3) / 4));
        if (E <= 512)
            route_topk_kernel<8, 64><<<grid, block, 0, stream>>>(logits, T, E, k, idx, w);
        else
            route_topk_kernel<16, 64><<<grid, block, 0, stream>>>(logits, T, E, k, idx, w);
    }
    return hipGetLastError();
}

int route_group_tokens(int E) { return E <= 256 ? 16 : 4; }

hipError_t launch_route_hist(const float *logits, int64_t T, int64_t chunk_tokens, int chunks,
                             int E, int k, int hrows, int32_t *idx, float *w, int32_t *hist,
                             hipStream_t stream)
{
    const dim3 block(256);
    const dim3 grid(static_cast<unsigned>(hrows), static_cast<unsigned>(chunks));
    const size_t lds = static_cast<size_t>(E) * sizeof(int32_t);
    const int64_t C = chunk_tokens;
    if (E <= 16)
        route_hist_kernel<1, 16><<<grid, block, lds, stream>>>(logits, T, C, E, k, hrows, idx, w, hist);
    else if (E <= 32)
        route_hist_kernel<2, 16><<<grid, block, lds, stream>>>(logits, T, C, E, k, hrows, idx, w, hist);
    else if (E <= 64)
        route_hist_kernel<4, 16><<<grid, block, lds, stream>>>(logits, T, C, E, k, hrows, idx, w, hist);
    else if (E <= 128)
        route_hist_kernel<8, 16><<<grid, block, lds, stream>>>(logits, T, C, E, k, hrows, idx, w, hist);
    else if (E <= 256)
        route_hist_kernel<16, 16><<<grid, block, lds, stream>>>(logits, T, C, E, k, hrows, idx, w, hist);
    else if (E <= 512)
        route_hist_kernel<8, 64><<<grid, block, lds, stream>>>(logits, T, C, E, k, hrows, idx, w, hist);
    else
        route_hist_kernel<16, 64><<<grid, block, lds, stream>>>(logits, T, C, E, k, hrows, idx, w, hist);
    return hipGetLastError();
}

}  // namespace moe
