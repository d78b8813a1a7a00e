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
// E <= 256, so four tokens per wave; the whole wave for larger E); each lane
// holds ceil(E/L) of the token's experts (a contiguous run read with 16-byte
// loads when rows allow it) as 64-bit keys (order-preserving image of the
// fp32 value << 32 | ~expert id), so "larger value, then lower id" is a
// single unsigned max.  k rounds of a group max pick the experts in
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

// Compare-exchange: the larger key to a, the smaller to b.
__device__ __forceinline__ void ce_desc(uint64_t &a, uint64_t &b)
{
    const bool gt = a > b;
    const uint64_t hi = gt ? a : b;
    const uint64_t lo = gt ? b : a;
    a = hi;
    b = lo;
}

// 32-bit keys: one v_max_u32 and one v_min_u32.
__device__ __forceinline__ void ce_desc(uint32_t &a, uint32_t &b)
{
    const uint32_t hi = max(a, b);
    const uint32_t lo = min(a, b);
    a = hi;
    b = lo;
}

// Batcher's odd-even merge sort of N (a power of two) keys, descending: for
// merge widths p = 1, 2, 4, ... and distances q = p, p/2, ..., 1, compare
// elements q apart that lie in the same 2p-block (19 comparators for N = 8,
// against 24 for a bitonic sort).  Fully unrolled: all indices are
// compile-time, so the keys stay in registers.
template <int N, typename K>
__device__ __forceinline__ void sort_desc(K *a)
{
#pragma unroll
    for (int p = 1; p < N; p <<= 1)
#pragma unroll
        for (int q = p; q >= 1; q >>= 1)
#pragma unroll
            for (int j = q % p; j + q < N; j += 2 * q)
#pragma unroll
                for (int i = 0; i < q; ++i)
                    if (i + j + q < N && (i + j) / (2 * p) == (i + j + q) / (2 * p))
                        ce_desc(a[i + j], a[i + j + q]);
}

// Max of a 32-bit value over one 16-lane row; every lane of the row gets it.
__device__ __forceinline__ uint32_t row_max_u32(uint32_t v)
{
    v = max(v, dpp32<0xB1>(v));
    v = max(v, dpp32<0x4E>(v));
    v = max(v, dpp32<0x141>(v));
    v = max(v, dpp32<0x140>(v));
    return v;
}

// Selection for 16 lanes per token whose experts are contiguous per lane
// (lane sub owns [sub*NE, sub*NE + NE)), k <= kSortedMaxK.  Each lane sorts
// its keys once and keeps its S = min(NE, 8) largest in order: a lane can
// supply at most min(k, NE) <= S of the token's k picks.  Each round then
// looks only at list heads: the row max of their value words (32-bit DPP),
// the lowest lane of the row holding that value wins (lower lanes own lower
// expert ids, and a lane's head is its lowest id at its largest value, so
// this is the "larger value, then lower id" order), a second row max
// broadcasts the winner's id word, and the winner pops its head.  About a
// third of the VALU work of k rounds of 64-bit max-and-retire over every key.
constexpr int kSortedMaxK = 8;

// The per-lane list lives in one vector value, not an array: a conditional
// pop written on an array (list[i] = win ? list[i+1] : list[i]) is folded by
// the compiler into a load from list[i + win], a dynamic index it lowers as
// a compare-and-select chain over every element (~150 VALU per round).
typedef uint64_t u64x4 __attribute__((ext_vector_type(4)));
typedef uint64_t u64x8 __attribute__((ext_vector_type(8)));

template <int S>
struct KeyList;
template <>
struct KeyList<4> {
    typedef u64x4 type;
    static __device__ __forceinline__ type pop(type v)
    {
        return __builtin_shufflevector(v, type{0, 0, 0, 0}, 1, 2, 3, 4);
    }
};
template <>
struct KeyList<8> {
    typedef u64x8 type;
    static __device__ __forceinline__ type pop(type v)
    {
        return __builtin_shufflevector(v, type{0, 0, 0, 0, 0, 0, 0, 0}, 1, 2, 3, 4, 5, 6, 7, 8);
    }
};

template <int NE>
__device__ __forceinline__ void select_sorted(uint64_t *key, int k, int sub, uint64_t &first,
                                              uint64_t &mine)
{
    static_assert(NE == 4 || NE == 8 || NE == 16, "sorted selection: NE in {4, 8, 16}");
    constexpr int S = NE < 8 ? NE : 8;
    uint64_t list[S];
    if constexpr (NE <= 8) {
        sort_desc<NE>(key);
#pragma unroll
        for (int i = 0; i < S; ++i)
            list[i] = key[i];
    } else {
        // both halves sorted; the top 8 of their union is max(a[i], b[7-i]),
        // a bitonic sequence, which three half-cleaner stages sort
        sort_desc<8>(key);
        sort_desc<8>(key + 8);
#pragma unroll
        for (int i = 0; i < 8; ++i)
            list[i] = umax64(key[i], key[15 - i]);
#pragma unroll
        for (int q = 4; q >= 1; q >>= 1)
#pragma unroll
            for (int i = 0; i < 8; ++i)
                if ((i & q) == 0)
                    ce_desc(list[i], list[i + q]);
    }
    using L = KeyList<S>;
    typename L::type v;
#pragma unroll
    for (int i = 0; i < S; ++i)
        v[i] = list[i];
    const int lane = lane_id();
    const uint64_t below = ((1ull << lane) - 1ull) & (0xFFFFull << (lane & ~15));
    uint32_t top0 = 0;
    mine = 0;
    for (int r = 0; r < k; ++r) {
        const uint64_t head = v[0];
        const uint32_t hv = static_cast<uint32_t>(head >> 32);
        const uint32_t top = row_max_u32(hv);
        const bool eq = hv == top;
        const bool win = eq && (__ballot(eq) & below) == 0;
        const uint32_t lo = row_max_u32(win ? static_cast<uint32_t>(head) : 0u);
        if (r == 0)
            top0 = top;
        if (sub == r)
            mine = (static_cast<uint64_t>(top) << 32) | lo;
        const typename L::type popped = L::pop(v);
#pragma unroll
        for (int i = 0; i < S; ++i)
            v[i] = win ? popped[i] : v[i];
    }
    first = static_cast<uint64_t>(top0) << 32;
}

// Fast selection on 32-bit keys (16 lanes per token, lane sub owning the
// contiguous experts [sub*NE, sub*NE + NE), E = 16 * NE <= 256, k <= 8).
// The key of expert e is the order-preserving image `ord` of its logit (-0
// mapped with +0) with the low 8 bits replaced by 255 - e: K = (ord | 255) -
// e.  K orders keys by the prefix ord >> 8, then by the lower id, and carries
// the id, so a compare-exchange is a v_max_u32 and a v_min_u32 (against a
// 64-bit compare, four selects and their wait states) and a round needs one
// row max instead of two.  Each lane sorts its keys once and keeps its S =
// min(NE, 9) largest: a lane supplies at most k <= 8 picks, so its next key
// after them is always still listed.  Then k rounds of row max over the list
// heads, the winner popping its head, as in select_sorted.
//
// Exactness.  Let f1 > ... > f(k+1) be the k+1 largest keys in K order.  If
// their prefixes strictly decrease, any other key z has prefix(z) <=
// prefix(f(k+1)) < prefix(fk), so z lies below fk in the exact order (ord,
// then lower id) as well, and f1..fk, ordered by distinct prefixes, are in
// exact order: the K selection is the exact one.  The rounds compare each
// pick's prefix with the previous pick's, and f(k+1)'s (the row max left
// after the k rounds) with fk's.  When any token of the wave has two equal
// prefixes there (ties, or logits less than 256 ulps apart at the cut that
// share their image's top 24 bits), the function returns false and the
// caller redoes the wave with 64-bit keys.
//
// key[i] (sorted in place) is the key of the lane's expert sub*NE + i.
// Outputs (valid when it returns true): `first` is the token's largest key,
// `mine` on lane sub = j < k the key of the j-th pick; expert = 255 - (key &
// 255).
__device__ __forceinline__ uint32_t ord32(uint32_t u)
{
    const uint32_t m = static_cast<uint32_t>(static_cast<int32_t>(u) >> 31);
    return (u ^ (m | 0x80000000u)) - m;  // negative: -u, so -0 -> 0x80000000 as +0
}

// The logit (bits) whose image is o: the inverse of ord32 (-0 comes back +0).
__device__ __forceinline__ uint32_t unord32(uint32_t o)
{
    return (o & 0x80000000u) ? (o & 0x7FFFFFFFu) : (0u - o);
}

typedef uint32_t u32x16 __attribute__((ext_vector_type(16)));

template <int NE>
__device__ __forceinline__ bool select_fast(uint32_t *key, int k, int sub, uint32_t &first,
                                            uint32_t &mine)
{
    static_assert(NE == 4 || NE == 8 || NE == 16, "fast selection: NE in {4, 8, 16}");
    constexpr int S = NE < 9 ? NE : 9;
    sort_desc<NE>(key);  // the compiler drops what feeds only keys past S
    // the list lives in one vector value (see KeyList): pops shift it down
    u32x16 v = {};
#pragma unroll
    for (int i = 0; i < S; ++i)
        v[i] = key[i];
    bool flag = false;
    uint32_t prev = 0;
    mine = 0;
    first = 0;
    for (int r = 0; r < k; ++r) {
        const uint32_t top = row_max_u32(v[0]);
        if (r == 0)
            first = top;
        else
            flag |= (top ^ prev) < 256u;  // same prefix as the previous pick
        prev = top;
        const bool win = v[0] == top;  // keys are distinct within a token
        if (sub == r)
            mine = top;
        const u32x16 popped = __builtin_shufflevector(v, u32x16{}, 1, 2, 3, 4, 5, 6, 7, 8, 9,
                                                      10, 11, 12, 13, 14, 15, 16);
#pragma unroll
        for (int i = 0; i < S; ++i)
            v[i] = win ? popped[i] : v[i];
    }
    flag |= (row_max_u32(v[0]) ^ prev) < 256u;  // f(k+1) against fk
    return __ballot(flag) == 0;
}

// Top-k of token t by the group of L lanes this lane belongs to (L = 16:
// four tokens per wave, for E <= 256; L = 64: one token per wave).  NE =
// keys per lane = ceil(E / L).  Absent experts hold key 0, below every finite
// logit (the smallest finite key is 0x00800000 << 32).  With L = 16 every
// reduction stays inside a 16-lane DPP row, so there is no cross-row step.
// Lanes sub < k of a valid token write idx/w and return the expert they
// hold; every other lane returns -1.  All lanes of the wave must call it.
//
// VEC (E % 4 == 0 and 16-byte aligned rows; NE % 4 == 0): lane sub owns the
// contiguous experts [sub*NE, sub*NE + NE) and reads them with NE/4 16-byte
// loads from clamped, always-valid addresses, issued together; keys past E
// are masked afterwards.  Otherwise lane sub owns experts sub, sub+L, ...
// with one 4-byte load each, which the compiler keeps under a branch per
// load and waits on one at a time.  Which lane holds which expert does not
// change the result: every key carries its expert id.
//
// stash: E bytes of LDS for this token, or null.  With it (VEC, L = 16, E =
// 16 * NE, k <= 8) the 32-bit selection (select_fast) runs first and the
// 64-bit one only for waves it flags; both give the same ids and weights.
template <int NE, int L, bool VEC>
__device__ __forceinline__ int route_token(const float *__restrict__ logits, int64_t t, bool ok,
                                           int E, int k, int32_t *__restrict__ idx,
                                           float *__restrict__ w, uint8_t *stash)
{
    const int sub = lane_id() % L;
    const float *row = logits + (ok ? t : 0) * E;

    uint64_t key[NE];
    if constexpr (VEC) {
        static_assert(NE % 4 == 0, "vector path needs NE % 4 == 0");
        u32x4 q[NE / 4];
#pragma unroll
        for (int c = 0; c < NE / 4; ++c) {
            const int e0 = sub * NE + 4 * c;
            q[c] = *reinterpret_cast<const u32x4 *>(row + (e0 < E ? e0 : E - 4));
        }
        if constexpr (L == 16 && NE >= 4) {
            // every lane holds NE real experts: the 32-bit fast path
            if (stash && E == NE * L && k <= kSortedMaxK) {  // uniform
                // keys, and the low byte of every expert's image in LDS (the
                // keys keep the top 24 bits): the picks' exact logits are
                // rebuilt from their keys and these bytes.  The token's
                // bytes are written and read by this wave only, in order.
                uint32_t key[NE];
                uint32_t low[NE / 4] = {};
#pragma unroll
                for (int c = 0; c < NE / 4; ++c)
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const uint32_t o = ord32(q[c][j]);
                        key[4 * c + j] = (o | 0xFFu) - static_cast<uint32_t>(sub * NE + 4 * c + j);
                        low[c] |= (o & 0xFFu) << (8 * j);
                    }
                uint32_t *st = reinterpret_cast<uint32_t *>(stash) + sub * (NE / 4);
#pragma unroll
                for (int c = 0; c < NE / 4; ++c)
                    st[c] = low[c];
                uint32_t first32, mine32;
                if (select_fast<NE>(key, k, sub, first32, mine32)) {
                    const bool sel = ok && sub < k;
                    const int e = 255 - static_cast<int>(mine32 & 0xFFu);
                    const int e_top = 255 - static_cast<int>(first32 & 0xFFu);
                    const uint32_t bm = sel ? stash[e] : 0u;  // lanes sub >= k hold no pick
                    const float lm = __uint_as_float(unord32((mine32 & 0xFFFFFF00u) | bm));
                    const float l0 =
                        __uint_as_float(unord32((first32 & 0xFFFFFF00u) | stash[e_top]));
                    const double a = sel ? exp(static_cast<double>(lm) - static_cast<double>(l0))
                                         : 0.0;
                    const double s = row_sum_f64(a);
                    if (!sel)
                        return -1;
                    idx[t * k + sub] = e;
                    w[t * k + sub] = static_cast<float>(a / s);
                    return e;
                }
            }
        }
#pragma unroll
        for (int c = 0; c < NE / 4; ++c)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int e = sub * NE + 4 * c + j;
                key[4 * c + j] = (ok && e < E) ? make_key(__uint_as_float(q[c][j]), e) : 0ull;
            }
    } else {
#pragma unroll
        for (int i = 0; i < NE; ++i) {
            const int e = i * L + sub;
            key[i] = (ok && e < E) ? make_key(row[e], e) : 0ull;
        }
    }

    uint64_t mine = 0;   // lane sub = j keeps the token's j-th selected key
    uint64_t first = 0;  // the token's largest key (its value word is what is used)
    bool sorted = false;
    if constexpr (VEC && L == 16 && NE >= 4) {
        if (k <= kSortedMaxK) {  // uniform
            select_sorted<NE>(key, k, sub, first, mine);
            sorted = true;
        }
    }
    for (int r = 0; r < (sorted ? 0 : k); ++r) {
        // this lane's largest key: a tree of depth log2(NE), not a chain of
        // NE - 1 dependent compares (few waves per SIMD hide little latency)
        uint64_t m[NE];
#pragma unroll
        for (int i = 0; i < NE; ++i)
            m[i] = key[i];
#pragma unroll
        for (int w = NE / 2; w >= 1; w /= 2)
#pragma unroll
            for (int i = 0; i < w; ++i)
                m[i] = umax64(m[i], m[i + w]);
        const uint64_t best = m[0];
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

// `stash` (fast 32-bit selection only): E bytes of LDS per token of the block.
template <int NE, int L, bool VEC>
__global__ __launch_bounds__(256) void route_topk_kernel(const float *__restrict__ logits,
                                                         int64_t T, int E, int k,
                                                         int32_t *__restrict__ idx,
                                                         float *__restrict__ w, int stash)
{
    extern __shared__ uint8_t lds_bytes[];
    constexpr int kTokensPerWave = kWave / L;
    const int tb = uniform(threadIdx.x / kWave) * kTokensPerWave + lane_id() / L;
    const int64_t wave = static_cast<int64_t>(blockIdx.x) * 4 + uniform(threadIdx.x / kWave);
    if (wave * kTokensPerWave >= T)
        return;  // whole wave past the end
    const int64_t t = wave * kTokensPerWave + lane_id() / L;
    route_token<NE, L, VEC>(logits, t, t < T, E, k, idx, w, stash ? lds_bytes + tb * E : nullptr);
}

// Routing fused with the first pass of the dispatch layout: block (g, c)
// routes group g of chunk c (the block's consecutive tokens of the chunk,
// the last group possibly shorter) and writes the group's expert histogram
// as row g of chunk c's histogram matrix, hist[c][g][E], so the layout does
// not read the expert ids a second time to count them.  A group is the
// tokens of one block: 16 waves when the batch has enough tokens for one
// such block per CU (every rank block of the layout folds all of its
// chunk's rows, so coarser rows shorten that fold 4x at the same
// occupancy), else 4 waves, so that small batches still spread over many
// CUs.  The kernel reads its group size from its block size.
template <int NE, int L, bool VEC>
__global__ __launch_bounds__(1024) void route_hist_kernel(const float *__restrict__ logits,
                                                         int64_t T, int64_t chunk_tokens, int E,
                                                         int k, int hrows,
                                                         int32_t *__restrict__ idx,
                                                         float *__restrict__ w,
                                                         int32_t *__restrict__ hist, int stash)
{
    extern __shared__ int32_t h[];  // [E] counts, then E stash bytes per token
    constexpr int kTokensPerWave = kWave / L;
    const int group_tokens = static_cast<int>(blockDim.x / kWave) * kTokensPerWave;
    const int tb = uniform(threadIdx.x / kWave) * kTokensPerWave + lane_id() / L;
    uint8_t *st = stash ? reinterpret_cast<uint8_t *>(h + E) + tb * E : nullptr;
    for (int e = threadIdx.x; e < E; e += blockDim.x)
        h[e] = 0;
    __syncthreads();
    const int64_t c0 = static_cast<int64_t>(blockIdx.y) * chunk_tokens;
    const int64_t c1 = min(T, c0 + chunk_tokens);
    const int64_t t = c0 + static_cast<int64_t>(blockIdx.x) * group_tokens +
                      uniform(threadIdx.x / kWave) * kTokensPerWave + lane_id() / L;
    const int e = route_token<NE, L, VEC>(logits, t, t < c1, E, k, idx, w, st);
    if (e >= 0)
        atomicAdd(&h[e], 1);
    __syncthreads();
    int32_t *row = hist + (static_cast<int64_t>(blockIdx.y) * hrows + blockIdx.x) * E;
    for (int x = threadIdx.x; x < E; x += blockDim.x)
        row[x] = h[x];
}

}  // namespace

// The vector path needs whole 16-byte expert groups in aligned rows.
static bool vec_rows(const float *logits, int E)
{
    return (E % 4) == 0 && (reinterpret_cast<uintptr_t>(logits) & 15) == 0;
}

#define MOE_ROUTE_DISPATCH(KERNEL, GRID, LDS, ...)                                            \
    do {                                                                                      \
        const bool vec = vec_rows(logits, E);                                                 \
        if (E <= 16)                                                                          \
            KERNEL<1, 16, false><<<GRID, block, LDS, stream>>>(__VA_ARGS__);                  \
        else if (E <= 32)                                                                     \
            KERNEL<2, 16, false><<<GRID, block, LDS, stream>>>(__VA_ARGS__);                  \
        else if (E <= 64)                                                                     \
            vec ? KERNEL<4, 16, true><<<GRID, block, LDS, stream>>>(__VA_ARGS__)              \
                : KERNEL<4, 16, false><<<GRID, block, LDS, stream>>>(__VA_ARGS__);            \
        else if (E <= 128)                                                                    \
            vec ? KERNEL<8, 16, true><<<GRID, block, LDS, stream>>>(__VA_ARGS__)              \
                : KERNEL<8, 16, false><<<GRID, block, LDS, stream>>>(__VA_ARGS__);            \
        else if (E <= 256)                                                                    \
            vec ? KERNEL<16, 16, true><<<GRID, block, LDS, stream>>>(__VA_ARGS__)             \
                : KERNEL<16, 16, false><<<GRID, block, LDS, stream>>>(__VA_ARGS__);           \
        else if (E <= 512)                                                                    \
            vec ? KERNEL<8, 64, true><<<GRID, block, LDS, stream>>>(__VA_ARGS__)              \
                : KERNEL<8, 64, false><<<GRID, block, LDS, stream>>>(__VA_ARGS__);            \
        else                                                                                  \
            vec ? KERNEL<16, 64, true><<<GRID, block, LDS, stream>>>(__VA_ARGS__)             \
                : KERNEL<16, 64, false><<<GRID, block, LDS, stream>>>(__VA_ARGS__);           \
    } while (0)

// Whether the router takes the 32-bit fast selection (a stash of E bytes of
// LDS per token): 16 lanes per token, each holding NE = E / 16 in {8, 16}
// whole experts read with 16-byte loads, and k <= 8.  At E = 64 (four keys
// per lane) the sort saves little and the T=4096 router, one wave per SIMD,
// took 4.6 us against 4.2 with 64-bit keys; E = 256 (T=16384) went from
// 10.4 to 8.7-9.9 us and E = 128 (T=32768) from 11.6 to 10.1-10.9.
static bool route_stash(const float *logits, int E, int k)
{
    return vec_rows(logits, E) && (E == 128 || E == 256) && k <= 8;
}

// 16 lanes per token (16 tokens per block) for E <= 256, else a wave per token
int64_t route_topk_blocks(int64_t T, int E) { return E <= 256 ? (T + 15) / 16 : (T + 3) / 4; }

hipError_t launch_route_topk(const float *logits, int64_t T, int E, int k,
                             int32_t *idx, float *w, hipStream_t stream)
{
    const dim3 block(kRouteThreads);
    const dim3 grid(static_cast<unsigned>(route_topk_blocks(T, E)));
    const int stash = route_stash(logits, E, k) ? 1 : 0;
    const size_t lds = stash ? static_cast<size_t>(16) * E : 0;
    MOE_ROUTE_DISPATCH(route_topk_kernel, grid, lds, logits, T, E, k, idx, w, stash);
    return hipGetLastError();
}

// Waves per block of the fused router: 16 once the batch fills one such
// block per CU (256 CUs), else 4.
static int route_hist_waves(int64_t T, int E)
{
    const int64_t per_wave = E <= 256 ? 4 : 1;
    return T >= 256 * 16 * per_wave ? 16 : 4;
}

int route_group_tokens(int E, int64_t T) { return (E <= 256 ? 4 : 1) * route_hist_waves(T, E); }

hipError_t launch_route_hist(const float *logits, int64_t T, int64_t chunk_tokens, int chunks,
                             int E, int k, int hrows, int32_t *idx, float *w, int32_t *hist,
                             hipStream_t stream)
{
    const dim3 block(static_cast<unsigned>(kWave * route_hist_waves(T, E)));
    const dim3 grid(static_cast<unsigned>(hrows), static_cast<unsigned>(chunks));
    const int stash = route_stash(logits, E, k) ? 1 : 0;
    const size_t lds = static_cast<size_t>(E) * sizeof(int32_t) +
                       (stash ? static_cast<size_t>(route_group_tokens(E, T)) * E : 0);
    MOE_ROUTE_DISPATCH(route_hist_kernel, grid, lds, logits, T, chunk_tokens, E, k, hrows, idx,
                       w, hist, stash);
    return hipGetLastError();
}

#undef MOE_ROUTE_DISPATCH

}  // namespace moe
