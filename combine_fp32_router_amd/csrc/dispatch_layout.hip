// Dispatch layout: per-expert histogram, scans, per-rank blocks and the
// stable slot <-> row maps.
//
// What it computes (aggregation by destination, ThunderEP write-up s2.1;
// contiguous expert placement, communication-wall EP example; flat buffer cut
// at prefix sums of the per-rank counts, NCCL EP article s3.3; capacity
// factor, sparse-communication article s2.1): rows are ordered by (rank,
// expert, token); expert e keeps its first min(count_e, capacity) slots in
// slot order; pos[s] = row of slot s or -1; row_src[p] = slot of row p or -1.
//
// gfx950 design: two small deterministic kernels, no global atomics.  The
// slots are cut into tiles of `tile_slots`, one tile per wavefront, four
// tiles per 256-thread block.
//   1. hist: each wave counts its tile into a private LDS histogram (slot
//      ids prefetched kBatch rounds at a time) and writes it as row `tile` of
//      hist[ntiles][E].
//   2. rank: every block reads the whole histogram matrix (coalesced, LDS
//      atomics to fold it): per-expert totals, the count of each expert in
//      the tiles before its own, and its four tiles' counts.  From the
//      totals it forms the kept counts and the exclusive expert offsets (a
//      block scan of <= 1024 values in LDS); block 0 writes the counts and
//      offsets.  Then each wave walks its tile in slot order, 64 slots a
//      step: lanes holding the same expert find each other with ceil(log2 E)
//      ballots; a lane's rank is base[e] + (earlier lanes with e), and the
//      group's last lane advances base[e].  That is the sequential
//      token-order definition, evaluated one wave-step at a time.
#include "common.hpp"
#include "launch.hpp"

namespace moe {
namespace {

constexpr int kBlock = 256;
constexpr int kWavesPerBlock = kBlock / kWave;
constexpr int kBatch = 8;  // slot-id loads each lane keeps in flight

__global__ __launch_bounds__(kBlock) void layout_hist_kernel(const int32_t *__restrict__ idx,
                                                             int64_t S, int E, int tile_slots,
                                                             int ntiles, int32_t *__restrict__ hist)
{
    extern __shared__ int32_t lds[];
    const int w = threadIdx.x / kWave;
    const int lane = lane_id();
    int32_t *h = lds + w * E;
    for (int e = lane; e < E; e += kWave)
        h[e] = 0;
    __syncthreads();
    const int tile = blockIdx.x * kWavesPerBlock + w;
    if (tile < ntiles) {
        const int64_t s0 = static_cast<int64_t>(tile) * tile_slots;
        const int64_t s1 = min(S, s0 + tile_slots);
        for (int64_t base = s0; base < s1; base += kWave * kBatch) {
            int e[kBatch];
#pragma unroll
            for (int b = 0; b < kBatch; ++b) {
                const int64_t s = base + b * kWave + lane;
                e[b] = (s < s1) ? idx[s] : -1;
            }
#pragma unroll
            for (int b = 0; b < kBatch; ++b)
                if (static_cast<unsigned>(e[b]) < static_cast<unsigned>(E))  // ids outside [0,E) are not counted
                    atomicAdd(&h[e[b]], 1);
        }
    }
    __syncthreads();
    if (tile < ntiles)
        for (int e = lane; e < E; e += kWave)
            hist[static_cast<int64_t>(tile) * E + e] = h[e];
}

__global__ __launch_bounds__(kBlock) void layout_rank_kernel(
    const int32_t *__restrict__ idx, int64_t S, int E, int R, int cap, int tile_slots, int ntiles,
    int nbits, const int32_t *__restrict__ hist, int32_t *__restrict__ expert_counts,
    int32_t *__restrict__ expert_offsets, int32_t *__restrict__ rank_counts,
    int32_t *__restrict__ rank_offsets, int32_t *__restrict__ pos, int32_t *__restrict__ row_src)
{
    extern __shared__ int32_t lds[];
    int32_t *cnt = lds;                        // [4][E] this block's tile counts, then rank bases
    int32_t *before = cnt + kWavesPerBlock * E;  // [E] count in tiles before this block's
    int32_t *total = before + E;                // [E]
    int32_t *kept = total + E;                  // [E]
    int32_t *eoff = kept + E;                   // [E+1]
    int32_t *wsum = eoff + E + 1;               // [4]
    const int tid = threadIdx.x;
    const int w = tid / kWave;
    const int lane = lane_id();
    const int tile0 = blockIdx.x * kWavesPerBlock;

    for (int i = tid; i < (kWavesPerBlock + 2) * E; i += kBlock)
        lds[i] = 0;
    __syncthreads();
    // Fold the histogram matrix.  Column e is summed by `g` threads, each
    // taking every g-th tile; a thread issues kFold loads before it adds
    // anything, so the fold costs a few L2 round trips, not one per tile.
    // Consecutive threads read consecutive experts (coalesced rows).
    {
        constexpr int kFold = 16;
        const int g = (E >= kBlock) ? 1 : kBlock / E;
        const int sub = tid / E;  // which tile subset (>= g: idle when E < 256)
        for (int e = tid % E; sub < g && e < E; e += (g == 1 ? kBlock : E)) {
            int tot = 0, bef = 0;
            for (int t0 = sub; t0 < ntiles; t0 += g * kFold) {
                int v[kFold];
#pragma unroll
                for (int b = 0; b < kFold; ++b) {
                    const int t = t0 + b * g;
                    v[b] = (t < ntiles) ? hist[static_cast<int64_t>(t) * E + e] : 0;
                }
#pragma unroll
                for (int b = 0; b < kFold; ++b) {
                    const int t = t0 + b * g;
                    tot += v[b];
                    if (t < tile0)
                        bef += v[b];
                    else if (t < tile0 + kWavesPerBlock)
                        cnt[(t - tile0) * E + e] = v[b];
                }
            }
            if (g == 1) {
                total[e] = tot;
                before[e] = bef;
            } else {
                atomicAdd(&total[e], tot);
                atomicAdd(&before[e], bef);
            }
        }
    }
    __syncthreads();
    for (int e = tid; e < E; e += kBlock) {
        const int c = total[e];
        kept[e] = (cap > 0 && c > cap) ? cap : c;
        int run = before[e];
#pragma unroll
        for (int q = 0; q < kWavesPerBlock; ++q) {
            const int v = cnt[q * E + e];
            cnt[q * E + e] = run;
            run += v;
        }
        if (blockIdx.x == 0)
            expert_counts[e] = c;
    }
    __syncthreads();

    // exclusive scan of kept over experts: each thread owns a contiguous run
    const int per = (E + kBlock - 1) / kBlock;
    const int e0 = tid * per;
    int local = 0;
    for (int i = 0; i < per; ++i)
        if (e0 + i < E)
            local += kept[e0 + i];
    const int incl = wave_inclusive_scan(local);
    if (lane == kWave - 1)
        wsum[w] = incl;
    __syncthreads();
    int run = incl - local;
    for (int i = 0; i < w; ++i)
        run += wsum[i];
    for (int i = 0; i < per; ++i) {
        const int e = e0 + i;
        if (e < E) {
            eoff[e] = run;
            run += kept[e];
        }
    }
    if (tid == kBlock - 1)
        eoff[E] = run;  // threads past E add nothing: the last one holds N
    __syncthreads();
    const int N = eoff[E];

    if (blockIdx.x == 0) {
        const int per_rank = E / R;
        for (int e = tid; e <= E; e += kBlock)
            expert_offsets[e] = eoff[e];
        for (int r = tid; r < R; r += kBlock) {
            rank_offsets[r] = eoff[r * per_rank];
            rank_counts[r] = eoff[(r + 1) * per_rank] - eoff[r * per_rank];
        }
        if (tid == 0)
            rank_offsets[R] = N;
    }

    const int tile = tile0 + w;
    if (tile < ntiles) {
        int32_t *c = cnt + w * E;
        const int64_t s0 = static_cast<int64_t>(tile) * tile_slots;
        const int64_t s1 = min(S, s0 + tile_slots);
        const uint64_t lt = (1ull << lane) - 1ull;
        for (int64_t base = s0; base < s1; base += kWave * kBatch) {
            int eb[kBatch];
#pragma unroll
            for (int b = 0; b < kBatch; ++b) {
                const int64_t s = base + b * kWave + lane;
                eb[b] = (s < s1) ? idx[s] : -1;
            }
#pragma unroll
            for (int b = 0; b < kBatch; ++b) {
                const int64_t s = base + b * kWave + lane;
                const bool in_tile = s < s1;
                // an id outside [0, E) breaks the precondition: its slot is dropped
                const bool valid = in_tile && static_cast<unsigned>(eb[b]) < static_cast<unsigned>(E);
                const int e = valid ? eb[b] : 0;
                if (in_tile && !valid)
                    pos[s] = -1;
                uint64_t same = __ballot(valid);
                for (int bit = 0; bit < nbits; ++bit) {
                    const bool set = (e >> bit) & 1;
                    const uint64_t bb = __ballot(set);
                    same &= set ? bb : ~bb;
                }
                const int below = __popcll(same & lt);
                const int grp = __popcll(same);
                if (valid) {
                    const int g = c[e] + below;
                    const int p = (g < kept[e]) ? eoff[e] + g : -1;
                    pos[s] = p;
                    if (p >= 0)
                        row_src[p] = static_cast<int32_t>(s);
                    if (below == grp - 1)
                        c[e] += grp;
                }
            }
        }
    }

    // rows [N, S) hold no slot; each block clears those inside its range
    int64_t r0 = static_cast<int64_t>(blockIdx.x) * kWavesPerBlock * tile_slots;
    const int64_t r1 = min(S, r0 + static_cast<int64_t>(kWavesPerBlock) * tile_slots);
    if (r0 < N)
        r0 = N;
    for (int64_t p = r0 + tid; p < r1; p += kBlock)
        row_src[p] = -1;
}

int ceil_log2(int v)
{
    int b = 0;
    while ((1 << b) < v)
        ++b;
    return b;
}

}  // namespace

LayoutTiling layout_tiling(int64_t slots, int E)
{
    // at most ~64K histogram entries (every rank block folds all of them),
    // between 16 and 256 tiles, tiles a multiple of 64 slots and >= 1024
    int64_t max_tiles = 65536 / (E > 0 ? E : 1);
    if (max_tiles < 16)
        max_tiles = 16;
    if (max_tiles > 256)
        max_tiles = 256;
    int64_t ts = (slots + max_tiles - 1) / max_tiles;
    ts = ((ts + kWave - 1) / kWave) * kWave;
    if (ts < 1024)
        ts = 1024;
    LayoutTiling t;
    t.tile_slots = static_cast<int>(ts);
    t.ntiles = static_cast<int>((slots + ts - 1) / ts);
    return t;
}

size_t layout_workspace_bytes(int64_t slots, int E)
{
    const LayoutTiling t = layout_tiling(slots, E);
    size_t b = static_cast<size_t>(E) * static_cast<size_t>(t.ntiles) * sizeof(int32_t);
    b = (b + 255) & ~static_cast<size_t>(255);
    return b < 256 ? 256 : b;
}

hipError_t launch_dispatch_layout(const int32_t *idx, int64_t T, int E, int k, int R,
                                  int capacity, int32_t *expert_counts, int32_t *expert_offsets,
                                  int32_t *rank_counts, int32_t *rank_offsets, int32_t *pos,
                                  int32_t *row_src, void *workspace, hipStream_t stream)
{
    const int64_t S = T * k;
    const LayoutTiling tl = layout_tiling(S, E);
    int32_t *hist = static_cast<int32_t *>(workspace);
    const int nblk = (tl.ntiles + kWavesPerBlock - 1) / kWavesPerBlock;
    if (nblk > 0) {
        layout_hist_kernel<<<nblk, kBlock, kWavesPerBlock * E * sizeof(int32_t), stream>>>(
            idx, S, E, tl.tile_slots, tl.ntiles, hist);
    }
    const size_t lds = ((kWavesPerBlock + 4) * E + 1 + kWavesPerBlock) * sizeof(int32_t);
    layout_rank_kernel<<<nblk > 0 ? nblk : 1, kBlock, lds, stream>>>(
        idx, S, E, R, capacity, tl.tile_slots, tl.ntiles, ceil_log2(E), hist, expert_counts,
        expert_offsets, rank_counts, rank_offsets, pos, row_src);
    return hipGetLastError();
}

}  // namespace moe
