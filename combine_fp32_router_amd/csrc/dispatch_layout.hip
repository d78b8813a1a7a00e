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
// gfx950 design: three small deterministic kernels, no global atomics.
//   1. hist: the slots are cut into tiles of `tile_slots`, one tile per
//      wavefront; each wave counts its tile in a private LDS histogram and
//      writes it column-wise, hist[e][tile].
//   2. scan: one wave per expert turns its column into exclusive tile bases
//      (in place) and writes the expert's total.
//   3. rank: every block recomputes kept counts and the expert offsets from
//      the totals (E <= 1024 values, block scan in LDS), then each wave walks
//      its tile in slot order, 64 slots a step.  Lanes holding the same
//      expert find each other with log2(E) ballots; a lane's row is
//      offset[e] + base[e] + (earlier lanes with e), and the group's last lane
//      advances base[e].  This is exactly the sequential token-order
//      definition, evaluated a wave-step at a time.
#include "common.hpp"
#include "launch.hpp"

namespace moe {
namespace {

constexpr int kBlock = 256;
constexpr int kWavesPerBlock = kBlock / kWave;

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
        for (int64_t s = s0 + lane; s < s1; s += kWave) {
            const int e = idx[s];
            if (static_cast<unsigned>(e) < static_cast<unsigned>(E))  // ids outside [0,E) are not counted
                atomicAdd(&h[e], 1);
        }
    }
    __syncthreads();
    if (tile < ntiles)
        for (int e = lane; e < E; e += kWave)
            hist[static_cast<int64_t>(e) * ntiles + tile] = h[e];
}

__global__ __launch_bounds__(kBlock) void layout_scan_kernel(int32_t *__restrict__ hist, int E,
                                                             int ntiles,
                                                             int32_t *__restrict__ expert_counts)
{
    const int e = blockIdx.x * kWavesPerBlock + uniform(threadIdx.x / kWave);
    if (e >= E)
        return;
    const int lane = lane_id();
    int32_t *col = hist + static_cast<int64_t>(e) * ntiles;
    int carry = 0;
    for (int base = 0; base < ntiles; base += kWave) {
        const int i = base + lane;
        const int v = (i < ntiles) ? col[i] : 0;
        const int incl = wave_inclusive_scan(v);
        if (i < ntiles)
            col[i] = carry + incl - v;
        carry += __shfl(incl, kWave - 1);
    }
    if (lane == 0)
        expert_counts[e] = carry;
}

__global__ __launch_bounds__(kBlock) void layout_rank_kernel(
    const int32_t *__restrict__ idx, int64_t S, int E, int R, int cap, int tile_slots, int ntiles,
    int nbits, const int32_t *__restrict__ tile_base, const int32_t *__restrict__ expert_counts,
    int32_t *__restrict__ expert_offsets, int32_t *__restrict__ rank_counts,
    int32_t *__restrict__ rank_offsets, int32_t *__restrict__ pos, int32_t *__restrict__ row_src)
{
    extern __shared__ int32_t lds[];
    int32_t *cnt = lds;                       // [4][E] running rank per expert, per wave
    int32_t *kept = cnt + kWavesPerBlock * E;  // [E]
    int32_t *eoff = kept + E;                  // [E+1]
    int32_t *wsum = eoff + E + 1;              // [4]
    const int tid = threadIdx.x;
    const int w = tid / kWave;
    const int lane = lane_id();

    // kept counts and their exclusive scan over experts (every block)
    const int per = (E + kBlock - 1) / kBlock;
    const int e0 = tid * per;
    int local = 0;
    for (int i = 0; i < per; ++i) {
        const int e = e0 + i;
        if (e < E) {
            const int c = expert_counts[e];
            const int kk = (cap > 0 && c > cap) ? cap : c;
            kept[e] = kk;
            local += kk;
        }
    }
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

    const int tile = blockIdx.x * kWavesPerBlock + w;
    for (int e = lane; e < E; e += kWave)
        cnt[w * E + e] = (tile < ntiles) ? tile_base[static_cast<int64_t>(e) * ntiles + tile] : 0;
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

    if (tile < ntiles) {
        int32_t *c = cnt + w * E;
        const int64_t s0 = static_cast<int64_t>(tile) * tile_slots;
        const int64_t s1 = min(S, s0 + tile_slots);
        const uint64_t lt = (1ull << lane) - 1ull;
        for (int64_t base = s0; base < s1; base += kWave) {
            const int64_t s = base + lane;
            const bool in_tile = s < s1;
            const int e_raw = in_tile ? idx[s] : 0;
            // an id outside [0, E) breaks the precondition: its slot is dropped
            const bool valid = in_tile && static_cast<unsigned>(e_raw) < static_cast<unsigned>(E);
            const int e = valid ? e_raw : 0;
            if (in_tile && !valid)
                pos[s] = -1;
            uint64_t same = __ballot(valid);
            for (int b = 0; b < nbits; ++b) {
                const bool bit = (e >> b) & 1;
                const uint64_t bb = __ballot(bit);
                same &= bit ? bb : ~bb;
            }
            const int below = __popcll(same & lt);
            const int total = __popcll(same);
            if (valid) {
                const int g = c[e] + below;
                const int p = (g < kept[e]) ? eoff[e] + g : -1;
                pos[s] = p;
                if (p >= 0)
                    row_src[p] = static_cast<int32_t>(s);
                if (below == total - 1)
                    c[e] += total;
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

LayoutTiling layout_tiling(int64_t slots)
{
    // about <= 256 tiles, each a multiple of 64 slots and at least 256
    int64_t ts = (slots + 255) / 256;
    ts = ((ts + kWave - 1) / kWave) * kWave;
    if (ts < 256)
        ts = 256;
    LayoutTiling t;
    t.tile_slots = static_cast<int>(ts);
    t.ntiles = static_cast<int>((slots + ts - 1) / ts);
    return t;
}

size_t layout_workspace_bytes(int64_t slots, int E)
{
    const LayoutTiling t = layout_tiling(slots);
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
    const LayoutTiling tl = layout_tiling(S);
    int32_t *hist = static_cast<int32_t *>(workspace);
    const int nblk = (tl.ntiles + kWavesPerBlock - 1) / kWavesPerBlock;
    if (nblk > 0) {
        layout_hist_kernel<<<nblk, kBlock, kWavesPerBlock * E * sizeof(int32_t), stream>>>(
            idx, S, E, tl.tile_slots, tl.ntiles, hist);
    }
    layout_scan_kernel<<<(E + kWavesPerBlock - 1) / kWavesPerBlock, kBlock, 0, stream>>>(
        hist, E, tl.ntiles, expert_counts);
    const size_t lds = (kWavesPerBlock * E + E + E + 1 + kWavesPerBlock) * sizeof(int32_t);
    layout_rank_kernel<<<nblk > 0 ? nblk : 1, kBlock, lds, stream>>>(
        idx, S, E, R, capacity, tl.tile_slots, tl.ntiles, ceil_log2(E), hist, expert_counts,
        expert_offsets, rank_counts, rank_offsets, pos, row_src);
    return hipGetLastError();
}

}  // namespace moe
