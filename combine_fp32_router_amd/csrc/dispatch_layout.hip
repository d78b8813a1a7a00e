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
// slots are cut into tiles; a tile is one block of NW wavefronts and each
// wave owns a contiguous run of `rounds` x 64 slots of it (one round for
// every chunk size used here), so a tile is ranked in parallel, not by one
// wave walking it serially.
//   1. hist: LDS histogram of the tile, written as row `tile` of
//      hist[ntiles][E].  (When the router runs fused with this pass, it
//      writes finer rows itself, one per group of tokens it routes, and a
//      tile covers `rows_per_tile` of them; the rank kernel folds either.)
//   2. rank: (a) each wave finds, for every 64-slot round, the lanes holding
//      the same expert with ceil(log2 E) ballots: a lane's rank among them
//      and the group size; group leaders add the size to the wave's LDS
//      count row.  (b) The block folds the histogram matrix (coalesced, a
//      few L2 round trips): per-expert totals and counts in earlier tiles.
//      (c) Kept counts and exclusive expert offsets (block scan of <= 1024
//      values); block 0 writes the counts and offsets.  (d) Per expert, a
//      prefix over the waves turns the count rows into each wave's base.
//      (e) Each lane's row is offset[e] + base[w][e] + earlier lanes; the
//      group's last lane advances base[w][e] between rounds.  This is the
//      sequential token-order definition, evaluated a block at a time.
#include "common.hpp"
#include "launch.hpp"

namespace moe {
namespace {

constexpr int kKeep = 4;   // rounds per wave whose match results stay in registers
constexpr int kFold = 16;  // histogram loads a thread issues before adding
constexpr int kFoldV = 8;  // the same with 16-byte loads
constexpr int kMaxWaves = 16;  // waves of a layout block (layout_waves)

// Lanes of the wave holding the same (valid) expert id as this lane.
__device__ __forceinline__ uint64_t match_lanes(bool valid, int e, int nbits)
{
    uint64_t same = __ballot(valid);
    for (int bit = 0; bit < nbits; ++bit) {
        const bool set = (e >> bit) & 1;
        const uint64_t bb = __ballot(set);
        same &= set ? bb : ~bb;
    }
    return same;
}

// Grid: (tiles per chunk, chunks).  Chunk c holds slots
// [c * chunk_slots, min(S_total, (c+1) * chunk_slots)) and its own hist rows.
__global__ __launch_bounds__(1024) void layout_hist_kernel(const int32_t *__restrict__ idx,
                                                           int64_t S_total, int64_t chunk_slots,
                                                           int E, int rounds, int ntiles,
                                                           int32_t *__restrict__ hist)
{
    extern __shared__ int32_t h[];  // [E]
    const int64_t cs0 = static_cast<int64_t>(blockIdx.y) * chunk_slots;
    const int64_t S = min(chunk_slots, S_total - cs0);
    idx += cs0;
    hist += static_cast<int64_t>(blockIdx.y) * ntiles * E;
    const int nw = blockDim.x / kWave;
    const int w = threadIdx.x / kWave;
    const int lane = lane_id();
    for (int e = threadIdx.x; e < E; e += blockDim.x)
        h[e] = 0;
    __syncthreads();
    const int tile = blockIdx.x;
    const int64_t tile_slots = static_cast<int64_t>(nw) * kWave * rounds;
    const int64_t s0 = tile * tile_slots + static_cast<int64_t>(w) * kWave * rounds;
    const int64_t s1 = min(S, s0 + static_cast<int64_t>(kWave) * rounds);
    for (int64_t base = s0; base < s1; base += kWave * kKeep) {
        int e[kKeep];
#pragma unroll
        for (int b = 0; b < kKeep; ++b) {
            const int64_t s = base + b * kWave + lane;
            e[b] = (s < s1) ? idx[s] : -1;
        }
#pragma unroll
        for (int b = 0; b < kKeep; ++b)
            if (static_cast<unsigned>(e[b]) < static_cast<unsigned>(E))  // ids outside [0,E) are not counted
                atomicAdd(&h[e[b]], 1);
    }
    __syncthreads();
    for (int e = threadIdx.x; e < E; e += blockDim.x)
        hist[static_cast<int64_t>(tile) * E + e] = h[e];
}

__global__ __launch_bounds__(1024) void layout_rank_kernel(
    const int32_t *__restrict__ idx, int64_t S_total, int64_t chunk_slots, int E, int R,
    const int32_t *__restrict__ cap_chunk, int cap_all, int rounds, int hrows, int rows_per_tile,
    int nbits,
    const int32_t *__restrict__ hist, int32_t *__restrict__ expert_counts,
    int32_t *__restrict__ expert_offsets, int32_t *__restrict__ rank_counts,
    int32_t *__restrict__ rank_offsets, int32_t *__restrict__ pos, int32_t *__restrict__ row_src)
{
    extern __shared__ int32_t lds[];
    const int chunk = blockIdx.y;
    const int64_t cs0 = static_cast<int64_t>(chunk) * chunk_slots;
    const int64_t S = min(chunk_slots, S_total - cs0);
    const int cap = cap_chunk ? cap_chunk[chunk] : cap_all;
    idx += cs0;
    pos += cs0;
    row_src += cs0;
    hist += static_cast<int64_t>(chunk) * hrows * E;
    expert_counts += static_cast<int64_t>(chunk) * E;
    expert_offsets += static_cast<int64_t>(chunk) * (E + 1);
    rank_counts += static_cast<int64_t>(chunk) * R;
    rank_offsets += static_cast<int64_t>(chunk) * (R + 1);
    const int nthr = blockDim.x;
    const int nw = nthr / kWave;
    int32_t *wcnt = lds;                // [nw][E] per-wave counts, then per-wave bases
    int32_t *before = wcnt + nw * E;    // [E] count in earlier tiles
    int32_t *total = before + E;        // [E]
    int32_t *kept = total + E;          // [E]
    int32_t *eoff = kept + E;           // [E+1]
    int32_t *wsum = eoff + E + 1;       // [nw]
    const int tid = threadIdx.x;
    const int w = tid / kWave;
    const int lane = lane_id();
    const int tile = blockIdx.x;

    for (int i = tid; i < (nw + 2) * E; i += nthr)
        lds[i] = 0;
    __syncthreads();

    // (a) this wave's slots: ids, match groups, per-wave counts
    const int64_t tile_slots = static_cast<int64_t>(nw) * kWave * rounds;
    const int64_t s0 = tile * tile_slots + static_cast<int64_t>(w) * kWave * rounds;
    const int64_t s1 = min(S, s0 + static_cast<int64_t>(kWave) * rounds);
    const uint64_t lt = (1ull << lane) - 1ull;
    int keep_e[kKeep], keep_below[kKeep], keep_grp[kKeep];
    auto match_round = [&](int64_t base, int &e_out, int &below, int &grp) {
        const int64_t s = base + lane;
        const bool in_tile = s < s1;
        const int e_raw = in_tile ? idx[s] : -1;
        // an id outside [0, E) breaks the precondition: its slot is dropped
        const bool valid = in_tile && static_cast<unsigned>(e_raw) < static_cast<unsigned>(E);
        const int e = valid ? e_raw : 0;
        const uint64_t same = match_lanes(valid, e, nbits);
        below = __popcll(same & lt);
        grp = __popcll(same);
        e_out = valid ? e : -1;
    };
#pragma unroll
    for (int r = 0; r < kKeep; ++r) {  // first rounds: results kept in registers
        keep_e[r] = -1;
        keep_below[r] = keep_grp[r] = 0;
        const int64_t base = s0 + static_cast<int64_t>(r) * kWave;
        if (base < s1) {
            match_round(base, keep_e[r], keep_below[r], keep_grp[r]);
            if (keep_e[r] >= 0 && keep_below[r] == keep_grp[r] - 1)
                wcnt[w * E + keep_e[r]] += keep_grp[r];
        }
    }
    for (int64_t base = s0 + kKeep * kWave; base < s1; base += kWave) {  // long tiles
        int e, below, grp;
        match_round(base, e, below, grp);
        if (e >= 0 && below == grp - 1)
            wcnt[w * E + e] += grp;
    }

    // (b) fold the histogram matrix into per-expert totals and counts in rows
    // before this tile's first row ("earlier").  With E % 4 == 0, a thread
    // takes four adjacent columns and every rp-th row, reading 16 bytes per
    // row through a buffer descriptor (rows past the matrix read zero), with
    // kFoldV loads in flight; rp = rows / kFoldV, so a handful of waves fold
    // and the rest wait at the barrier.  Otherwise column e is summed by g
    // threads with 4-byte loads.
    const int first_row = tile * rows_per_tile;
    if ((E & 3) == 0 && E / 4 <= nthr) {
        const int V = E / 4;  // column groups
        int rp = (hrows + kFoldV - 1) / kFoldV;
        if (rp > nthr / V)
            rp = nthr / V;
        const int cv = tid % V;
        const int r0 = tid / V;
        if (r0 < rp) {
            const __amdgpu_buffer_rsrc_t hr = row_rsrc(const_cast<int32_t *>(hist),
                                                       static_cast<int>(hrows * E * 4));
            u32x4 tot = {0, 0, 0, 0}, bef = {0, 0, 0, 0};
            for (int t0 = r0; t0 < hrows; t0 += rp * kFoldV) {
                u32x4 v[kFoldV];
#pragma unroll
                for (int b = 0; b < kFoldV; ++b)
                    v[b] = __builtin_amdgcn_raw_buffer_load_b128(
                        hr, ((t0 + b * rp) * E + 4 * cv) * 4, 0, 0);
#pragma unroll
                for (int b = 0; b < kFoldV; ++b) {
                    tot += v[b];
                    if (t0 + b * rp < first_row)
                        bef += v[b];
                }
            }
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                if (rp == 1) {
                    total[4 * cv + j] = static_cast<int>(tot[j]);
                    before[4 * cv + j] = static_cast<int>(bef[j]);
                } else {
                    atomicAdd(&total[4 * cv + j], static_cast<int>(tot[j]));
                    atomicAdd(&before[4 * cv + j], static_cast<int>(bef[j]));
                }
            }
        }
    } else {
        const int g = (E >= nthr) ? 1 : nthr / E;
        const int sub = tid / E;
        for (int e = tid % E; sub < g && e < E; e += (g == 1 ? nthr : E)) {
            int tot = 0, bef = 0;
            for (int t0 = sub; t0 < hrows; t0 += g * kFold) {
                int v[kFold];
#pragma unroll
                for (int b = 0; b < kFold; ++b) {
                    const int t = t0 + b * g;
                    v[b] = (t < hrows) ? hist[static_cast<int64_t>(t) * E + e] : 0;
                }
#pragma unroll
                for (int b = 0; b < kFold; ++b) {
                    tot += v[b];
                    bef += (t0 + b * g < first_row) ? v[b] : 0;
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

    // (c) kept counts and their exclusive scan over experts
    for (int e = tid; e < E; e += nthr) {
        const int c = total[e];
        kept[e] = (cap > 0 && c > cap) ? cap : c;
        if (tile == 0)
            expert_counts[e] = c;
    }
    __syncthreads();
    const int per = (E + nthr - 1) / nthr;
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
    if (tid == nthr - 1)
        eoff[E] = run;  // threads past E add nothing: the last one holds N
    // (d) per-wave bases: earlier tiles + earlier waves of this tile (all of
    // an expert's counts read before the first write, so the reads overlap)
    for (int e = tid; e < E; e += nthr) {
        int v[kMaxWaves];
#pragma unroll
        for (int q = 0; q < kMaxWaves; ++q)
            v[q] = (q < nw) ? wcnt[q * E + e] : 0;
        int b = before[e];
#pragma unroll
        for (int q = 0; q < kMaxWaves; ++q) {
            if (q < nw)
                wcnt[q * E + e] = b;
            b += v[q];
        }
    }
    __syncthreads();
    const int N = eoff[E];

    if (tile == 0) {
        const int per_rank = E / R;
        for (int e = tid; e <= E; e += nthr)
            expert_offsets[e] = eoff[e];
        for (int r = tid; r < R; r += nthr) {
            rank_offsets[r] = eoff[r * per_rank];
            rank_counts[r] = eoff[(r + 1) * per_rank] - eoff[r * per_rank];
        }
        if (tid == 0)
            rank_offsets[R] = N;
    }

    // (e) rows, round by round in slot order
    int32_t *cb = wcnt + w * E;
    auto place = [&](int64_t s, int e, int below, int grp) {
        if (s >= s1)
            return;
        if (e < 0) {
            pos[s] = -1;
            return;
        }
        const int g = cb[e] + below;
        const int p = (g < kept[e]) ? eoff[e] + g : -1;
        pos[s] = p;
        if (p >= 0)
            row_src[p] = static_cast<int32_t>(s);
        if (below == grp - 1)
            cb[e] += grp;
    };
#pragma unroll
    for (int r = 0; r < kKeep; ++r)
        place(s0 + static_cast<int64_t>(r) * kWave + lane, keep_e[r], keep_below[r], keep_grp[r]);
    for (int64_t base = s0 + kKeep * kWave; base < s1; base += kWave) {
        int e, below, grp;
        match_round(base, e, below, grp);
        place(base + lane, e, below, grp);
    }

    // rows [N, S) hold no slot; each block clears those inside its range
    int64_t r0 = tile * tile_slots;
    const int64_t r1 = min(S, r0 + tile_slots);
    if (r0 < N)
        r0 = N;
    for (int64_t p = r0 + tid; p < r1; p += nthr)
        row_src[p] = -1;
}

int ceil_log2(int v)
{
    int b = 0;
    while ((1 << b) < v)
        ++b;
    return b;
}

int layout_waves(int E) { return E <= 512 ? 16 : 8; }

}  // namespace

LayoutTiling layout_tiling(int64_t slots, int E)
{
    // tiles of waves x 64 x rounds slots; at most ~64K histogram entries (each
    // rank block folds all of them) and at most 256 tiles
    int64_t max_tiles = 65536 / (E > 0 ? E : 1);
    if (max_tiles < 16)
        max_tiles = 16;
    if (max_tiles > 256)
        max_tiles = 256;
    const int64_t round_slots = static_cast<int64_t>(layout_waves(E)) * kWave;
    int64_t rounds = (slots + round_slots * max_tiles - 1) / (round_slots * max_tiles);
    if (rounds < 1)
        rounds = 1;
    LayoutTiling t;
    t.tile_slots = static_cast<int>(round_slots * rounds);
    t.ntiles = static_cast<int>((slots + t.tile_slots - 1) / t.tile_slots);
    return t;
}

int layout_chunks(int64_t T, int64_t chunk_tokens)
{
    if (T <= 0 || chunk_tokens <= 0)
        return 1;
    return static_cast<int>((T + chunk_tokens - 1) / chunk_tokens);
}

size_t layout_workspace_bytes(int64_t T, int64_t chunk_tokens, int E, int k)
{
    const LayoutTiling t = layout_tiling(chunk_tokens * k, E);
    size_t b = static_cast<size_t>(E) * static_cast<size_t>(t.ntiles) *
               static_cast<size_t>(layout_chunks(T, chunk_tokens)) * sizeof(int32_t);
    b = (b + 255) & ~static_cast<size_t>(255);
    return b < 256 ? 256 : b;
}

hipError_t launch_dispatch_layout(const int32_t *idx, int64_t T, int64_t chunk_tokens, int E,
                                  int k, int R, const int32_t *cap_chunk, int cap_all,
                                  int32_t *expert_counts, int32_t *expert_offsets,
                                  int32_t *rank_counts, int32_t *rank_offsets, int32_t *pos,
                                  int32_t *row_src, void *workspace, hipStream_t stream)
{
    const int64_t S = T * k;
    const int64_t chunk_slots = chunk_tokens * k;
    const int chunks = layout_chunks(T, chunk_tokens);
    const LayoutTiling tl = layout_tiling(chunk_slots, E);
    const int nw = layout_waves(E);
    const int rounds = tl.tile_slots / (nw * kWave);
    const int threads = nw * kWave;
    int32_t *hist = static_cast<int32_t *>(workspace);
    if (tl.ntiles > 0 && S > 0) {
        layout_hist_kernel<<<dim3(tl.ntiles, chunks), threads, E * sizeof(int32_t), stream>>>(
            idx, S, chunk_slots, E, rounds, tl.ntiles, hist);
    }
    const size_t lds = (static_cast<size_t>(nw + 4) * E + 1 + nw) * sizeof(int32_t);
    layout_rank_kernel<<<dim3(tl.ntiles > 0 ? tl.ntiles : 1, chunks), threads, lds, stream>>>(
        idx, S, chunk_slots, E, R, cap_chunk, cap_all, rounds, tl.ntiles, 1, ceil_log2(E), hist,
        expert_counts, expert_offsets, rank_counts, rank_offsets, pos, row_src);
    return hipGetLastError();
}

// Fused routing is used when a layout tile holds whole router groups and the
// finer histogram (one row per group) stays within the fold budget the
// tiling itself keeps (~64K entries, which every rank block reads); past it
// the extra folding costs more than the counting pass it saves.  The group
// size depends on the call's token count T (route_group_tokens).
static bool route_layout_fusable(int64_t T, int64_t chunk_tokens, int E, int k)
{
    if (chunk_tokens <= 0)
        return false;
    const LayoutTiling tl = layout_tiling(chunk_tokens * k, E);
    const int G = route_group_tokens(E, T);
    const int64_t group_slots = static_cast<int64_t>(G) * k;
    const int64_t hrows = (chunk_tokens + G - 1) / G;
    return tl.tile_slots % group_slots == 0 && hrows * E <= 65536;
}

size_t route_layout_workspace_bytes(int64_t T, int64_t chunk_tokens, int E, int k)
{
    if (!route_layout_fusable(T, chunk_tokens, E, k))
        return layout_workspace_bytes(T, chunk_tokens, E, k);
    const int G = route_group_tokens(E, T);
    const int64_t hrows = (chunk_tokens + G - 1) / G;
    size_t b = static_cast<size_t>(E) * static_cast<size_t>(hrows) *
               static_cast<size_t>(layout_chunks(T, chunk_tokens)) * sizeof(int32_t);
    return (b + 255) / 256 * 256;
}

hipError_t launch_route_layout(const float *logits, int64_t T, int64_t chunk_tokens, int E,
                               int k, int R, const int32_t *cap_chunk, int cap_all,
                               int32_t *idx, float *w, int32_t *expert_counts,
                               int32_t *expert_offsets, int32_t *rank_counts,
                               int32_t *rank_offsets, int32_t *pos, int32_t *row_src,
                               void *workspace, hipStream_t stream)
{
    if (T <= 0 || !route_layout_fusable(T, chunk_tokens, E, k)) {
        if (T > 0) {
            const hipError_t e = launch_route_topk(logits, T, E, k, idx, w, stream);
            if (e != hipSuccess)
                return e;
        }
        return launch_dispatch_layout(idx, T, chunk_tokens, E, k, R, cap_chunk, cap_all,
                                      expert_counts, expert_offsets, rank_counts, rank_offsets,
                                      pos, row_src, workspace, stream);
    }
    const int64_t S = T * k;
    const int64_t chunk_slots = chunk_tokens * k;
    const int chunks = layout_chunks(T, chunk_tokens);
    const LayoutTiling tl = layout_tiling(chunk_slots, E);
    const int G = route_group_tokens(E, T);
    const int hrows = static_cast<int>((chunk_tokens + G - 1) / G);
    const int rows_per_tile = static_cast<int>(tl.tile_slots / (static_cast<int64_t>(G) * k));
    const int nw = layout_waves(E);
    const int rounds = tl.tile_slots / (nw * kWave);
    int32_t *hist = static_cast<int32_t *>(workspace);
    hipError_t e = launch_route_hist(logits, T, chunk_tokens, chunks, E, k, hrows, idx, w, hist,
                                     stream);
    if (e != hipSuccess)
        return e;
    const size_t lds = (static_cast<size_t>(nw + 4) * E + 1 + nw) * sizeof(int32_t);
    layout_rank_kernel<<<dim3(tl.ntiles, chunks), nw * kWave, lds, stream>>>(
        idx, S, chunk_slots, E, R, cap_chunk, cap_all, rounds, hrows, rows_per_tile,
        ceil_log2(E), hist, expert_counts, expert_offsets, rank_counts, rank_offsets, pos,
        row_src);
    return hipGetLastError();
}

}  // namespace moe
