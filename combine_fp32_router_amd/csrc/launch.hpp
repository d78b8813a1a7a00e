// Host-side launchers of the gfx950 kernels.  Arguments are validated by the
// C ABI (abi.cpp) before any of these is called; each returns the HIP error
// of its launch(es).
#pragma once

#include <hip/hip_runtime_api.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/moe_route.h"

namespace moe {

hipError_t launch_route_topk(const float *logits, int64_t T, int E, int k,
                             int32_t *idx, float *w, hipStream_t stream);
// Workgroups of kRouteThreads threads that launch_route_topk runs for T tokens.
constexpr int kRouteThreads = 256;
int64_t route_topk_blocks(int64_t T, int E);

// A HIP launch counts the work-items of each grid dimension in 32 bits: a
// dimension of `blocks` workgroups of `threads` work-items must stay below
// 2^32.  The C ABI refuses calls whose grid would not (MOE_ERR_SHAPE).
inline bool grid_fits(int64_t blocks, int threads)
{
    return blocks <= int64_t(0xFFFFFFFF) / threads;
}

// Tiling of the layout: `tile_slots` slots per wave-tile, `ntiles` tiles.
struct LayoutTiling {
    int tile_slots;
    int ntiles;
};
LayoutTiling layout_tiling(int64_t slots, int E);
// Chunks of a batched layout: ceil(T / chunk_tokens) (1 when T == 0).
int layout_chunks(int64_t T, int64_t chunk_tokens);
size_t layout_workspace_bytes(int64_t T, int64_t chunk_tokens, int E, int k);

// Layout of every chunk of chunk_tokens tokens (the last may be shorter) in
// one pair of launches.  Capacity of chunk c: cap_chunk[c] (device array)
// when cap_chunk is not NULL, else cap_all (<= 0: unlimited).
hipError_t launch_dispatch_layout(const int32_t *idx, int64_t T, int64_t chunk_tokens, int E,
                                  int k, int R, const int32_t *cap_chunk, int cap_all,
                                  int32_t *expert_counts, int32_t *expert_offsets,
                                  int32_t *rank_counts, int32_t *rank_offsets, int32_t *pos,
                                  int32_t *row_src, void *workspace, hipStream_t stream);

// Router fused with the layout's histogram pass (two launches; falls back to
// route + layout when a layout tile does not hold whole router groups).
// Tokens per router group (one histogram row) of a fused call over T tokens.
int route_group_tokens(int E, int64_t T);
hipError_t launch_route_hist(const float *logits, int64_t T, int64_t chunk_tokens, int chunks,
                             int E, int k, int hrows, int32_t *idx, float *w, int32_t *hist,
                             hipStream_t stream);
size_t route_layout_workspace_bytes(int64_t T, int64_t chunk_tokens, int E, int k);
hipError_t launch_route_layout(const float *logits, int64_t T, int64_t chunk_tokens, int E,
                               int k, int R, const int32_t *cap_chunk, int cap_all,
                               int32_t *idx, float *w, int32_t *expert_counts,
                               int32_t *expert_offsets, int32_t *rank_counts,
                               int32_t *rank_offsets, int32_t *pos, int32_t *row_src,
                               void *workspace, hipStream_t stream);

// Device address of the static histogram scratch (MOE_NOALLOC_SCRATCH_BYTES)
// on the device of `stream` (the current device for the null stream), looked
// up on the first call on each device.
hipError_t static_scratch(hipStream_t stream, void **ptr);

// Quantised payloads (quant != 0) write / read one fp32 scale per row in
// `scales` (send / recv rows at the same index); bf16 ignores it.
// stream_stores: the send rows are written with streaming device-scope
// stores (not kept in the last-level cache) instead of device-scope stores.
hipError_t launch_dispatch_pack(const void *x, int64_t T, int H, int k,
                                const int32_t *pos, int quant, bool stream_stores, void *send,
                                float *scales, hipStream_t stream);

hipError_t launch_combine(const void *recv, const float *scales, int quant, const int32_t *pos,
                          const float *w, int64_t T, int H, int k, void *out,
                          hipStream_t stream);

// Combine of Tc tokens (blocks first) and pack of Tp tokens in one grid;
// stream_stores applies to the pack half, as for launch_dispatch_pack.
hipError_t launch_combine_pack(const void *recv, const float *rscales, const int32_t *pos_c,
                               const float *w, int64_t Tc, void *out, const void *x,
                               const int32_t *pos_p, int64_t Tp, void *send, float *sscales,
                               int H, int k, int quant, bool stream_stores, hipStream_t stream);

// Receiver side: segment offsets, expert-major starts and the two row maps
// (group_pos: receive row -> grouped row, group_src: the inverse; -1 past N).
hipError_t launch_recv_layout(const int32_t *src_offsets, int E, int R, int64_t max_rows,
                              int32_t *recv_offsets, int32_t *group_offsets, int32_t *group_seg,
                              int32_t *group_pos, int32_t *group_src, hipStream_t stream);

// out[i] = in[map[i]] for i < max_rows, rows of row_bytes(H, quant) bytes
// (and their scales for quant != 0); rows whose map entry is outside
// [0, max_rows) are not written.
hipError_t launch_gather_rows(const void *in, const float *in_scales, void *out, float *out_scales,
                              int64_t max_rows, int H, int quant, const int32_t *map,
                              hipStream_t stream);

// Threads per block and 16-byte vectors per thread covering one row of
// `vecs` 16-byte vectors with one block (<= 1024 threads, a whole number of
// 64-lane waves): one vector per thread up to 1024 vectors, then 2, 4, 8.
struct RowTiling {
    int threads;
    int vpt;
};
// The int8 / fp8 / int4 kernels tile 16-element groups: G = H / 16 <= 4096
// groups, so their vpt is at most 4 and only 1, 2 and 4 are built (the bf16
// kernels tile H / 8 <= 8192 vectors and take up to 8).
static_assert(MOE_MAX_HIDDEN / 16 <= 4 * 1024, "16-element groups: at most four per thread");
inline RowTiling row_tiling(int vecs)
{
    RowTiling r;
    r.vpt = 1;
    while (r.vpt < 8 && (vecs + r.vpt - 1) / r.vpt > 1024)
        r.vpt *= 2;
    int thr = (vecs + r.vpt - 1) / r.vpt;
    thr = ((thr + 63) / 64) * 64;
    r.threads = thr < 64 ? 64 : thr;
    return r;
}

// Threads of the one-workgroup-per-token pack, combine and combine+pack
// kernels: the bf16 kernels tile H / 8 vectors, the others H / 16 groups.
inline int token_threads(int H, int quant)
{
    return row_tiling(quant == MOE_QUANT_BF16 ? H / 8 : H / 16).threads;
}

}  // namespace moe
