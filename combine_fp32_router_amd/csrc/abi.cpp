// C ABI of the dispatch/combine library: host-side validation of every
// argument, then the kernel launchers.  Nothing is launched and no output is
// touched when validation fails; no call aborts, exits or throws.
#include <hip/hip_runtime_api.h>

#include <stdint.h>

#include "../../include/moe_recv.h"
#include "../../include/moe_route.h"
#include "checks.hpp"
#include "launch.hpp"

using namespace moe;

namespace {

// A byte range [p, p + bytes); a null pointer is an empty range.
struct Extent {
    const void *p;
    int64_t bytes;
};

bool overlap(const Extent &a, const Extent &b)
{
    if (!a.p || !b.p || a.bytes <= 0 || b.bytes <= 0)
        return false;
    const uintptr_t a0 = reinterpret_cast<uintptr_t>(a.p), b0 = reinterpret_cast<uintptr_t>(b.p);
    return a0 < b0 + static_cast<uintptr_t>(b.bytes) && b0 < a0 + static_cast<uintptr_t>(a.bytes);
}

}  // namespace

extern "C" {

int64_t moe_row_bytes(int H, int quant)
{
    if (quant == MOE_QUANT_BF16)
        return 2 * static_cast<int64_t>(H);
    if (quant == MOE_QUANT_INT8 || quant == MOE_QUANT_FP8)
        return static_cast<int64_t>(H);
    if (quant == MOE_QUANT_INT4)
        return static_cast<int64_t>(H) / 2;
    return -1;
}

const char *moe_status_string(int status)
{
    switch (status) {
    case MOE_OK: return "MOE_OK";
    case MOE_ERR_NULL: return "MOE_ERR_NULL: a required pointer is NULL";
    case MOE_ERR_SHAPE: return "MOE_ERR_SHAPE: a size argument is out of range";
    case MOE_ERR_ALIGN: return "MOE_ERR_ALIGN: a buffer is not aligned as required";
    case MOE_ERR_WORKSPACE: return "MOE_ERR_WORKSPACE: workspace missing or too small";
    case MOE_ERR_HIP: return "MOE_ERR_HIP: the HIP runtime rejected a launch";
    case MOE_ERR_ALIAS: return "MOE_ERR_ALIAS: an output is the same buffer as an input";
    case MOE_ERR_SCRATCH:
        return "MOE_ERR_SCRATCH: the call needs more than the static scratch buffer holds";
    default: return "unknown moe status";
    }
}

int moe_route_topk(const float *logits, int64_t T, int E, int k, int32_t *topk_idx,
                   float *topk_w, hipStream_t stream)
{
    if (T < 0 || check_ek(E, k) != MOE_OK || too_many_slots(T, k) ||
        !grid_fits(route_topk_blocks(T, E), kRouteThreads))
        return MOE_ERR_SHAPE;
    if (T == 0)
        return MOE_OK;
    if (!logits || !topk_idx || !topk_w)
        return MOE_ERR_NULL;
    if (!aligned(logits, 4) || !aligned(topk_idx, 4) || !aligned(topk_w, 4))
        return MOE_ERR_ALIGN;
    return hip_status(moe::launch_route_topk(logits, T, E, k, topk_idx, topk_w, stream));
}

int moe_dispatch_layout(const int32_t *topk_idx, int64_t T, int E, int k, int R, int capacity,
                        int32_t *expert_counts, int32_t *expert_offsets, int32_t *rank_counts,
                        int32_t *rank_offsets, int32_t *pos, int32_t *row_src, void *workspace,
                        size_t *workspace_bytes, hipStream_t stream)
{
    // one chunk of T tokens
    return moe_dispatch_layout_chunks(topk_idx, T, T, E, k, R, capacity, nullptr, expert_counts,
                                      expert_offsets, rank_counts, rank_offsets, pos, row_src,
                                      workspace, workspace_bytes, stream);
}

int moe_dispatch_layout_chunks(const int32_t *topk_idx, int64_t T, int64_t chunk_tokens, int E,
                               int k, int R, int capacity, const int32_t *chunk_capacity,
                               int32_t *expert_counts, int32_t *expert_offsets,
                               int32_t *rank_counts, int32_t *rank_offsets, int32_t *pos,
                               int32_t *row_src, void *workspace, size_t *workspace_bytes,
                               hipStream_t stream)
{
    if (!workspace_bytes)
        return MOE_ERR_NULL;
    if (T < 0 || check_ek(E, k) != MOE_OK || R < 1 || (E % R) != 0 || too_many_slots(T, k) ||
        chunk_tokens < 0 || (T > 0 && chunk_tokens < 1))
        return MOE_ERR_SHAPE;
    if (chunk_tokens > T)
        chunk_tokens = T;  // one chunk
    if (moe::layout_chunks(T, chunk_tokens) > 65535)  // grid y dimension
        return MOE_ERR_SHAPE;
    const size_t need = moe::layout_workspace_bytes(T, chunk_tokens, E, k);
    if (!workspace) {
        *workspace_bytes = need;
        return MOE_OK;
    }
    if (*workspace_bytes < need)
        return MOE_ERR_WORKSPACE;
    if (!expert_counts || !expert_offsets || !rank_counts || !rank_offsets)
        return MOE_ERR_NULL;
    if (T > 0 && (!topk_idx || !pos || !row_src))
        return MOE_ERR_NULL;
    if (!aligned(expert_counts, 4) || !aligned(expert_offsets, 4) || !aligned(rank_counts, 4) ||
        !aligned(rank_offsets, 4) || !aligned(topk_idx, 4) || !aligned(pos, 4) ||
        !aligned(row_src, 4) || !aligned(chunk_capacity, 4) || !aligned(workspace, 256))
        return MOE_ERR_ALIGN;
    return hip_status(moe::launch_dispatch_layout(topk_idx, T, chunk_tokens, E, k, R,
                                                  chunk_capacity, capacity, expert_counts,
                                                  expert_offsets, rank_counts, rank_offsets, pos,
                                                  row_src, workspace, stream));
}

}  // extern "C"

namespace {

// Sizes of the fused route + layout.  On MOE_OK, chunk_tokens is clamped to
// T (one chunk) and `need` holds the histogram scratch the call takes.
int route_layout_sizes(int64_t T, int64_t &chunk_tokens, int E, int k, int R, size_t &need)
{
    // (the router's grid is checked as for moe_route_topk: a call the fused
    // kernel cannot take runs it over the whole batch)
    if (T < 0 || check_ek(E, k) != MOE_OK || R < 1 || (E % R) != 0 || too_many_slots(T, k) ||
        chunk_tokens < 0 || (T > 0 && chunk_tokens < 1) ||
        !grid_fits(route_topk_blocks(T, E), kRouteThreads))
        return MOE_ERR_SHAPE;
    if (chunk_tokens > T)
        chunk_tokens = T;  // one chunk
    if (moe::layout_chunks(T, chunk_tokens) > 65535)  // grid y dimension
        return MOE_ERR_SHAPE;
    need = moe::route_layout_workspace_bytes(T, chunk_tokens, E, k);
    return MOE_OK;
}

// Array arguments of the fused route + layout.
int route_layout_pointers(int64_t T, const float *logits, const int32_t *chunk_capacity,
                          const int32_t *topk_idx, const float *topk_w,
                          const int32_t *expert_counts, const int32_t *expert_offsets,
                          const int32_t *rank_counts, const int32_t *rank_offsets,
                          const int32_t *pos, const int32_t *row_src)
{
    if (!expert_counts || !expert_offsets || !rank_counts || !rank_offsets)
        return MOE_ERR_NULL;
    if (T > 0 && (!logits || !topk_idx || !topk_w || !pos || !row_src))
        return MOE_ERR_NULL;
    if (!aligned(logits, 4) || !aligned(topk_idx, 4) || !aligned(topk_w, 4) ||
        !aligned(expert_counts, 4) || !aligned(expert_offsets, 4) || !aligned(rank_counts, 4) ||
        !aligned(rank_offsets, 4) || !aligned(pos, 4) || !aligned(row_src, 4) ||
        !aligned(chunk_capacity, 4))
        return MOE_ERR_ALIGN;
    return MOE_OK;
}

}  // namespace

extern "C" {

int moe_route_layout_chunks(const float *logits, int64_t T, int64_t chunk_tokens, int E, int k,
                            int R, int capacity, const int32_t *chunk_capacity, int32_t *topk_idx,
                            float *topk_w, int32_t *expert_counts, int32_t *expert_offsets,
                            int32_t *rank_counts, int32_t *rank_offsets, int32_t *pos,
                            int32_t *row_src, void *workspace, size_t *workspace_bytes,
                            hipStream_t stream)
{
    if (!workspace_bytes)
        return MOE_ERR_NULL;
    size_t need = 0;
    int s = route_layout_sizes(T, chunk_tokens, E, k, R, need);
    if (s != MOE_OK)
        return s;
    if (!workspace) {
        *workspace_bytes = need;
        return MOE_OK;
    }
    if (*workspace_bytes < need)
        return MOE_ERR_WORKSPACE;
    s = route_layout_pointers(T, logits, chunk_capacity, topk_idx, topk_w, expert_counts,
                              expert_offsets, rank_counts, rank_offsets, pos, row_src);
    if (s != MOE_OK)
        return s;
    if (!aligned(workspace, 256))
        return MOE_ERR_ALIGN;
    return hip_status(moe::launch_route_layout(logits, T, chunk_tokens, E, k, R, chunk_capacity,
                                               capacity, topk_idx, topk_w, expert_counts,
                                               expert_offsets, rank_counts, rank_offsets, pos,
                                               row_src, workspace, stream));
}

int moe_route_layout_chunks_noalloc(const float *logits, int64_t T, int64_t chunk_tokens, int E,
                                    int k, int R, int capacity, const int32_t *chunk_capacity,
                                    int32_t *topk_idx, float *topk_w, int32_t *expert_counts,
                                    int32_t *expert_offsets, int32_t *rank_counts,
                                    int32_t *rank_offsets, int32_t *pos, int32_t *row_src,
                                    hipStream_t stream)
{
    size_t need = 0;
    int s = route_layout_sizes(T, chunk_tokens, E, k, R, need);
    if (s != MOE_OK)
        return s;
    s = route_layout_pointers(T, logits, chunk_capacity, topk_idx, topk_w, expert_counts,
                              expert_offsets, rank_counts, rank_offsets, pos, row_src);
    if (s != MOE_OK)
        return s;
    if (need > MOE_NOALLOC_SCRATCH_BYTES)
        return MOE_ERR_SCRATCH;
    void *scratch = nullptr;  // the stream's device's copy of the static buffer
    if (moe::static_scratch(stream, &scratch) != hipSuccess)
        return MOE_ERR_HIP;
    return hip_status(moe::launch_route_layout(logits, T, chunk_tokens, E, k, R, chunk_capacity,
                                               capacity, topk_idx, topk_w, expert_counts,
                                               expert_offsets, rank_counts, rank_offsets, pos,
                                               row_src, scratch, stream));
}

int moe_dispatch_pack(const void *x_bf16, int64_t T, int H, int k, const int32_t *pos,
                      int quant_flags, void *send, float *send_scales, hipStream_t stream)
{
    const int quant = quant_flags & ~MOE_PACK_STREAM;
    const bool stream_stores = (quant_flags & MOE_PACK_STREAM) != 0;
    int s = check_rows(T, H, k, quant);
    if (s != MOE_OK)
        return s;
    if (!grid_fits(T, token_threads(H, quant)))
        return MOE_ERR_SHAPE;
    if (T == 0)
        return MOE_OK;
    if (!x_bf16 || !pos || !send)
        return MOE_ERR_NULL;
    if (!aligned(x_bf16, 16) || !aligned(send, 16) || !aligned(pos, 4))
        return MOE_ERR_ALIGN;
    if ((s = check_scales(send_scales, quant)) != MOE_OK)
        return s;
    return hip_status(moe::launch_dispatch_pack(x_bf16, T, H, k, pos, quant, stream_stores, send,
                                                send_scales, stream));
}

int moe_combine(const void *recv, const float *recv_scales, int quant, const int32_t *pos,
                const float *topk_w, int64_t T, int H, int k, void *out_bf16, hipStream_t stream)
{
    int s = check_rows(T, H, k, quant);
    if (s != MOE_OK)
        return s;
    if (!grid_fits(T, token_threads(H, quant)))
        return MOE_ERR_SHAPE;
    if (T == 0)
        return MOE_OK;
    if (!recv || !pos || !topk_w || !out_bf16)
        return MOE_ERR_NULL;
    if (!aligned(recv, 16) || !aligned(out_bf16, 16) || !aligned(pos, 4) || !aligned(topk_w, 4))
        return MOE_ERR_ALIGN;
    if ((s = check_scales(recv_scales, quant)) != MOE_OK)
        return s;
    return hip_status(
        moe::launch_combine(recv, recv_scales, quant, pos, topk_w, T, H, k, out_bf16, stream));
}

int moe_combine_pack(const void *recv, const float *recv_scales, const int32_t *pos_c,
                     const float *topk_w, int64_t Tc, void *out_bf16, const void *x_bf16,
                     const int32_t *pos_p, int64_t Tp, void *send, float *send_scales, int H,
                     int k, int quant_flags, hipStream_t stream)
{
    const int quant = quant_flags & ~MOE_PACK_STREAM;
    const bool stream_stores = (quant_flags & MOE_PACK_STREAM) != 0;
    int s = check_rows(Tc, H, k, quant);
    if (s == MOE_OK)
        s = check_rows(Tp, H, k, quant);
    if (s != MOE_OK)
        return s;
    if (Tc + Tp >= kMaxSlots || !grid_fits(Tc + Tp, token_threads(H, quant)))
        return MOE_ERR_SHAPE;
    if (Tc > 0) {
        if (!recv || !pos_c || !topk_w || !out_bf16)
            return MOE_ERR_NULL;
        if (!aligned(recv, 16) || !aligned(out_bf16, 16) || !aligned(pos_c, 4) ||
            !aligned(topk_w, 4))
            return MOE_ERR_ALIGN;
        if ((s = check_scales(recv_scales, quant)) != MOE_OK)
            return s;
    }
    if (Tp > 0) {
        if (!x_bf16 || !pos_p || !send)
            return MOE_ERR_NULL;
        if (!aligned(x_bf16, 16) || !aligned(send, 16) || !aligned(pos_p, 4))
            return MOE_ERR_ALIGN;
        if ((s = check_scales(send_scales, quant)) != MOE_OK)
            return s;
    }
    if (Tc > 0 && Tp > 0) {
        // The halves run concurrently: what the pack writes must not meet
        // anything the combine touches, nor the combine's output anything the
        // pack reads.  Row buffers are taken at their largest extent (every
        // slot kept: Tc*k and Tp*k rows).
        const int64_t rb = moe_row_bytes(H, quant);
        const bool q = quant != MOE_QUANT_BF16;
        const Extent send_e{send, Tp * k * rb}, sscale_e{q ? send_scales : nullptr, Tp * k * 4};
        const Extent out_e{out_bf16, Tc * H * 2};
        const Extent comb[] = {{recv, Tc * k * rb}, {q ? recv_scales : nullptr, Tc * k * 4},
                               out_e, {pos_c, Tc * k * 4}, {topk_w, Tc * k * 4}};
        for (const Extent &c : comb)
            if (overlap(send_e, c) || overlap(sscale_e, c))
                return MOE_ERR_ALIAS;
        if (overlap(out_e, {x_bf16, Tp * H * 2}) || overlap(out_e, {pos_p, Tp * k * 4}))
            return MOE_ERR_ALIAS;
    }
    return hip_status(moe::launch_combine_pack(recv, recv_scales, pos_c, topk_w, Tc, out_bf16,
                                               x_bf16, pos_p, Tp, send, send_scales, H, k, quant,
                                               stream_stores, stream));
}

int moe_recv_layout(const int32_t *src_offsets, int E, int R, int64_t max_rows,
                    int32_t *recv_offsets, int32_t *group_offsets, int32_t *group_seg,
                    int32_t *group_pos, int32_t *group_src, hipStream_t stream)
{
    if (check_er(E, R) != MOE_OK || max_rows < 0 || max_rows >= kMaxSlots)
        return MOE_ERR_SHAPE;
    if (!src_offsets || !recv_offsets || !group_offsets || !group_seg)
        return MOE_ERR_NULL;
    if (max_rows > 0 && (!group_pos || !group_src))
        return MOE_ERR_NULL;
    if (!aligned(src_offsets, 4) || !aligned(recv_offsets, 4) || !aligned(group_offsets, 4) ||
        !aligned(group_seg, 4) || !aligned(group_pos, 4) || !aligned(group_src, 4))
        return MOE_ERR_ALIGN;
    return hip_status(moe::launch_recv_layout(src_offsets, E, R, max_rows, recv_offsets,
                                              group_offsets, group_seg, group_pos, group_src,
                                              stream));
}

static int gather_rows(const void *in, const float *in_scales, void *out, float *out_scales,
                       int64_t max_rows, int H, int quant, const int32_t *map, hipStream_t stream)
{
    if (max_rows < 0 || max_rows >= kMaxSlots || check_rows(0, H, 1, quant) != MOE_OK ||
        !grid_fits(max_rows, row_tiling(static_cast<int>(moe_row_bytes(H, quant) / 16)).threads))
        return MOE_ERR_SHAPE;
    if (max_rows == 0)
        return MOE_OK;
    if (!in || !out || !map)
        return MOE_ERR_NULL;
    if (!aligned(in, 16) || !aligned(out, 16) || !aligned(map, 4))
        return MOE_ERR_ALIGN;
    int s = check_scales(in_scales, quant);
    if (s == MOE_OK)
        s = check_scales(out_scales, quant);
    if (s != MOE_OK)
        return s;
    return hip_status(
        moe::launch_gather_rows(in, in_scales, out, out_scales, max_rows, H, quant, map, stream));
}

int moe_recv_regroup(const void *recv, const float *recv_scales, int64_t max_rows, int H,
                     int quant, const int32_t *group_src, void *grouped, float *grouped_scales,
                     hipStream_t stream)
{
    return gather_rows(recv, recv_scales, grouped, grouped_scales, max_rows, H, quant, group_src,
                       stream);
}

int moe_recv_ungroup(const void *grouped, const float *grouped_scales, int64_t max_rows, int H,
                     int quant, const int32_t *group_pos, void *recv, float *recv_scales,
                     hipStream_t stream)
{
    return gather_rows(grouped, grouped_scales, recv, recv_scales, max_rows, H, quant, group_pos,
                       stream);
}

}  // extern "C"
