// C ABI of the dispatch/combine library: host-side validation of every
// argument, then the kernel launchers.  Nothing is launched and no output is
// touched when validation fails; no call aborts, exits or throws.
#include <hip/hip_runtime_api.h>

#include <stdint.h>

#include "../../include/moe_harness.h"
#include "../../include/moe_recv.h"
#include "../../include/moe_route.h"
#include "launch.hpp"

namespace {

bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

constexpr int64_t kMaxSlots = int64_t(1) << 31;  // T*k must fit an int32 row index

int check_ek(int E, int k)
{
    if (E < 1 || E > MOE_MAX_EXPERTS || k < 1 || k > E || k > MOE_MAX_TOPK)
        return MOE_ERR_SHAPE;
    return MOE_OK;
}

int check_rows(int64_t T, int H, int k, int quant)
{
    if (T < 0 || k < 1 || k > MOE_MAX_TOPK || H < 16 || H > MOE_MAX_HIDDEN || (H % 16) != 0 ||
        (quant != MOE_QUANT_BF16 && quant != MOE_QUANT_INT8 && quant != MOE_QUANT_INT4 &&
         quant != MOE_QUANT_FP8) ||
        (quant == MOE_QUANT_INT4 && (H % 32) != 0) || T * k >= kMaxSlots)
        return MOE_ERR_SHAPE;
    return MOE_OK;
}

int hip_status(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ERR_HIP; }

int check_er(int E, int R)
{
    if (E < 1 || E > MOE_MAX_EXPERTS || R < 1 || (E % R) != 0)
        return MOE_ERR_SHAPE;
    return MOE_OK;
}

// Scale array of a quantised row buffer: required (4-byte aligned) when
// quant != bf16 and the call moves rows; ignored for bf16.
int check_scales(const void *scales, int quant)
{
    if (quant == MOE_QUANT_BF16)
        return MOE_OK;
    if (!scales)
        return MOE_ERR_NULL;
    if (!aligned(scales, 4))
        return MOE_ERR_ALIGN;
    return MOE_OK;
}

// Arguments of the exchange stand-in.
int check_recv_rows(const void *a, const void *as, const void *b, const void *bs,
                    int64_t max_rows, int H, int quant, const int32_t *src_offsets, int E, int R,
                    const int32_t *recv_offsets)
{
    if (check_er(E, R) != MOE_OK || max_rows < 0 || max_rows >= kMaxSlots ||
        check_rows(0, H, 1, quant) != MOE_OK)
        return MOE_ERR_SHAPE;
    if (max_rows == 0)
        return MOE_OK;
    if (!a || !b || !src_offsets || !recv_offsets)
        return MOE_ERR_NULL;
    if (!aligned(a, 16) || !aligned(b, 16) || !aligned(src_offsets, 4) || !aligned(recv_offsets, 4))
        return MOE_ERR_ALIGN;
    int s = check_scales(as, quant);
    if (s == MOE_OK)
        s = check_scales(bs, quant);
    return s;
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
    default: return "unknown moe status";
    }
}

int moe_route_topk(const float *logits, int64_t T, int E, int k, int32_t *topk_idx,
                   float *topk_w, hipStream_t stream)
{
    if (T < 0 || check_ek(E, k) != MOE_OK || T * k >= kMaxSlots)
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
    if (T < 0 || check_ek(E, k) != MOE_OK || R < 1 || (E % R) != 0 || T * k >= kMaxSlots ||
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

int moe_route_layout_chunks(const float *logits, int64_t T, int64_t chunk_tokens, int E, int k,
                            int R, int capacity, const int32_t *chunk_capacity, int32_t *topk_idx,
                            float *topk_w, int32_t *expert_counts, int32_t *expert_offsets,
                            int32_t *rank_counts, int32_t *rank_offsets, int32_t *pos,
                            int32_t *row_src, void *workspace, size_t *workspace_bytes,
                            hipStream_t stream)
{
    if (!workspace_bytes)
        return MOE_ERR_NULL;
    if (T < 0 || check_ek(E, k) != MOE_OK || R < 1 || (E % R) != 0 || T * k >= kMaxSlots ||
        chunk_tokens < 0 || (T > 0 && chunk_tokens < 1))
        return MOE_ERR_SHAPE;
    if (chunk_tokens > T)
        chunk_tokens = T;  // one chunk
    if (moe::layout_chunks(T, chunk_tokens) > 65535)  // grid y dimension
        return MOE_ERR_SHAPE;
    const size_t need = moe::route_layout_workspace_bytes(T, chunk_tokens, E, k);
    if (!workspace) {
        *workspace_bytes = need;
        return MOE_OK;
    }
    if (*workspace_bytes < need)
        return MOE_ERR_WORKSPACE;
    if (!expert_counts || !expert_offsets || !rank_counts || !rank_offsets)
        return MOE_ERR_NULL;
    if (T > 0 && (!logits || !topk_idx || !topk_w || !pos || !row_src))
        return MOE_ERR_NULL;
    if (!aligned(logits, 4) || !aligned(topk_idx, 4) || !aligned(topk_w, 4) ||
        !aligned(expert_counts, 4) || !aligned(expert_offsets, 4) || !aligned(rank_counts, 4) ||
        !aligned(rank_offsets, 4) || !aligned(pos, 4) || !aligned(row_src, 4) ||
        !aligned(chunk_capacity, 4) || !aligned(workspace, 256))
        return MOE_ERR_ALIGN;
    return hip_status(moe::launch_route_layout(logits, T, chunk_tokens, E, k, R, chunk_capacity,
                                               capacity, topk_idx, topk_w, expert_counts,
                                               expert_offsets, rank_counts, rank_offsets, pos,
                                               row_src, workspace, stream));
}

int moe_dispatch_pack(const void *x_bf16, int64_t T, int H, int k, const int32_t *pos,
                      int quant, void *send, float *send_scales, hipStream_t stream)
{
    int s = check_rows(T, H, k, quant);
    if (s != MOE_OK)
        return s;
    if (T == 0)
        return MOE_OK;
    if (!x_bf16 || !pos || !send)
        return MOE_ERR_NULL;
    if (!aligned(x_bf16, 16) || !aligned(send, 16) || !aligned(pos, 4))
        return MOE_ERR_ALIGN;
    if ((s = check_scales(send_scales, quant)) != MOE_OK)
        return s;
    return hip_status(
        moe::launch_dispatch_pack(x_bf16, T, H, k, pos, quant, send, send_scales, stream));
}

int moe_combine(const void *recv, const float *recv_scales, int quant, const int32_t *pos,
                const float *topk_w, int64_t T, int H, int k, void *out_bf16, hipStream_t stream)
{
    int s = check_rows(T, H, k, quant);
    if (s != MOE_OK)
        return s;
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
                     int k, int quant, hipStream_t stream)
{
    int s = check_rows(Tc, H, k, quant);
    if (s == MOE_OK)
        s = check_rows(Tp, H, k, quant);
    if (s != MOE_OK)
        return s;
    if (Tc + Tp >= kMaxSlots)
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
    if (Tc > 0 && Tp > 0 &&
        (send == recv || (quant != MOE_QUANT_BF16 && send_scales == recv_scales)))
        return MOE_ERR_ALIAS;
    return hip_status(moe::launch_combine_pack(recv, recv_scales, pos_c, topk_w, Tc, out_bf16,
                                               x_bf16, pos_p, Tp, send, send_scales, H, k, quant,
                                               stream));
}

int moe_expert_standin(const void *recv, const float *recv_scales, int quant_in,
                       const int32_t *expert_offsets, int E, int64_t max_rows, int H,
                       int quant_out, void *ret, float *ret_scales, hipStream_t stream)
{
    if (E < 1 || E > MOE_MAX_EXPERTS || max_rows < 0 || max_rows >= kMaxSlots ||
        check_rows(0, H, 1, quant_in) != MOE_OK || check_rows(0, H, 1, quant_out) != MOE_OK)
        return MOE_ERR_SHAPE;
    if (max_rows == 0)
        return MOE_OK;
    if (!recv || !expert_offsets || !ret)
        return MOE_ERR_NULL;
    if (!aligned(recv, 16) || !aligned(ret, 16) || !aligned(expert_offsets, 4))
        return MOE_ERR_ALIGN;
    int s = check_scales(recv_scales, quant_in);
    if (s == MOE_OK)
        s = check_scales(ret_scales, quant_out);
    if (s != MOE_OK)
        return s;
    return hip_status(moe::launch_expert_standin(recv, recv_scales, quant_in, expert_offsets, E,
                                                 max_rows, H, quant_out, ret, ret_scales, stream));
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
    if (max_rows < 0 || max_rows >= kMaxSlots || check_rows(0, H, 1, quant) != MOE_OK)
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

int moe_exchange_blocks(void *send, float *send_scales, int64_t source_rows, void *recv,
                        float *recv_scales, int64_t max_rows, int H, int quant,
                        const int32_t *src_offsets, int E, int R, const int32_t *recv_offsets,
                        int reverse, hipStream_t stream)
{
    if (source_rows < 0 || (R >= 1 && source_rows * R >= kMaxSlots))
        return MOE_ERR_SHAPE;
    const int s = check_recv_rows(send, send_scales, recv, recv_scales, max_rows, H, quant,
                                  src_offsets, E, R, recv_offsets);
    if (s != MOE_OK || max_rows == 0)
        return s;
    return hip_status(moe::launch_exchange_blocks(send, send_scales, source_rows, recv,
                                                  recv_scales, max_rows, H, quant, src_offsets, E,
                                                  R, recv_offsets, reverse != 0, stream));
}

int moe_copy_probe(const void *src, void *dst, size_t bytes, int blocks, hipStream_t stream)
{
    if ((bytes % 16) != 0)
        return MOE_ERR_SHAPE;
    if (bytes == 0)
        return MOE_OK;
    if (!src || !dst)
        return MOE_ERR_NULL;
    if (!aligned(src, 16) || !aligned(dst, 16))
        return MOE_ERR_ALIGN;
    return hip_status(moe::launch_copy_probe(src, dst, bytes, blocks, stream));
}

}  // extern "C"
