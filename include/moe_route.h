/*
 * moe_route.h -- C ABI of the MI355X (gfx950) MoE expert-parallel
 * dispatch/combine data path: the work one GPU does around the all-to-all.
 *
 * Problem statement (ThunderEP write-up on bjdmk.com.cn, s1.3; the
 * "communication wall" explainer on juhe.plus, traffic section): T tokens
 * of hidden size H, E experts in total split into R contiguous blocks of
 * E/R (one per destination rank), each token routed to its top-k experts.
 *
 * One MoE layer, per chunk of Tc tokens (the batch is cut into 1/4..1/8
 * chunks, ThunderEP s2.1/s2.2):
 *
 *   moe_route_topk       logits -> top-k expert ids + renormalised weights
 *   moe_dispatch_layout  ids -> per-expert/per-rank counts and offsets,
 *                        slot->row map `pos`, row->slot map `row_src`
 *   moe_dispatch_pack    hidden rows -> one contiguous send buffer whose
 *                        rank blocks are the aggregated messages (bf16, or
 *                        per-token dynamic int8)
 *   (all-to-all, experts: not part of this library)
 *   moe_combine          returned rows -> gate-weighted sum in token order
 *
 * Batched and fused forms of the same steps: moe_dispatch_layout_chunks
 * (every chunk's layout in one call), moe_route_layout_chunks (the router
 * fused with the layout's counting pass; moe_route_layout_chunks_noalloc
 * for callers that cannot allocate), moe_combine_pack (the combine of one
 * chunk and the pack of the next in one launch).  The receiver side of the
 * exchange is declared in moe_recv.h.
 *
 * Conventions shared by every call
 *   - All array arguments are DEVICE pointers owned by the caller; the
 *     library allocates nothing and keeps no global state, so calls are
 *     thread-safe (the one exception is moe_route_layout_chunks_noalloc,
 *     which uses a static device buffer of the library).  Calls are
 *     asynchronous on `stream` (NULL = the null stream); results are
 *     visible once the stream has reached them.
 *   - Arguments are validated on the host before anything is launched; on
 *     any error nothing is launched and no output is touched.  No call
 *     aborts, exits or throws.
 *   - Layouts are row-major and dense.  bf16 values are passed as their raw
 *     16-bit patterns, int8 codes as bytes, behind `void *`.
 *   - A "slot" is s = t*k + j (token t of the chunk, its j-th expert).
 *     `pos` and `row_src` are relative to the chunk.
 *   - A HIP launch counts the work-items of each grid dimension in 32 bits.
 *     The router runs 256-thread workgroups of 16 tokens (E <= 256) or 4
 *     tokens; pack, combine and the receiver regroup run one workgroup per
 *     token or row, of 64-1024 threads covering its H/8 (bf16) or H/16
 *     (quantised) 16-byte vectors (H = 7168 bf16: 896).  A call whose grid
 *     would reach 2^32 work-items returns MOE_ERR_SHAPE (pack or combine of
 *     more than 4,793,490 tokens at H = 7168 bf16; the router of more than
 *     268,435,440 tokens at E <= 256).
 *   - Preconditions the library does not check on the host: logits are
 *     finite; topk_idx holds k distinct ids in [0, E) per token (as
 *     moe_route_topk writes them); `pos` is a layout written by
 *     moe_dispatch_layout for the same T, E, k; hidden values are finite.
 */
#ifndef MOE_ROUTE_H
#define MOE_ROUTE_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes returned by every call. */
enum moe_status {
    MOE_OK = 0,
    MOE_ERR_NULL = 1,      /* a required pointer is NULL                        */
    MOE_ERR_SHAPE = 2,     /* a size is out of range (see each call)            */
    MOE_ERR_ALIGN = 3,     /* a buffer is not aligned as required               */
    MOE_ERR_WORKSPACE = 4, /* workspace missing or smaller than required        */
    MOE_ERR_HIP = 5,       /* the HIP runtime rejected a launch                 */
    MOE_ERR_ALIAS = 6,     /* an output is the same buffer as an input it must
                              not overwrite                                     */
    MOE_ERR_SCRATCH = 7    /* the call needs more scratch than the library's
                              static buffer holds (MOE_NOALLOC_SCRATCH_BYTES)   */
};

#define MOE_MAX_EXPERTS 1024 /* E <= 1024                                    */
#define MOE_MAX_TOPK 16      /* k <= 16                                      */
#define MOE_MAX_HIDDEN 65536 /* H <= 65536, H % 16 == 0                      */
/* Size of the static device scratch of moe_route_layout_chunks_noalloc: one
 * copy per GPU the library runs on, held until the process ends. */
#define MOE_NOALLOC_SCRATCH_BYTES (4u << 20)

/* Payload formats of a send/return row.  A row buffer holds rows of
 * moe_row_bytes(H, quant) bytes back to back; a quantised row's fp32 scale
 * is kept at the same row index of a separate scale array (one float per
 * row), which travels beside the rows (the exchange moves both, segment for
 * segment).  Rows therefore stay whole 128-byte lines whenever 2H (bf16),
 * H (int8, fp8) or H/2 (int4) is a multiple of 128, and every rank block of
 * a row buffer stays 16-byte aligned.
 *   MOE_QUANT_BF16: H bf16 values, 2*H bytes; no scale.
 *   MOE_QUANT_INT8: per-token dynamic int8 (ThunderEP s2.3): H int8 codes
 *     and the row's scale.  scale = max_h |x_h| / 127 (one fp32 IEEE
 *     division); code_h = x_h / scale (fp32 IEEE division) rounded to
 *     nearest, ties to even, clamped to [-127, 127]; an all-zero row has
 *     scale 0 and zero codes.  Dequantised value: (float)code_h * scale (fp32
 *     multiply).
 *   MOE_QUANT_INT4: per-token dynamic int4, the write-up's 4-bit follow-up
 *     (ThunderEP s5.2): the int8 rule with scale = max_h |x_h| / 7 and codes
 *     clamped to [-7, 7], stored two per byte (element 2i in the low nibble
 *     of byte i, 4-bit two's complement): H/2 bytes and the scale.  Requires
 *     H % 32 == 0 (16-byte aligned rows).
 *   MOE_QUANT_FP8: per-token dynamic fp8 (OCP E4M3: bias 7, no infinities,
 *     largest finite 448), the NCCL EP article's FP8 communication (s6.3):
 *     the int8 rule with scale = max_h |x_h| / 448 and code_h = E4M3(x_h /
 *     scale) rounded to nearest, ties to even; H codes and the scale.
 *     Dequantised value: decode(code_h) * scale. */
#define MOE_QUANT_BF16 0
#define MOE_QUANT_INT8 1
#define MOE_QUANT_INT4 2
#define MOE_QUANT_FP8 3

/* Flag OR-ed into the `quant` argument of moe_dispatch_pack and
 * moe_combine_pack (only those): write the send rows with streaming stores
 * that are not kept in the last-level cache.  Without it the rows are kept
 * there, which pays when their consumer reads them back from this GPU soon
 * (on one device, the combine of the same chunk); with it, nothing dirty is
 * left for later kernels to evict and write back, which pays when the rows
 * leave the GPU or are read only after other traffic.  The rows written are
 * the same either way. */
#define MOE_PACK_STREAM 0x100

/* Bytes per row of a row buffer for hidden size H and payload format
 * `quant` (2*H, H, H/2 or H); -1 for an unknown format.  Quantised formats
 * add 4 bytes per row in the scale array. */
int64_t moe_row_bytes(int H, int quant);

/* Human-readable name of a status code (static string, never NULL). */
const char *moe_status_string(int status);

/*
 * moe_route_topk -- router top-k with renormalised gate weights.
 * Defined by the sparse-communication article (intelliparadigm.com, s2.1:
 * softmax over the router logits, then top-k) and the communication-wall
 * router example (each token to its k best experts); the weights are the
 * top-k probabilities renormalised to sum to one.
 *
 *   logits    [T, E] fp32, row-major, finite.                  (in)
 *   topk_idx  [T, k] int32: the k experts with the largest logits, in
 *             descending logit order; equal logits (including +0 / -0) go
 *             to the lower expert id.                          (out)
 *   topk_w    [T, k] fp32: w_j = exp(l_j - l_max) / sum_i exp(l_i - l_max)
 *             over the k selected logits (the full softmax renormalised
 *             over the selection).  Computed in double, rounded once.  (out)
 *
 * Errors: MOE_ERR_NULL (a pointer NULL with T > 0); MOE_ERR_SHAPE (T < 0,
 * E < 1, E > MOE_MAX_EXPERTS, k < 1, k > E, k > MOE_MAX_TOPK,
 * T*k >= 2^31); MOE_ERR_ALIGN (a pointer not 4-byte aligned).
 * T == 0: MOE_OK, nothing launched.
 */
int moe_route_topk(const float *logits, int64_t T, int E, int k,
                   int32_t *topk_idx, float *topk_w, hipStream_t stream);

/*
 * moe_dispatch_layout -- where every (token, expert) slot goes in the send
 * buffer.  Aggregation by destination (ThunderEP s2.1: the rows for one
 * destination are gathered into one contiguous block, at most R blocks);
 * contiguous expert placement (communication-wall EP example: rank r owns
 * experts r*E/R .. (r+1)*E/R - 1); the flat buffer whose segment r starts at
 * the prefix sum of the earlier counts (NCCL EP article, s3.3); an optional
 * per-expert capacity (sparse-communication article, s2.1, capacity factor).
 * Rows are ordered by (rank, expert, token): within an expert bucket the
 * token order is kept (a stable scatter).  With a capacity, each expert
 * keeps its first `capacity` slots in token order and drops the rest.
 *
 *   topk_idx       [T, k] int32, k distinct ids in [0, E) per token.  (in)
 *   T, E, k, R     R divides E.
 *   capacity       per-expert row limit; <= 0 means unlimited.
 *   expert_counts  [E]   raw number of slots per expert (sums to T*k).  (out)
 *   expert_offsets [E+1] exclusive prefix sum of kept rows per expert;
 *                  expert_offsets[E] = N, the number of rows.           (out)
 *   rank_counts    [R]   kept rows per destination rank.                (out)
 *   rank_offsets   [R+1] rank_offsets[r] = expert_offsets[r*E/R];
 *                  rank_offsets[R] = N.                                 (out)
 *   pos            [T*k] row of slot s in the send buffer, -1 if the slot
 *                  was dropped by the capacity.                         (out)
 *   row_src        [T*k] slot that row p holds for p < N, -1 for p >= N. (out)
 *   workspace      device scratch of *workspace_bytes bytes, 256-byte
 *                  aligned, not shared with a concurrent call.  Pass NULL
 *                  to query: the required size is written to
 *                  *workspace_bytes and MOE_OK returned, nothing launched.
 *   workspace_bytes host pointer, never NULL.
 *
 * N stays on the device (expert_offsets[E]); size the send buffer for the
 * worst case T*k rows (or min(T*k, E*capacity)).  pack and combine are
 * driven by `pos`, so the host never needs N.
 *
 * Errors: MOE_ERR_NULL; MOE_ERR_SHAPE (T < 0, E or k out of range as for
 * moe_route_topk, R < 1, E % R != 0, T*k >= 2^31); MOE_ERR_ALIGN (int32
 * arrays not 4-byte aligned, workspace not 256-byte aligned);
 * MOE_ERR_WORKSPACE (*workspace_bytes smaller than required).
 * T == 0 still writes the zero counts and offsets.
 */
int moe_dispatch_layout(const int32_t *topk_idx, int64_t T, int E, int k, int R,
                        int capacity, int32_t *expert_counts,
                        int32_t *expert_offsets, int32_t *rank_counts,
                        int32_t *rank_offsets, int32_t *pos, int32_t *row_src,
                        void *workspace, size_t *workspace_bytes,
                        hipStream_t stream);

/*
 * moe_dispatch_layout_chunks -- moe_dispatch_layout for every chunk of a
 * batch at once.  The batch is cut into chunks of `chunk_tokens` tokens
 * (ThunderEP s2.1/s2.2: the batch is processed in chunks, aggregated inside
 * each chunk); chunk c covers tokens [c*chunk_tokens, min(T,
 * (c+1)*chunk_tokens)), C = ceil(T / chunk_tokens) chunks, and the result is
 * exactly that of calling moe_dispatch_layout once per chunk, written into the
 * chunk's slice of each output.  Two launches serve all chunks.
 *
 *   chunk_tokens    >= 1 when T > 0; values >= T mean one chunk.
 *   capacity        per-expert limit for every chunk (<= 0: unlimited),
 *                   used when chunk_capacity is NULL.
 *   chunk_capacity  NULL, or a DEVICE array [C] of per-chunk limits.
 *   expert_counts   [C][E]      expert_offsets [C][E+1]
 *   rank_counts     [C][R]      rank_offsets   [C][R+1]
 *   pos, row_src    [T*k]: chunk c owns entries [c*chunk_tokens*k, ...), with
 *                   rows and slots relative to the chunk, as for one call.
 *   workspace       as for moe_dispatch_layout (query with NULL); the size
 *                   depends on T, chunk_tokens, E and k.
 *
 * Errors: as moe_dispatch_layout, plus MOE_ERR_SHAPE for chunk_tokens < 1
 * with T > 0 or more than 65535 chunks.
 */
int moe_dispatch_layout_chunks(const int32_t *topk_idx, int64_t T, int64_t chunk_tokens, int E,
                               int k, int R, int capacity, const int32_t *chunk_capacity,
                               int32_t *expert_counts, int32_t *expert_offsets,
                               int32_t *rank_counts, int32_t *rank_offsets, int32_t *pos,
                               int32_t *row_src, void *workspace, size_t *workspace_bytes,
                               hipStream_t stream);

/*
 * moe_route_layout_chunks -- moe_route_topk followed by
 * moe_dispatch_layout_chunks, with the router fused into the layout's
 * counting pass: while it picks each token's experts, the router counts
 * them per group of consecutive tokens (bucketing by destination during
 * routing, so the expert ids are not traversed a second time to count
 * them; ThunderEP write-up s5.2, first direction).  Every output is
 * identical, bit for bit, to the two separate calls with the same
 * arguments.  Two launches when a layout tile holds whole router groups
 * and the per-group histogram of a chunk has at most 65536 entries
 * (ceil(chunk_tokens / group) * E); otherwise three (the separate calls).
 * A group is 64 tokens (16 for E > 256) when T >= 16384 (4096 for
 * E > 256), else 16 (4): k = 1, 2, 4, 8 or 16 tiles whole groups.  The
 * workspace size therefore depends on T as well as on the chunking.
 *
 *   logits          [T, E] fp32, as moe_route_topk.                 (in)
 *   topk_idx/topk_w [T, k] outputs of the routing.                  (out)
 *   the rest        as moe_dispatch_layout_chunks.  The workspace
 *                   size differs from that call's: query it with
 *                   workspace == NULL.
 *
 * Errors: as moe_route_topk and moe_dispatch_layout_chunks.
 */
int moe_route_layout_chunks(const float *logits, int64_t T, int64_t chunk_tokens, int E,
                            int k, int R, int capacity, const int32_t *chunk_capacity,
                            int32_t *topk_idx, float *topk_w, int32_t *expert_counts,
                            int32_t *expert_offsets, int32_t *rank_counts,
                            int32_t *rank_offsets, int32_t *pos, int32_t *row_src,
                            void *workspace, size_t *workspace_bytes, hipStream_t stream);

/*
 * moe_route_layout_chunks_noalloc -- moe_route_layout_chunks for callers
 * that cannot allocate device memory: code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc.  It takes no workspace:
 * the layout's histogram scratch is a static device array of the library,
 * MOE_NOALLOC_SCRATCH_BYTES (4 MiB) on each GPU, whose device address is
 * looked up on the first call on each device.  The copy used is that of the
 * stream's device (the current device for the null stream).  The caller still
 * passes every input and output; the call allocates nothing (no hipMalloc,
 * no allocating library routine).  Outputs are identical, bit for bit, to
 * moe_route_layout_chunks with the same arguments.
 *
 * The scratch needs no clearing (every entry the call reads it writes
 * first), but every call on one GPU shares that GPU's copy: calls whose
 * execution overlaps on one GPU (different streams, no ordering between
 * them) race on it and may return wrong layouts.  Order such calls on one
 * stream or with events.
 *
 *   arguments   as moe_route_layout_chunks, without the workspace.
 *
 * Errors: as moe_route_layout_chunks; MOE_ERR_SCRATCH when the call needs
 * more than MOE_NOALLOC_SCRATCH_BYTES of scratch (the size
 * moe_route_layout_chunks's workspace query reports for the same
 * arguments: at most 256 KiB per chunk, so 16 chunks always fit);
 * MOE_ERR_HIP when the scratch address cannot be obtained.  Nothing is
 * launched on error.
 */
int moe_route_layout_chunks_noalloc(const float *logits, int64_t T, int64_t chunk_tokens, int E,
                                    int k, int R, int capacity, const int32_t *chunk_capacity,
                                    int32_t *topk_idx, float *topk_w, int32_t *expert_counts,
                                    int32_t *expert_offsets, int32_t *rank_counts,
                                    int32_t *rank_offsets, int32_t *pos, int32_t *row_src,
                                    hipStream_t stream);

/*
 * moe_dispatch_pack -- stable scatter of hidden rows into the send buffer,
 * optionally compressed to per-token dynamic int8, int4 or fp8 (ThunderEP
 * s2.1 aggregation, s2.3 per-token int8 compression, s5.2 4-bit; NCCL EP
 * article s6.3 FP8).  For every slot s with pos[s] >= 0, row pos[s] of
 * `send` receives token s/k's row: a bit copy (MOE_QUANT_BF16) or its int8 /
 * int4 / fp8 codes (formats above), whose scale goes to send_scales[pos[s]].
 * Each token is read once and written to all of its kept slots.  Rows of
 * `send` that no slot points to are not written.
 *
 *   x_bf16       [T, H] bf16 bits, 16-byte aligned.                    (in)
 *   pos          [T*k] int32, from moe_dispatch_layout.                (in)
 *   quant        MOE_QUANT_BF16, MOE_QUANT_INT8, MOE_QUANT_INT4 or
 *                MOE_QUANT_FP8, optionally OR MOE_PACK_STREAM.
 *   send         [>= N rows, moe_row_bytes(H, quant)] bytes, 16-byte
 *                aligned.                                              (out)
 *   send_scales  [>= N] fp32, 4-byte aligned; quantised formats only
 *                (ignored, may be NULL, for MOE_QUANT_BF16).           (out)
 *
 * Errors: MOE_ERR_NULL; MOE_ERR_SHAPE (T < 0, k out of range, H < 16,
 * H > MOE_MAX_HIDDEN, H % 16 != 0, unknown quant, H % 32 != 0 for int4,
 * T*k >= 2^31);
 * MOE_ERR_ALIGN.  T == 0: MOE_OK, nothing launched.
 */
int moe_dispatch_pack(const void *x_bf16, int64_t T, int H, int k,
                      const int32_t *pos, int quant, void *send, float *send_scales,
                      hipStream_t stream);

/*
 * moe_combine -- gather, dequantise and gate-weighted sum back into token
 * order (ThunderEP s1.3: the expert results return to the token's GPU,
 * which forms the weighted sum).
 *     out[t, h] = bf16_rne( sum_{j < k, pos[t*k+j] >= 0}
 *                            topk_w[t*k+j] * deq(recv[pos[t*k+j]])[h] )
 * accumulated in fp32 in slot order j = 0..k-1, starting from -0, one fused
 * multiply-add per kept slot and element; a token whose slots were all
 * dropped gets +0.  Dropped slots are not renormalised.  The association is
 * the kernel's, not the formula's: bf16 adds w * x; the quantised formats
 * multiply the row's weight and scale once (w * scale, fp32) and add
 * code * (w * scale) (for int4, (16 * code) * (w * scale / 16), the same
 * product), where the format's dequantised value is (float)code * scale.  A
 * single kept bf16 slot with w = 1 returns its row bit for bit; otherwise
 * the result differs from the exactly rounded sum by fp32 rounding only
 * (held to 1e-3 + 1e-2 * |exact| element-wise).
 *
 *   recv         return buffer, rows as written for `quant`, 16-byte
 *                aligned.                                              (in)
 *   recv_scales  their scales (quantised formats; ignored for bf16).  (in)
 *   pos          [T*k] int32, the layout used for the dispatch.        (in)
 *   topk_w       [T*k] fp32 gate weights.                              (in)
 *   out          [T, H] bf16 bits, 16-byte aligned.                    (out)
 *
 * Errors: as moe_dispatch_pack.  T == 0: MOE_OK, nothing launched.
 */
int moe_combine(const void *recv, const float *recv_scales, int quant, const int32_t *pos,
                const float *topk_w, int64_t T, int H, int k, void *out_bf16,
                hipStream_t stream);

/*
 * moe_combine_pack -- moe_combine of one chunk and moe_dispatch_pack of
 * another in a single launch (chunks of one batch overlap, ThunderEP s2.2:
 * the combine of chunk c runs beside the pack of chunk c+1).  The outputs
 * are bit for bit those of
 *     moe_combine(recv, recv_scales, quant, pos_c, topk_w, Tc, H, k, out_bf16, stream);
 *     moe_dispatch_pack(x_bf16, Tp, H, k, pos_p, quant, send, send_scales, stream);
 * but the two run concurrently, so `send` / `send_scales` must not overlap
 * `recv`, `recv_scales`, `out_bf16`, `x_bf16`, `pos_c` or `topk_w`, and
 * `out_bf16` must not overlap `recv`, `recv_scales`, `x_bf16` or `pos_p`: a
 * staging ring of two buffers, the combine reading one while the pack fills
 * the other, is the intended use.  Both halves use the same payload format
 * `quant`; MOE_PACK_STREAM in `quant` applies to the pack half.
 *
 *   recv, recv_scales, pos_c, topk_w, Tc, out_bf16   as moe_combine (chunk c).
 *   x_bf16, pos_p, Tp, send, send_scales             as moe_dispatch_pack
 *                                                    (chunk c+1).
 *   H, k, quant                                      shared.
 *
 * Errors: MOE_ERR_SHAPE as moe_dispatch_pack for either half (Tc or Tp
 * negative, ...); MOE_ERR_NULL and MOE_ERR_ALIGN for the pointers of a half
 * with work (Tc > 0, resp. Tp > 0); MOE_ERR_ALIAS when both halves have work
 * and one of the overlaps above is possible: the byte ranges are taken at the
 * largest extent the sizes allow (send: Tp*k rows, send_scales: Tp*k floats,
 * recv: Tc*k rows, recv_scales, pos_c and topk_w: Tc*k entries, out_bf16:
 * Tc*H, x_bf16: Tp*H bf16, pos_p: Tp*k), so buffers that touch only beyond
 * the rows actually used are rejected too.  Tc == 0 and Tp == 0: MOE_OK,
 * nothing launched; one of them 0: the other call alone.
 */
int moe_combine_pack(const void *recv, const float *recv_scales, const int32_t *pos_c,
                     const float *topk_w, int64_t Tc, void *out_bf16, const void *x_bf16,
                     const int32_t *pos_p, int64_t Tp, void *send, float *send_scales, int H,
                     int k, int quant, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_ROUTE_H */
