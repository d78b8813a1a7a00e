/*
 * moe_recv.h -- the receiver side of the expert-parallel exchange: where
 * each source's segment lands in a rank's receive buffer, and the regroup of
 * the received rows into one contiguous run per expert, ready for the
 * experts, with its inverse for the return trip.  Exported by the same
 * library as moe_route.h; conventions (device pointers, caller-owned,
 * asynchronous on `stream`, host-side validation, status codes) are those of
 * moe_route.h.
 *
 * The group has R ranks; every rank is a source and a receiver.  Rank r owns
 * the contiguous experts [r*E/R, (r+1)*E/R) (the EP=8 placement example of
 * the "communication wall" explainer on juhe.plus).  Source s's send buffer
 * is one flat block cut into R segments at the prefix sums of its per-rank
 * counts, and a receive buffer is laid out the same way, the segment from
 * source s following those from sources < s (NCCL EP article on
 * hotelren.com, s3.3).  The experts then run on the received rows (Perseus
 * write-up on itsolotime.com, s1.1), so the receiver gathers each expert's
 * rows into one run: expert ascending, then source ascending, then arrival
 * order.  When the sources are consecutive token shards of one batch, that
 * order is the batch's own (expert, token) order.
 *
 * Input shared by the calls: src_offsets [R][E+1] int32, the kept expert
 * offsets of every source's dispatch layout (moe_dispatch_layout's
 * expert_offsets, one row per source, e.g. moe_dispatch_layout_chunks with
 * one chunk per source), as the count exchange delivers them to every rank.
 * Source s's segment for rank r is its send rows [src_offsets[s][r*E/R],
 * src_offsets[s][(r+1)*E/R]).  Offsets must be non-decreasing in e, and the
 * total over all sources must be < 2^31.
 *
 * Flat numbering.  The receive buffers of all R ranks lie end to end in rank
 * order, and so do their grouped buffers, so every offset below is a row of
 * one flat buffer (this is how all ranks are run on one device).  A rank
 * holding only its own buffer subtracts recv_offsets[r][0] from its rows.
 */
#ifndef MOE_RECV_H
#define MOE_RECV_H

#include "moe_route.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * moe_recv_layout -- receive offsets, expert-major segment starts, and the
 * two row maps that drive the regroup (the receiver's counterpart of
 * moe_dispatch_layout's pos / row_src).  Two launches: one workgroup for the
 * offsets, one thread per row for the maps.
 *
 *   src_offsets    [R][E+1] int32, as above.                          (in)
 *   E, R           1 <= R, R divides E, E <= MOE_MAX_EXPERTS.
 *   max_rows       entries of each row map, >= N (the total kept rows of
 *                  all sources), < 2^31.  The sum of all sources' slot
 *                  counts is always enough.
 *   recv_offsets   [R][R+1] int32: recv_offsets[r][s] is the first row of
 *                  source s's segment in rank r's region;
 *                  recv_offsets[r][R] ends the region (= the next rank's
 *                  [0]); recv_offsets[R-1][R] = N.                     (out)
 *   group_offsets  [E+1] int32: first grouped row of expert e; [E] = N.
 *                  Rank r's grouped rows start at group_offsets[r*E/R] =
 *                  recv_offsets[r][0].                                 (out)
 *   group_seg      [E][R] int32: first grouped row of source s's rows of
 *                  expert e.                                          (out)
 *   group_pos      [max_rows] int32: grouped row of receive row q for
 *                  q < N, -1 for q >= N.                               (out)
 *   group_src      [max_rows] int32: receive row held by grouped row p for
 *                  p < N (the inverse permutation), -1 for p >= N.     (out)
 *
 * Errors: MOE_ERR_NULL, MOE_ERR_SHAPE (E or R out of range, max_rows < 0 or
 * >= 2^31), MOE_ERR_ALIGN (arrays not 4-byte aligned).  With max_rows ==
 * 0 the maps may be NULL and only the offsets are written.  N > max_rows
 * leaves the maps incomplete (never written out of bounds).
 */
int moe_recv_layout(const int32_t *src_offsets, int E, int R, int64_t max_rows,
                    int32_t *recv_offsets, int32_t *group_offsets,
                    int32_t *group_seg, int32_t *group_pos, int32_t *group_src,
                    hipStream_t stream);

/*
 * moe_recv_regroup -- receive buffer -> grouped buffer:
 *     grouped[p] = recv[group_src[p]]   for every p < max_rows with
 *                                       0 <= group_src[p] < max_rows
 * and, for a quantised format, grouped_scales[p] = recv_scales[group_src[p]].
 * One workgroup per grouped row, one 16-byte vector per thread.  Rows (bf16
 * rows or quantised codes, moe_route.h) are moved unchanged; rows with a -1
 * map entry are not written.
 *
 *   recv            [max_rows rows, moe_row_bytes(H, quant)], 16-byte
 *                   aligned.                                          (in)
 *   recv_scales     [max_rows] fp32 (quantised formats; ignored, may be
 *                   NULL, for bf16).                                  (in)
 *   group_src       [max_rows] int32 from moe_recv_layout.            (in)
 *   grouped         [max_rows rows, same stride], 16-byte aligned, not
 *                   overlapping recv.                                 (out)
 *   grouped_scales  [max_rows] fp32, as recv_scales, not overlapping
 *                   it.                                               (out)
 *
 * Errors: MOE_ERR_NULL, MOE_ERR_SHAPE (H, quant as for moe_dispatch_pack;
 * max_rows < 0 or >= 2^31), MOE_ERR_ALIGN.  max_rows == 0: MOE_OK, nothing
 * launched.
 */
int moe_recv_regroup(const void *recv, const float *recv_scales, int64_t max_rows, int H,
                     int quant, const int32_t *group_src, void *grouped, float *grouped_scales,
                     hipStream_t stream);

/*
 * moe_recv_ungroup -- the inverse, after the experts: grouped buffer (the
 * experts' output rows, in grouped order) -> receive order, ready for the
 * return exchange:
 *     recv[q] = grouped[group_pos[q]]   (and the scales alike)
 * Arguments and errors as moe_recv_regroup with the buffers' roles swapped.
 */
int moe_recv_ungroup(const void *grouped, const float *grouped_scales, int64_t max_rows, int H,
                     int quant, const int32_t *group_pos, void *recv, float *recv_scales,
                     hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_RECV_H */
