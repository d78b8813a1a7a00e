/*
 * moe_harness.h -- test-support library libmoe_harness.so, built beside the
 * product library libmoe_route.so but not part of it: nothing on the data
 * path calls these.  The expert stand-in replaces the expert FFN between
 * dispatch and combine so that the round trip can be checked end to end on
 * one GPU; the exchange stand-in replaces the all-to-all when every rank
 * lives on one device; the stream probe measures achievable bandwidth and
 * evicts the last-level cache between measured kernels.  Conventions
 * (device pointers, caller-owned, asynchronous on `stream`, host-side
 * validation, status codes from moe_route.h) are those of moe_route.h.
 */
#ifndef MOE_HARNESS_H
#define MOE_HARNESS_H

#include "moe_route.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * moe_expert_standin -- stand-in expert for the tests: experts run between
 * dispatch and combine (Perseus write-up on itsolotime.com, s1.1; ThunderEP
 * s3.3 pseudo-code), on rows decompressed at the destination (ThunderEP
 * s2.3).  Row p < N = expert_offsets[E] belongs to the expert e with
 * expert_offsets[e] <= p < expert_offsets[e+1]; its output is
 *     y_h = bf16_rne( fl32( v_h * (1 + e/8) ) )
 * with v the dequantised input row.  quant_out = MOE_QUANT_INT8 re-quantises
 * the bf16 row y with the dispatch rule (moe_route.h).  Rows p >= N are not
 * written.
 *
 *   recv            [max_rows, moe_row_bytes(H, quant_in)] bytes.     (in)
 *   recv_scales     [max_rows] fp32 when quant_in is quantised (else
 *                   ignored, may be NULL).                            (in)
 *   expert_offsets  [E+1] int32 from moe_dispatch_layout (device).   (in)
 *   max_rows        rows the buffers can hold (>= N); the grid covers
 *                   max_rows and rows >= N return at once.
 *   ret             [max_rows, moe_row_bytes(H, quant_out)] bytes; must
 *                   not overlap recv unless quant_in == quant_out and
 *                   ret == recv (in place).                           (out)
 *   ret_scales      [max_rows] fp32 when quant_out is quantised; may be
 *                   recv_scales itself when working in place.         (out)
 *
 * Errors: MOE_ERR_NULL, MOE_ERR_SHAPE (E, H as in moe_route.h, max_rows <
 * 0 or >= 2^31, unknown quant), MOE_ERR_ALIGN.
 */
int moe_expert_standin(const void *recv, const float *recv_scales, int quant_in,
                       const int32_t *expert_offsets, int E, int64_t max_rows, int H,
                       int quant_out, void *ret, float *ret_scales, hipStream_t stream);

/*
 * moe_exchange_blocks -- stand-in for the payload all-to-all when all R
 * ranks run on one device (the exchange itself belongs to the collective
 * library): a block transpose of the NCCL EP article's flat buffers (s3.3).
 * Source s's send buffer starts at row s*source_rows of `send`; its segment
 * for rank r (rows [src_offsets[s][r*E/R], src_offsets[s][(r+1)*E/R]))
 * lands at rows recv_offsets[r][s].. of the flat receive buffer `recv`
 * (moe_recv.h); a quantised row's scale moves with it between the two scale
 * arrays.  reverse != 0 moves every row the other way (the return exchange
 * after the experts): recv -> send.
 *
 *   send, send_scales   [R*source_rows rows, moe_row_bytes(H, quant)] and
 *                       [R*source_rows] fp32 (scales: quantised formats
 *                       only).
 *   source_rows         rows of one source's send buffer (>= its N).
 *   recv, recv_scales   [max_rows rows, same stride] and [max_rows] fp32,
 *                       not overlapping send / send_scales.
 *   max_rows            >= N total rows, < 2^31.
 *
 * Errors: MOE_ERR_NULL, MOE_ERR_SHAPE, MOE_ERR_ALIGN as moe_recv_regroup,
 * plus source_rows < 0 or R*source_rows >= 2^31.
 */
int moe_exchange_blocks(void *send, float *send_scales, int64_t source_rows, void *recv,
                        float *recv_scales, int64_t max_rows, int H, int quant,
                        const int32_t *src_offsets, int E, int R, const int32_t *recv_offsets,
                        int reverse, hipStream_t stream);

/* Modes of moe_stream_probe. */
#define MOE_PROBE_COPY 0        /* dst = src                                    */
#define MOE_PROBE_READ_CACHED 1 /* read src with loads that allocate in the
                                   last-level cache                             */
#define MOE_PROBE_READ_STREAM 2 /* read src with streaming loads                */

/*
 * moe_stream_probe -- reference bandwidth kernels (one workgroup per tile of
 * contiguous bytes, 16-byte vectors through buffer descriptors).
 *   MOE_PROBE_COPY: dst[i] = src[i] for i < bytes; 4 KiB tiles, streaming
 *     loads, device-scope stores.  Traffic 2 * bytes.  dst 16-byte aligned.
 *   MOE_PROBE_READ_CACHED / MOE_PROBE_READ_STREAM: reads src once in 16 KiB
 *     tiles and adds to the uint32 at dst (atomically) the number of 16-byte
 *     vectors of src whose bits are all set; for other data nothing is
 *     written.  Traffic `bytes`.  dst 4-byte aligned.  Cached loads allocate
 *     in the last-level cache: a sweep over more than the cache (256 MB on
 *     MI355X) leaves it holding only clean lines of src, which is how
 *     measured kernels are made to start from memory.  Streaming loads
 *     measure the read bandwidth without displacing the cache.
 * bytes % 16 == 0; src 16-byte aligned; src and dst do not overlap.
 *
 * Errors: MOE_ERR_SHAPE (bytes % 16 != 0, bytes >= 2^40, unknown mode),
 * MOE_ERR_NULL, MOE_ERR_ALIGN.  bytes == 0: MOE_OK, nothing launched.
 */
int moe_stream_probe(const void *src, void *dst, size_t bytes, int mode, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_HARNESS_H */
