// Test-support library (libmoe_harness.so), not part of the data path: the
// expert stand-in that sits between dispatch and combine in the round-trip
// tests, the stand-in for the payload all-to-all when every rank lives on one
// device, and the bandwidth probes (achievable copy and read bandwidth, and a
// read sweep that evicts the last-level cache between measured kernels).  The
// C entry points are declared in moe_harness.h.
#include "../../include/moe_harness.h"
#include "checks.hpp"
#include "common.hpp"
#include "launch.hpp"
#include "recv_rows.hpp"

namespace moe {
namespace {

// Stand-in expert: one block per row p < N.  Row p belongs to the expert e
// with offsets[e] <= p < offsets[e+1] (binary search over block-uniform
// scalar loads).  y = bf16(v * (1 + e/8)), v the dequantised input; int8 /
// int4 / fp8 output re-quantises y with the dispatch rule.  Each thread
// reads all of its input (row and scale) before any write, and quantised
// output writes only after a block barrier, so ret == recv (same format,
// same scale array) is safe.  No __restrict__ on the row and scale pointers:
// they may alias.
template <int VPT>
__global__ __launch_bounds__(1024) void standin_kernel(const uint8_t *recv,
                                                       const float *rscales, int quant_in,
                                                       const int32_t *__restrict__ offsets,
                                                       int E, int HV, int quant_out,
                                                       uint8_t *ret, float *oscales)
{
    __shared__ float red[16];
    const int64_t p = blockIdx.x;
    const int N = offsets[E];
    if (p >= N)
        return;
    int lo = 0, hi = E;  // offsets[lo] <= p < offsets[hi]
    while (hi - lo > 1) {
        const int mid = (lo + hi) / 2;
        if (offsets[mid] <= p)
            lo = mid;
        else
            hi = mid;
    }
    const float fac = 1.0f + static_cast<float>(lo) / 8.0f;
    const int H = HV * 8;
    const int64_t sin = row_bytes(H, quant_in);
    const int64_t sout = row_bytes(H, quant_out);
    const uint8_t *rin = recv + p * sin;
    uint8_t *rout = ret + p * sout;
    const int nthr = blockDim.x;
    const float scale_in = quant_in ? rscales[p] : 0.0f;

    float y[VPT][8];
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
        const int c = threadIdx.x + i * nthr;
        float v[8] = {0, 0, 0, 0, 0, 0, 0, 0};
        if (c < HV) {
            if (quant_in == 1)
                dequant8(reinterpret_cast<const u32x2 *>(rin)[c], scale_in, v);
            else if (quant_in == 3)
                dequant_fp8x8(reinterpret_cast<const u32x2 *>(rin)[c], scale_in, v);
            else if (quant_in == 2)
                dequant4x8(reinterpret_cast<const uint32_t *>(rin)[c], scale_in, v);
            else
                unpack8(reinterpret_cast<const u32x4 *>(rin)[c], v);
        }
#pragma unroll
        for (int q = 0; q < 8; ++q)
            v[q] = v[q] * fac;
        // round to bf16 and widen back: y is the bf16 expert output
        const u32x4 b = pack8(v);
        unpack8(b, y[i]);
#pragma unroll
        for (int q = 0; q < 8; ++q)
            amax = fmaxf(amax, fabsf(y[i][q]));
    }
    if (!quant_out) {
#pragma unroll
        for (int i = 0; i < VPT; ++i) {
            const int c = threadIdx.x + i * nthr;
            if (c < HV)
                reinterpret_cast<u32x4 *>(rout)[c] = pack8(y[i]);
        }
        return;
    }
    amax = block_max_nonneg(amax, red);
    const bool zero = (amax == 0.0f);
    const float qmax = quant_out == 1 ? 127.0f : (quant_out == 2 ? 7.0f : 448.0f);
    const float scale = zero ? 0.0f : amax / qmax;
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
        const int c = threadIdx.x + i * nthr;
        if (c < HV) {
            if (quant_out == 1)
                reinterpret_cast<u32x2 *>(rout)[c] = quant8(y[i], scale, zero);
            else if (quant_out == 3)
                reinterpret_cast<u32x2 *>(rout)[c] =
                    u32x2{fp8x4(y[i], scale, zero), fp8x4(y[i] + 4, scale, zero)};
            else
                reinterpret_cast<uint32_t *>(rout)[c] = quant4x8(y[i], scale, zero);
        }
    }
    if (threadIdx.x == 0)
        oscales[p] = scale;
}

// Bandwidth probes: one workgroup per tile of contiguous bytes, one 16-byte
// vector per thread, through a buffer descriptor bounded to the tile (the
// last tile may be short: loads past it read zeros, stores are dropped).
// Copy: 256-thread (4 KiB) tiles, streaming loads and streaming
// device-scope stores, the fastest of the tile shapes (4-16 KiB, runs of
// tiles taken in permuted or interleaved order) and cache policies measured
// for a copy larger than the last-level cache.  Read: 1024-thread (16 KiB) tiles; a
// lane whose vector has all bits set adds one to a counter (so the loads
// cannot be dropped; for other data nothing is written), with
// default-policy loads, which allocate in the last-level cache (a read
// sweep larger than the cache leaves it holding only clean lines of the
// swept buffer), or streaming loads, which do not.
constexpr int kCopyTileThreads = 256;
constexpr int kReadTileThreads = 1024;

__global__ __launch_bounds__(kCopyTileThreads) void probe_copy_kernel(const uint8_t *src,
                                                                      uint8_t *dst,
                                                                      int64_t bytes)
{
    const int64_t tile = static_cast<int64_t>(kCopyTileThreads) * 16;
    const int64_t t0 = static_cast<int64_t>(blockIdx.x) * tile;
    const int n = static_cast<int>(bytes - t0 < tile ? bytes - t0 : tile);
    const __amdgpu_buffer_rsrc_t rs = row_rsrc(const_cast<uint8_t *>(src) + t0, n);
    const __amdgpu_buffer_rsrc_t rd = row_rsrc(dst + t0, n);
    store_row<true>(rd, threadIdx.x * 16, load_stream16(rs, threadIdx.x * 16));
}

template <bool STREAM>
__global__ __launch_bounds__(kReadTileThreads) void probe_read_kernel(const uint8_t *src,
                                                                     uint32_t *ones,
                                                                     int64_t bytes)
{
    const int64_t tile = static_cast<int64_t>(kReadTileThreads) * 16;
    const int64_t t0 = static_cast<int64_t>(blockIdx.x) * tile;
    const int n = static_cast<int>(bytes - t0 < tile ? bytes - t0 : tile);
    const __amdgpu_buffer_rsrc_t rs = row_rsrc(const_cast<uint8_t *>(src) + t0, n);
    const u32x4 v = STREAM ? load_stream16(rs, threadIdx.x * 16) : load_cached(rs, threadIdx.x * 16);
    if ((v.x & v.y & v.z & v.w) == 0xFFFFFFFFu)
        atomicAdd(ones, 1u);
}

// The all-to-all of R ranks on one device, one workgroup per row and one
// 16-byte vector per thread, each row loaded before its destination is
// searched (the search overlaps the load).  Forward walks the send rows: row
// u of source s belongs to the segment of the last rank r whose segment
// starts at or before u, and lands at recv_offsets[r][s] + (u - start).
// Scales (quantised rows; NULL for bf16) move with their rows, by thread 0.
template <int VPT>
__global__ __launch_bounds__(1024) void exchange_fwd_kernel(const u32x4 *__restrict__ send,
                                                            const float *__restrict__ sscales,
                                                            int64_t source_rows,
                                                            u32x4 *__restrict__ recv,
                                                            float *__restrict__ rscales, int vecs,
                                                            int64_t max_rows,
                                                            const int32_t *__restrict__ so, int E,
                                                            int R,
                                                            const int32_t *__restrict__ recv_offsets)
{
    const int u = blockIdx.x;
    const int s = blockIdx.y;
    const int32_t *o = so + static_cast<int64_t>(s) * (E + 1);
    if (u >= o[E])
        return;
    const int64_t src_row = static_cast<int64_t>(s) * source_rows + u;
    const u32x4 *a = send + src_row * vecs;
    u32x4 v[VPT];
#pragma unroll
    for (int j = 0; j < VPT; ++j) {
        const int c = threadIdx.x + j * blockDim.x;
        if (c < vecs)
            v[j] = a[c];
    }
    const int per = E / R;
    int lo = 0, hi = R;
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (o[mid * per] <= u)
            lo = mid;
        else
            hi = mid;
    }
    const int64_t q = recv_offsets[lo * (R + 1) + s] + (u - o[lo * per]);
    if (q < 0 || q >= max_rows)  // inconsistent tables: move nothing
        return;
    u32x4 *b = recv + q * vecs;
#pragma unroll
    for (int j = 0; j < VPT; ++j) {
        const int c = threadIdx.x + j * blockDim.x;
        if (c < vecs)
            __builtin_nontemporal_store(v[j], b + c);
    }
    if (sscales && threadIdx.x == 0)
        rscales[q] = sscales[src_row];
}

// Reverse (the return exchange): walks the receive rows q < N and moves each
// back to its source's send buffer.
template <int VPT>
__global__ __launch_bounds__(1024) void exchange_rev_kernel(u32x4 *__restrict__ send,
                                                            float *__restrict__ sscales,
                                                            int64_t source_rows,
                                                            const u32x4 *__restrict__ recv,
                                                            const float *__restrict__ rscales,
                                                            int vecs, const int32_t *__restrict__ so,
                                                            int E, int R,
                                                            const int32_t *__restrict__ recv_offsets)
{
    const int q = blockIdx.x;
    if (q >= recv_offsets[R * (R + 1) - 1])
        return;
    const u32x4 *a = recv + static_cast<int64_t>(q) * vecs;
    u32x4 v[VPT];
#pragma unroll
    for (int j = 0; j < VPT; ++j) {
        const int c = threadIdx.x + j * blockDim.x;
        if (c < vecs)
            v[j] = a[c];
    }
    const RecvRow x = locate_recv_row(q, recv_offsets, R);
    const int64_t first = so[static_cast<int64_t>(x.s) * (E + 1) + x.r * (E / R)];
    if (first < 0 || first + x.u >= source_rows)  // inconsistent tables: move nothing
        return;
    const int64_t dst_row = static_cast<int64_t>(x.s) * source_rows + first + x.u;
    u32x4 *b = send + dst_row * vecs;
#pragma unroll
    for (int j = 0; j < VPT; ++j) {
        const int c = threadIdx.x + j * blockDim.x;
        if (c < vecs)
            __builtin_nontemporal_store(v[j], b + c);
    }
    if (rscales && threadIdx.x == 0)
        sscales[dst_row] = rscales[q];
}

template <int VPT>
void launch_exchange_vpt(void *send, float *sscales, int64_t source_rows, void *recv,
                         float *rscales, int64_t max_rows, int vecs, int threads,
                         const int32_t *so, int E, int R, const int32_t *recv_offsets,
                         bool reverse, hipStream_t stream)
{
    u32x4 *sv = static_cast<u32x4 *>(send);
    u32x4 *rv = static_cast<u32x4 *>(recv);
    if (reverse)
        exchange_rev_kernel<VPT><<<dim3(static_cast<unsigned>(max_rows)), threads, 0, stream>>>(
            sv, sscales, source_rows, rv, rscales, vecs, so, E, R, recv_offsets);
    else
        exchange_fwd_kernel<VPT><<<dim3(static_cast<unsigned>(source_rows), R), threads, 0,
                                   stream>>>(sv, sscales, source_rows, rv, rscales, vecs, max_rows,
                                             so, E, R, recv_offsets);
}

hipError_t launch_exchange_blocks(void *send, float *send_scales, int64_t source_rows, void *recv,
                                  float *recv_scales, int64_t max_rows, int H, int quant,
                                  const int32_t *src_offsets, int E, int R,
                                  const int32_t *recv_offsets, bool reverse, hipStream_t stream)
{
    const int vecs = static_cast<int>(row_bytes(H, quant) / 16);
    if ((reverse ? max_rows : source_rows) == 0)
        return hipSuccess;
    if (quant == 0)
        send_scales = recv_scales = nullptr;
    const RowTiling rt = row_tiling(vecs);
#define MOE_XCH(V)                                                                             \
    launch_exchange_vpt<V>(send, send_scales, source_rows, recv, recv_scales, max_rows, vecs,   \
                           rt.threads, src_offsets, E, R, recv_offsets, reverse, stream)
    switch (rt.vpt) {
    case 1: MOE_XCH(1); break;
    case 2: MOE_XCH(2); break;
    case 4: MOE_XCH(4); break;
    default: MOE_XCH(8); break;
    }
#undef MOE_XCH
    return hipGetLastError();
}

hipError_t launch_expert_standin(const void *recv, const float *recv_scales, int quant_in,
                                 const int32_t *expert_offsets, int E, int64_t max_rows, int H,
                                 int quant_out, void *ret, float *ret_scales, hipStream_t stream)
{
    const int HV = H / 8;
    const RowTiling rt = row_tiling(HV);
    const dim3 grid(static_cast<unsigned>(max_rows));
    const dim3 block(rt.threads);
    const uint8_t *in = static_cast<const uint8_t *>(recv);
    uint8_t *o = static_cast<uint8_t *>(ret);
#define MOE_STANDIN(V)                                                                         \
    standin_kernel<V><<<grid, block, 0, stream>>>(in, recv_scales, quant_in, expert_offsets, E, \
                                                  HV, quant_out, o, ret_scales)
    switch (rt.vpt) {
    case 1: MOE_STANDIN(1); break;
    case 2: MOE_STANDIN(2); break;
    case 4: MOE_STANDIN(4); break;
    default: MOE_STANDIN(8); break;
    }
#undef MOE_STANDIN
    return hipGetLastError();
}

hipError_t launch_stream_probe(const void *src, void *dst, size_t bytes, int mode,
                              hipStream_t stream)
{
    const int64_t n = static_cast<int64_t>(bytes);
    const uint8_t *sp = static_cast<const uint8_t *>(src);
    if (mode == MOE_PROBE_COPY) {
        const int64_t tiles = (n + kCopyTileThreads * 16 - 1) / (kCopyTileThreads * 16);
        probe_copy_kernel<<<static_cast<unsigned>(tiles), kCopyTileThreads, 0, stream>>>(
            sp, static_cast<uint8_t *>(dst), n);
    } else {
        const int64_t tiles = (n + kReadTileThreads * 16 - 1) / (kReadTileThreads * 16);
        uint32_t *ones = static_cast<uint32_t *>(dst);
        if (mode == MOE_PROBE_READ_CACHED)
            probe_read_kernel<false><<<static_cast<unsigned>(tiles), kReadTileThreads, 0, stream>>>(
                sp, ones, n);
        else
            probe_read_kernel<true><<<static_cast<unsigned>(tiles), kReadTileThreads, 0, stream>>>(
                sp, ones, n);
    }
    return hipGetLastError();
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
}  // namespace moe

using namespace moe;

extern "C" {

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
    return hip_status(launch_expert_standin(recv, recv_scales, quant_in, expert_offsets, E,
                                            max_rows, H, quant_out, ret, ret_scales, stream));
}

int moe_exchange_blocks(void *send, float *send_scales, int64_t source_rows, void *recv,
                        float *recv_scales, int64_t max_rows, int H, int quant,
                        const int32_t *src_offsets, int E, int R, const int32_t *recv_offsets,
                        int reverse, hipStream_t stream)
{
    if (source_rows < 0 || (R >= 1 && too_many_slots(source_rows, R)))
        return MOE_ERR_SHAPE;
    const int s = check_recv_rows(send, send_scales, recv, recv_scales, max_rows, H, quant,
                                  src_offsets, E, R, recv_offsets);
    if (s != MOE_OK || max_rows == 0)
        return s;
    return hip_status(launch_exchange_blocks(send, send_scales, source_rows, recv, recv_scales,
                                             max_rows, H, quant, src_offsets, E, R, recv_offsets,
                                             reverse != 0, stream));
}

int moe_stream_probe(const void *src, void *dst, size_t bytes, int mode, hipStream_t stream)
{
    if ((bytes % 16) != 0 || bytes >= (size_t(1) << 40) ||
        (mode != MOE_PROBE_COPY && mode != MOE_PROBE_READ_CACHED &&
         mode != MOE_PROBE_READ_STREAM))
        return MOE_ERR_SHAPE;
    if (bytes == 0)
        return MOE_OK;
    if (!src || !dst)
        return MOE_ERR_NULL;
    if (!aligned(src, 16) || !aligned(dst, mode == MOE_PROBE_COPY ? 16 : 4))
        return MOE_ERR_ALIGN;
    return hip_status(launch_stream_probe(src, dst, bytes, mode, stream));
}

}  // extern "C"
