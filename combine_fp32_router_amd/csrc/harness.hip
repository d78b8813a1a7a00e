// Test and measurement helpers (not on the data path): the expert stand-in
// that sits between dispatch and combine in the round-trip tests, the
// stand-in for the payload all-to-all when every rank lives on one device,
// and a plain 16-byte copy kernel used as the achievable-bandwidth reference.
#include "common.hpp"
#include "launch.hpp"
#include "recv_rows.hpp"

namespace moe {
namespace {

// Stand-in expert: one block per row p < N.  Row p belongs to the expert e
// with offsets[e] <= p < offsets[e+1] (binary search over block-uniform
// scalar loads).  y = bf16(v * (1 + e/8)), v the dequantised input; int8 /
// int4 / fp8 output re-quantises y with the dispatch rule.  Each thread reads all of its
// input before any write, and int8 output writes only after a block barrier,
// so ret == recv (same format) is safe.
template <int VPT>
__global__ __launch_bounds__(1024) void standin_kernel(const uint8_t *__restrict__ recv,
                                                       int quant_in,
                                                       const int32_t *__restrict__ offsets,
                                                       int E, int HV, int quant_out,
                                                       uint8_t *__restrict__ ret)
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
    const int64_t sin = record_bytes(H, quant_in);
    const int64_t sout = record_bytes(H, quant_out);
    const uint8_t *rin = recv + p * sin;
    uint8_t *rout = ret + p * sout;
    const int nthr = blockDim.x;
    const float scale_in =
        quant_in ? *reinterpret_cast<const float *>(rin + code_bytes(H, quant_in)) : 0.0f;

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
        *reinterpret_cast<u32x4 *>(rout + code_bytes(H, quant_out)) =
            u32x4{__float_as_uint(scale), 0u, 0u, 0u};
}

// dst = src, 16-byte vectors, 4 loads in flight per thread, grid-stride.
__global__ __launch_bounds__(256) void copy_kernel(const u32x4 *__restrict__ src,
                                                   u32x4 *__restrict__ dst, int64_t n)
{
    const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
    int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    for (; i + 3 * stride < n; i += 4 * stride) {
        const u32x4 a = __builtin_nontemporal_load(src + i);
        const u32x4 b = __builtin_nontemporal_load(src + i + stride);
        const u32x4 c = __builtin_nontemporal_load(src + i + 2 * stride);
        const u32x4 d = __builtin_nontemporal_load(src + i + 3 * stride);
        __builtin_nontemporal_store(a, dst + i);
        __builtin_nontemporal_store(b, dst + i + stride);
        __builtin_nontemporal_store(c, dst + i + 2 * stride);
        __builtin_nontemporal_store(d, dst + i + 3 * stride);
    }
    for (; i < n; i += stride)
        __builtin_nontemporal_store(__builtin_nontemporal_load(src + i), dst + i);
}

// The all-to-all of R ranks on one device, one workgroup per row and one
// 16-byte vector per thread, each row loaded before its destination is
// searched (the search overlaps the load).  Forward walks the send rows: row
// u of source s belongs to the segment of the last rank r whose segment
// starts at or before u, and lands at recv_offsets[r][s] + (u - start).
template <int VPT>
__global__ __launch_bounds__(1024) void exchange_fwd_kernel(const u32x4 *__restrict__ send,
                                                            int64_t source_rows,
                                                            u32x4 *__restrict__ recv, int vecs,
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
    const u32x4 *a = send + (static_cast<int64_t>(s) * source_rows + u) * vecs;
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
}

// Reverse (the return exchange): walks the receive rows q < N and moves each
// back to its source's send buffer.
template <int VPT>
__global__ __launch_bounds__(1024) void exchange_rev_kernel(u32x4 *__restrict__ send,
                                                            int64_t source_rows,
                                                            const u32x4 *__restrict__ recv,
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
    u32x4 *b = send + (static_cast<int64_t>(x.s) * source_rows + first + x.u) * vecs;
#pragma unroll
    for (int j = 0; j < VPT; ++j) {
        const int c = threadIdx.x + j * blockDim.x;
        if (c < vecs)
            __builtin_nontemporal_store(v[j], b + c);
    }
}

template <int VPT>
void launch_exchange_vpt(void *send, int64_t source_rows, void *recv, int64_t max_rows, int vecs,
                         int threads, const int32_t *so, int E, int R, const int32_t *recv_offsets,
                         bool reverse, hipStream_t stream)
{
    u32x4 *sv = static_cast<u32x4 *>(send);
    u32x4 *rv = static_cast<u32x4 *>(recv);
    if (reverse)
        exchange_rev_kernel<VPT><<<dim3(static_cast<unsigned>(max_rows)), threads, 0, stream>>>(
            sv, source_rows, rv, vecs, so, E, R, recv_offsets);
    else
        exchange_fwd_kernel<VPT><<<dim3(static_cast<unsigned>(source_rows), R), threads, 0,
                                   stream>>>(sv, source_rows, rv, vecs, max_rows, so, E, R,
                                             recv_offsets);
}

}  // namespace

hipError_t launch_exchange_blocks(void *send, int64_t source_rows, void *recv, int64_t max_rows,
                                  int H, int quant, const int32_t *src_offsets, int E, int R,
                                  const int32_t *recv_offsets, bool reverse, hipStream_t stream)
{
    const int vecs = static_cast<int>(record_bytes(H, quant) / 16);
    if ((reverse ? max_rows : source_rows) == 0)
        return hipSuccess;
    const RowTiling rt = row_tiling(vecs);
    switch (rt.vpt) {
    case 1: launch_exchange_vpt<1>(send, source_rows, recv, max_rows, vecs, rt.threads, src_offsets, E, R, recv_offsets, reverse, stream); break;
    case 2: launch_exchange_vpt<2>(send, source_rows, recv, max_rows, vecs, rt.threads, src_offsets, E, R, recv_offsets, reverse, stream); break;
    case 4: launch_exchange_vpt<4>(send, source_rows, recv, max_rows, vecs, rt.threads, src_offsets, E, R, recv_offsets, reverse, stream); break;
    default: launch_exchange_vpt<8>(send, source_rows, recv, max_rows, vecs, rt.threads, src_offsets, E, R, recv_offsets, reverse, stream); break;
    }
    return hipGetLastError();
}

hipError_t launch_expert_standin(const void *recv, int quant_in, const int32_t *expert_offsets,
                                 int E, int64_t max_rows, int H, int quant_out, void *ret,
                                 hipStream_t stream)
{
    const int HV = H / 8;
    const RowTiling rt = row_tiling(HV);
    const dim3 grid(static_cast<unsigned>(max_rows));
    const dim3 block(rt.threads);
    const uint8_t *in = static_cast<const uint8_t *>(recv);
    uint8_t *o = static_cast<uint8_t *>(ret);
    switch (rt.vpt) {
    case 1: standin_kernel<1><<<grid, block, 0, stream>>>(in, quant_in, expert_offsets, E, HV, quant_out, o); break;
    case 2: standin_kernel<2><<<grid, block, 0, stream>>>(in, quant_in, expert_offsets, E, HV, quant_out, o); break;
    case 4: standin_kernel<4><<<grid, block, 0, stream>>>(in, quant_in, expert_offsets, E, HV, quant_out, o); break;
    default: standin_kernel<8><<<grid, block, 0, stream>>>(in, quant_in, expert_offsets, E, HV, quant_out, o); break;
    }
    return hipGetLastError();
}

hipError_t launch_copy_probe(const void *src, void *dst, size_t bytes, int blocks,
                             hipStream_t stream)
{
    const int64_t n = static_cast<int64_t>(bytes / 16);
    if (blocks <= 0) {
        int64_t b = (n + 256 * 4 - 1) / (256 * 4);
        blocks = static_cast<int>(b < 8192 ? (b < 1 ? 1 : b) : 8192);
    }
    copy_kernel<<<blocks, 256, 0, stream>>>(static_cast<const u32x4 *>(src), static_cast<u32x4 *>(dst), n);
    return hipGetLastError();
}

}  // namespace moe
