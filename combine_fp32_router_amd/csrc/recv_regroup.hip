// Receiver side of the exchange: where each source's segment lands, the
// regroup of the received rows into one contiguous run per expert (expert,
// then source, then arrival order), and its inverse for the return trip.
//
//   recv_layout_kernel  one 1024-thread workgroup: stage every source's kept
//                       expert offsets in LDS, per-expert totals, block scan
//                       -> expert-major offsets and segment starts,
//                       per-receiver segment offsets.
//   recv_map_kernel     one thread per row: binary searches place receive
//                       row q in (receiver, source, expert) and give its
//                       grouped row p; writes group_pos[q] = p and
//                       group_src[p] = q (-1 past the last row).
//   gather_rows_kernel  one workgroup per output row, one 16-byte vector per
//                       thread: out[i] = in[map[i]].  Writes are sequential
//                       and reads follow the map; a gather measured faster
//                       than the equivalent scatter on this part, and both
//                       directions (regroup, ungroup) are gathers through
//                       one of the two maps.  HBM-bound.
#include "common.hpp"
#include "launch.hpp"
#include "recv_rows.hpp"

namespace moe {
namespace {

constexpr int kLayoutThreads = 1024;        // >= MOE_MAX_EXPERTS: one expert per thread
constexpr int kStageInts = 14336;           // LDS staging of src_offsets (56 KiB; with
                                            // the scan arrays the workgroup stays < 64 KiB)

// STAGED: src_offsets ([R][E+1]) copied to LDS first (R*(E+1) <= kStageInts).
template <bool STAGED>
__global__ __launch_bounds__(kLayoutThreads) void recv_layout_kernel(
    const int32_t *__restrict__ so_g, int E, int R, int32_t *__restrict__ recv_offsets,
    int32_t *__restrict__ group_offsets, int32_t *__restrict__ group_seg)
{
    extern __shared__ int32_t stage[];
    __shared__ int32_t goff[kLayoutThreads + 1];
    __shared__ int32_t wsum[kLayoutThreads / kWave];
    const int t = threadIdx.x;
    const int lane = lane_id();
    const int w = t / kWave;
    const int ostride = E + 1;
    const int32_t *so = so_g;
    if (STAGED) {
        const int n = R * ostride;
        for (int i = t; i < n; i += kLayoutThreads)
            stage[i] = so_g[i];
        __syncthreads();
        so = stage;
    }

    // rows of expert t summed over the sources
    int tot = 0;
    if (t < E)
        for (int s = 0; s < R; ++s)
            tot += so[s * ostride + t + 1] - so[s * ostride + t];

    // exclusive scan over experts
    const int incl = wave_inclusive_scan(tot);
    if (lane == kWave - 1)
        wsum[w] = incl;
    __syncthreads();
    int run = incl - tot;
    for (int i = 0; i < w; ++i)
        run += wsum[i];
    goff[t] = run;
    if (t == kLayoutThreads - 1)
        goff[kLayoutThreads] = run + tot;  // experts past E add nothing: the total
    __syncthreads();

    if (t < E) {
        group_offsets[t] = run;
        int g = run;
        for (int s = 0; s < R; ++s) {
            group_seg[static_cast<int64_t>(t) * R + s] = g;
            g += so[s * ostride + t + 1] - so[s * ostride + t];
        }
    }
    if (t == 0)
        group_offsets[E] = goff[kLayoutThreads];

    // receiver r: its region starts where its first expert's rows start
    const int per = E / R;
    for (int r = t; r < R; r += kLayoutThreads) {
        int q = goff[r * per];
        int32_t *ro = recv_offsets + static_cast<int64_t>(r) * (R + 1);
        for (int s = 0; s < R; ++s) {
            ro[s] = q;
            q += so[s * ostride + (r + 1) * per] - so[s * ostride + r * per];
        }
        ro[R] = q;
    }
}

__global__ __launch_bounds__(256) void recv_map_kernel(const int32_t *__restrict__ so, int E,
                                                       int R, const int32_t *__restrict__ recv_offsets,
                                                       const int32_t *__restrict__ group_seg,
                                                       int64_t max_rows,
                                                       int32_t *__restrict__ group_pos,
                                                       int32_t *__restrict__ group_src)
{
    const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    if (i >= max_rows)
        return;
    const int N = recv_offsets[R * (R + 1) - 1];
    if (i >= N) {
        group_pos[i] = -1;
        group_src[i] = -1;
        return;
    }
    const int q = static_cast<int>(i);
    const RecvRow x = locate_recv_row(q, recv_offsets, R);
    const int per = E / R;
    const int32_t *o = so + static_cast<int64_t>(x.s) * (E + 1) + x.r * per;
    const int base = o[0];
    int lo = 0, hi = per;  // last expert of the segment whose run starts <= u
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (o[mid] - base <= x.u)
            lo = mid;
        else
            hi = mid;
    }
    const int e = x.r * per + lo;
    const int p = group_seg[static_cast<int64_t>(e) * R + x.s] + (x.u - (o[lo] - base));
    group_pos[q] = p;
    if (p >= 0 && p < max_rows)
        group_src[p] = q;
}

// out[i] = in[map[i]] for every i < max_rows with 0 <= map[i] < max_rows;
// thread 0 moves the row's scale when the rows are quantised (in_scales
// not NULL).  Both rows go through buffer descriptors: nontemporal loads
// (lanes past the row read zeros) and device-scope stores, which write the
// grouped row through L2 for the next kernel to read from the last-level
// cache.  Against cached global loads and nontemporal stores this cut
// regroup / ungroup at the dsv3 receiver shape (131072 rows) from 577 / 594
// to 558 / 563 µs for bf16 and from 297 / 306 to 270 / 277 µs for int8.
template <int VPT>
__global__ __launch_bounds__(1024) void gather_rows_kernel(const u32x4 *__restrict__ in,
                                                           const float *__restrict__ in_scales,
                                                           u32x4 *__restrict__ out,
                                                           float *__restrict__ out_scales, int vecs,
                                                           int64_t max_rows,
                                                           const int32_t *__restrict__ map)
{
    const int64_t i = blockIdx.x;
    const int64_t src = map[i];
    if (src < 0 || src >= max_rows)
        return;
    const __amdgpu_buffer_rsrc_t a = row_rsrc(const_cast<u32x4 *>(in) + src * vecs, vecs * 16);
    const __amdgpu_buffer_rsrc_t b = row_rsrc(out + i * vecs, vecs * 16);
    u32x4 v[VPT];
#pragma unroll
    for (int j = 0; j < VPT; ++j)
        v[j] = load_stream16(a, (threadIdx.x + j * blockDim.x) * 16);
#pragma unroll
    for (int j = 0; j < VPT; ++j) {
        const int c = threadIdx.x + j * blockDim.x;
        if (c < vecs)
            store_device(b, c * 16, v[j]);
    }
    if (in_scales && threadIdx.x == 0)
        out_scales[i] = in_scales[src];
}

}  // namespace

hipError_t launch_recv_layout(const int32_t *src_offsets, int E, int R, int64_t max_rows,
                              int32_t *recv_offsets, int32_t *group_offsets, int32_t *group_seg,
                              int32_t *group_pos, int32_t *group_src, hipStream_t stream)
{
    const int64_t table = static_cast<int64_t>(R) * (E + 1);
    if (table <= kStageInts)
        recv_layout_kernel<true><<<1, kLayoutThreads, table * sizeof(int32_t), stream>>>(
            src_offsets, E, R, recv_offsets, group_offsets, group_seg);
    else
        recv_layout_kernel<false><<<1, kLayoutThreads, 0, stream>>>(
            src_offsets, E, R, recv_offsets, group_offsets, group_seg);
    if (max_rows > 0) {
        const int64_t blocks = (max_rows + 255) / 256;
        recv_map_kernel<<<dim3(static_cast<unsigned>(blocks)), 256, 0, stream>>>(
            src_offsets, E, R, recv_offsets, group_seg, max_rows, group_pos, group_src);
    }
    return hipGetLastError();
}

hipError_t launch_gather_rows(const void *in, const float *in_scales, void *out, float *out_scales,
                              int64_t max_rows, int H, int quant, const int32_t *map,
                              hipStream_t stream)
{
    const int vecs = static_cast<int>(row_bytes(H, quant) / 16);
    const RowTiling rt = row_tiling(vecs);
    const dim3 grid(static_cast<unsigned>(max_rows));
    const u32x4 *i = static_cast<const u32x4 *>(in);
    u32x4 *o = static_cast<u32x4 *>(out);
    if (quant == 0) {
        in_scales = nullptr;
        out_scales = nullptr;
    }
#define MOE_GATHER(V)                                                                          \
    gather_rows_kernel<V><<<grid, rt.threads, 0, stream>>>(i, in_scales, o, out_scales, vecs,  \
                                                           max_rows, map)
    switch (rt.vpt) {
    case 1: MOE_GATHER(1); break;
    case 2: MOE_GATHER(2); break;
    case 4: MOE_GATHER(4); break;
    default: MOE_GATHER(8); break;
    }
#undef MOE_GATHER
    return hipGetLastError();
}

}  // namespace moe
