// Receiver side of the exchange: where each source's segment lands, and the
// regroup of the received rows into one contiguous run per expert (expert,
// then source, then arrival order), plus its inverse for the return trip.
//
//   recv_layout_kernel  one 1024-thread block: per-expert totals over the
//                       sources, block scan -> expert-major offsets, segment
//                       starts; per-receiver segment offsets.
//   regroup_kernel      one wave per received row: scalar binary searches
//                       find (receiver, source, expert), then the wave moves
//                       the row with 16-byte accesses.  HBM-bound.
#include "common.hpp"
#include "launch.hpp"
#include "recv_rows.hpp"

namespace moe {
namespace {

constexpr int kLayoutThreads = 1024;  // >= MOE_MAX_EXPERTS: one expert per thread

__global__ __launch_bounds__(kLayoutThreads) void recv_layout_kernel(
    const int32_t *__restrict__ so, int E, int R, int32_t *__restrict__ recv_offsets,
    int32_t *__restrict__ group_offsets, int32_t *__restrict__ group_seg)
{
    __shared__ int32_t goff[kLayoutThreads + 1];
    __shared__ int32_t wsum[kLayoutThreads / kWave];
    const int t = threadIdx.x;
    const int lane = lane_id();
    const int w = t / kWave;
    const int64_t ostride = E + 1;

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

// UNGROUP = false: grouped[dst(q)] = recv[q];  true: recv[q] = grouped[dst(q)].
template <bool UNGROUP, int B>
__global__ __launch_bounds__(256) void regroup_kernel(const u32x4 *__restrict__ in,
                                                      u32x4 *__restrict__ out, int vecs,
                                                      int64_t max_rows,
                                                      const int32_t *__restrict__ so, int E, int R,
                                                      const int32_t *__restrict__ recv_offsets,
                                                      const int32_t *__restrict__ group_seg)
{
    const int waves = blockDim.x / kWave;
    const int wv = static_cast<int>(uniform(threadIdx.x / kWave));
    const int64_t q64 = static_cast<int64_t>(blockIdx.x) * waves + wv;
    const int N = recv_offsets[R * (R + 1) - 1];
    if (q64 >= max_rows || q64 >= N)
        return;
    const int q = static_cast<int>(q64);
    const RecvRow x = locate_recv_row(q, recv_offsets, R);
    // expert: last e of the receiver's experts whose run in the segment starts <= u
    const int per = E / R;
    const int32_t *o = so + static_cast<int64_t>(x.s) * (E + 1) + x.r * per;
    const int base = o[0];
    int lo = 0, hi = per;
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (o[mid] - base <= x.u)
            lo = mid;
        else
            hi = mid;
    }
    const int e = x.r * per + lo;
    const int64_t dst = group_seg[static_cast<int64_t>(e) * R + x.s] + (x.u - (o[lo] - base));
    if (dst < 0 || dst >= max_rows)  // inconsistent tables or a short buffer: move nothing
        return;
    const int lane = lane_id();
    if (UNGROUP)
        wave_copy_row<B>(in + dst * vecs, out + static_cast<int64_t>(q) * vecs, vecs, lane);
    else
        wave_copy_row<B>(in + static_cast<int64_t>(q) * vecs, out + dst * vecs, vecs, lane);
}

template <bool UNGROUP>
hipError_t launch_regroup_dir(const void *in, void *out, int64_t max_rows, int H, int quant,
                              const int32_t *so, int E, int R, const int32_t *recv_offsets,
                              const int32_t *group_seg, hipStream_t stream)
{
    const int vecs = static_cast<int>((quant ? H + 16 : 2 * H) / 16);
    constexpr int kThreads = 256;
    const int64_t blocks = (max_rows + kThreads / kWave - 1) / (kThreads / kWave);
    const u32x4 *i = static_cast<const u32x4 *>(in);
    u32x4 *o = static_cast<u32x4 *>(out);
    if (vecs <= 8 * kWave)
        regroup_kernel<UNGROUP, 8><<<dim3(static_cast<unsigned>(blocks)), kThreads, 0, stream>>>(
            i, o, vecs, max_rows, so, E, R, recv_offsets, group_seg);
    else
        regroup_kernel<UNGROUP, 16><<<dim3(static_cast<unsigned>(blocks)), kThreads, 0, stream>>>(
            i, o, vecs, max_rows, so, E, R, recv_offsets, group_seg);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_recv_layout(const int32_t *src_offsets, int E, int R, int32_t *recv_offsets,
                              int32_t *group_offsets, int32_t *group_seg, hipStream_t stream)
{
    recv_layout_kernel<<<1, kLayoutThreads, 0, stream>>>(src_offsets, E, R, recv_offsets,
                                                         group_offsets, group_seg);
    return hipGetLastError();
}

hipError_t launch_recv_regroup(const void *in, void *out, int64_t max_rows, int H, int quant,
                               const int32_t *src_offsets, int E, int R,
                               const int32_t *recv_offsets, const int32_t *group_seg, bool ungroup,
                               hipStream_t stream)
{
    if (ungroup)
        return launch_regroup_dir<true>(in, out, max_rows, H, quant, src_offsets, E, R,
                                        recv_offsets, group_seg, stream);
    return launch_regroup_dir<false>(in, out, max_rows, H, quant, src_offsets, E, R, recv_offsets,
                                     group_seg, stream);
}

}  // namespace moe
