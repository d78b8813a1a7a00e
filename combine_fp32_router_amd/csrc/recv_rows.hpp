// Row addressing on the receiver side of the exchange, shared by the row-map
// kernel and the exchange stand-in.
//
// An EP group has R ranks; rank r owns experts [r*E/R, (r+1)*E/R).  Every
// rank is a source: src_offsets[s*(E+1) + e] are the kept expert offsets of
// source s's dispatch layout, so its segment for rank r is its rows
// [src_offsets[s][r*E/R], src_offsets[s][(r+1)*E/R]).  The receive buffers
// of all ranks lie end to end in rank order; inside receiver r's region the
// segments follow in source order, their first rows being
// recv_offsets[r*(R+1) + s] (flat row numbers; [r*(R+1) + R] ends it).
#pragma once

#include "common.hpp"

namespace moe {

struct RecvRow {
    int r;  // receiving rank
    int s;  // source rank
    int u;  // row inside the source's segment
};

// Locate flat receive row q (q < total rows).  All loads depend only on q
// and the tables, so a wave-uniform q keeps the search in scalar registers.
// Each search keeps table[lo] <= q < table[hi] with table[R] taken as +inf,
// so an empty receiver or segment (equal neighbouring starts) is skipped.
__device__ __forceinline__ RecvRow locate_recv_row(int q, const int32_t *__restrict__ recv_offsets,
                                                   int R)
{
    RecvRow x;
    int lo = 0, hi = R;
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (recv_offsets[mid * (R + 1)] <= q)
            lo = mid;
        else
            hi = mid;
    }
    x.r = lo;
    const int32_t *ro = recv_offsets + lo * (R + 1);
    lo = 0;
    hi = R;
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (ro[mid] <= q)
            lo = mid;
        else
            hi = mid;
    }
    x.s = lo;
    x.u = q - ro[lo];
    return x;
}

}  // namespace moe
