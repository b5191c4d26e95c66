// Per-query-head statistics of a GQA head from the per-tile partial sums the
// GQA score kernels write (sum, sum of squares, count of finite scores,
// largest |score| of each 512-row tile and query head).
//
// Source: dimensionstp.github.io "TriAttention ... Review", section 3-2
// item 6 (each query head's scores are z-score normalized over the head's
// cached keys).  Readings: the mean and the population deviation run over
// the finite scores; a deviation of at most kGqaFlat of the largest |score|
// counts as zero.
//
// Both the statistics kernel and the GQA selection (which forms the statistics
// itself when no normalized score array is written) call gqa_query_head_stats,
// so the two give the same bits.
#pragma once

#include "tri_internal.h"

namespace tri {

constexpr int kGqaTileRows = 512;       // rows per GQA score tile
constexpr double kGqaFlat = 1e-9;       // deviation at or below kGqaFlat * max|s| counts as zero

// (mean, deviation) of query head g of one head.  partial_head: the head's
// [tiles][group][4] partial sums.  Lane t adds tiles t, t + 64, ... in order,
// then a fixed butterfly combines the lanes; all 64 lanes of one wave call it
// and every lane gets the result.
__device__ __forceinline__ double2 gqa_query_head_stats(const double* __restrict__ partial_head,
                                                        int tiles, int group, int g, int lane)
{
    double s1 = 0.0, s2 = 0.0, cnt = 0.0, big = 0.0;
    for (int tile = lane; tile < tiles; tile += 64) {
        const double* p = partial_head + ((size_t)tile * group + g) * 4;
        s1 += p[0];
        s2 += p[1];
        cnt += p[2];
        big = fmax(big, p[3]);
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
        s1 += __shfl_xor(s1, o);
        s2 += __shfl_xor(s2, o);
        cnt += __shfl_xor(cnt, o);
        big = fmax(big, __shfl_xor(big, o));
    }
    double mean = 0.0, sd = 0.0;
    if (cnt > 0.0) {
        mean = s1 / cnt;
        sd = sqrt(fmax(s2 / cnt - mean * mean, 0.0));
        if (sd <= kGqaFlat * big) sd = 0.0;
    }
    return make_double2(mean, sd);
}

}  // namespace tri
