// rans_frontend.hpp -- the per-position arithmetic of the mean-scale front
// end (kompressor BENCHMARKS.md, sections 3 and 4: the codec derives each
// position's symbol from the latent and its predicted mean, and its table
// index from the predicted scale, on the GPU, before the coder runs).
// Shared by the stand-alone front-end kernel and the interleaved encoder that
// fuses it.  Readings:
//   symbol = round-half-even(y - mean) in single precision, saturated to
//            int32 (NaN -> INT32_MIN), so a value int32 cannot hold reaches
//            the coder as one it refuses as out of range;
//   index  = (K - 1) - #{k < K - 1 : scale <= table[k]}: the first table
//            scale at or above the predicted scale, K - 1 when there is none
//            or the scale is NaN.
#pragma once

#include "rans_internal.hpp"

namespace rans {

__device__ inline int32_t saturate_round(float d)
{
    if (d != d)
        return INT32_MIN;
    const float r = rintf(d);   // half to even
    if (r >= 2147483648.0f)
        return INT32_MAX;
    if (r < -2147483648.0f)
        return INT32_MIN;
    return (int32_t)r;
}

// The scale table in LDS.  When its first K - 1 entries are non-decreasing
// the counted set is a suffix of them, and the index is a branch-free binary
// search of fixed trip count; otherwise the count is taken entry by entry.
struct ScaleTable {
    const float *t;   // LDS
    int32_t K;
    int32_t steps;    // highest power of two <= K - 1 (0 when K == 1)
    bool sorted;

    __device__ int32_t index(float s) const
    {
        const int32_t m = K - 1;   // slots counted against
        if (sorted) {
            // j = #{k < m : table[k] < s} = first k with s <= table[k]
            int32_t j = 0;
            for (int32_t step = steps; step > 0; step >>= 1)
                if (j + step <= m && t[j + step - 1] < s)
                    j += step;
            return s != s ? m : j;
        }
        int32_t idx = m;
        for (int32_t k = 0; k < m; ++k)
            idx -= s <= t[k] ? 1 : 0;
        return idx;
    }

    // index() of N scales at once, the binary search taken level by level
    // across them, so that their dependent LDS reads overlap.
    template <int N>
    __device__ inline void index_n(const float (&s)[N], int32_t (&out)[N]) const
    {
        const int32_t m = K - 1;
        if (sorted) {
            int32_t j[N];
#pragma unroll
            for (int u = 0; u < N; ++u)
                j[u] = 0;
            for (int32_t step = steps; step > 0; step >>= 1) {
#pragma unroll
                for (int u = 0; u < N; ++u) {
                    const int32_t c = j[u] + step;
                    const bool up = c <= m && t[min(c, m) - 1] < s[u];
                    j[u] = up ? c : j[u];
                }
            }
#pragma unroll
            for (int u = 0; u < N; ++u)
                out[u] = s[u] != s[u] ? m : j[u];
        } else {
#pragma unroll
            for (int u = 0; u < N; ++u)
                out[u] = index(s[u]);
        }
    }
};

// Stage K scale-table entries into LDS and classify the table.  `flag` is a
// zeroed LDS word of the block (left zeroed).  Every thread of the block
// must call this.
template <int TPB>
__device__ inline ScaleTable stage_scale_table(const float *table, int32_t K, float *lds,
                                               uint32_t *flag)
{
    for (int32_t k = threadIdx.x; k < K; k += TPB)
        lds[k] = table[k];
    __syncthreads();
    bool unsorted = false;
    for (int32_t k = threadIdx.x; k + 2 < K; k += TPB)
        unsorted |= !(lds[k] <= lds[k + 1]);   // NaN entries count as unsorted
    ScaleTable st;
    st.t = lds;
    st.K = K;
    st.sorted = !block_or(flag, unsorted);
    int32_t p = 1;
    while (2 * p <= K - 1)
        p *= 2;
    st.steps = K > 1 ? p : 0;
    return st;
}

}  // namespace rans
