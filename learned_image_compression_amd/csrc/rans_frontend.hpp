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

// Cells of the optional index lookup table: the non-negative floats split by
// their bits 30..19 (exponent and top four mantissa bits), 4096 cells.
constexpr uint32_t kScaleLutShift = 19;
constexpr uint32_t kScaleLutCells = 1u << (31 - kScaleLutShift);

// The scale table in LDS.  When its first K - 1 entries are non-decreasing
// the counted set is a suffix of them, and the index is a branch-free binary
// search of fixed trip count; otherwise the count is taken entry by entry.
// A sorted table with no negative first entry may also carry `lut`: cell c
// holds #{k < K - 1 : table[k] < lo_c}, lo_c the smallest float of the cell,
// so the index of a scale in cell c is lut[c] plus the entries in [lo_c, s),
// a forward scan of a step or two when cells are finer than the table (any
// negative scale counts nothing, NaN gives K - 1).
struct ScaleTable {
    const float *t;   // LDS
    int32_t K;
    int32_t steps;    // highest power of two <= K - 1 (0 when K == 1)
    bool sorted;
    const uint16_t *lut;   // LDS, or null

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
        if (lut) {
            int32_t j[N];
#pragma unroll
            for (int u = 0; u < N; ++u) {
                const uint32_t b = __float_as_uint(s[u]);
                // a scale with the sign bit set lies at or below every entry
                // (all are >= -0.0 here): it counts nothing
                j[u] = (b >> 31) ? 0 : (int32_t)lut[b >> kScaleLutShift];
            }
            bool go;
            do {
                go = false;
#pragma unroll
                for (int u = 0; u < N; ++u) {
                    const bool c = j[u] < m && t[min(j[u], m - 1)] < s[u];
                    j[u] += c ? 1 : 0;
                    go = go | c;
                }
            } while (__any(go));
#pragma unroll
            for (int u = 0; u < N; ++u)
                out[u] = s[u] != s[u] ? m : j[u];
            return;
        }
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
    // the counted entries must be non-decreasing and none NaN (a NaN entry
    // is neither below nor at or above a scale, so no search can count it)
    bool unsorted = false;
    for (int32_t k = threadIdx.x; k + 1 < K; k += TPB)
        unsorted |= !(lds[k] == lds[k]) || (k + 2 < K && !(lds[k] <= lds[k + 1]));
    ScaleTable st;
    st.t = lds;
    st.K = K;
    st.sorted = !block_or(flag, unsorted);
    st.lut = nullptr;
    int32_t p = 1;
    while (2 * p <= K - 1)
        p *= 2;
    st.steps = K > 1 ? p : 0;
    return st;
}

// Fill the index lookup table of a staged scale table when it qualifies
// (sorted, first entry not negative); `lut` holds kScaleLutCells entries in
// LDS.  Every thread of the block must call this.
template <int TPB>
__device__ inline void build_scale_lut(ScaleTable &st, uint16_t *lut)
{
    if (!st.sorted || st.K < 2 || st.t[0] < 0.0f)
        return;   // (the same decision in every thread)
    for (uint32_t c = threadIdx.x; c < kScaleLutCells; c += TPB) {
        const float lo = __uint_as_float(c << kScaleLutShift);
        // #{k < K - 1 : t[k] < lo}: the binary search of index()
        int32_t j = 0;
        for (int32_t step = st.steps; step > 0; step >>= 1)
            if (j + step <= st.K - 1 && st.t[j + step - 1] < lo)
                j += step;
        lut[c] = (uint16_t)j;
    }
    __syncthreads();
    st.lut = lut;
}

}  // namespace rans
