// rans_tables.hip -- 16-bit quantised CDF rows built on the device: from pmf
// rows, or as discretised zero-mean Gaussians of given scales.  One
// workgroup per row.
//
// The coder consumes rows of alphabet + escape slot + terminal entry
// (torch_ans 0.3.0, "Range limit" under rans*_push) and builds them from
// batched pmfs itself (torch_ans "Parameter Setup" and "Other Features";
// "Performance Tuning", item 6: init_params rebuilds the quantised CDFs and
// the lookup table); the 1080p y latent uses 64 Gaussian rows of at most 3133
// entries (kompressor BENCHMARKS.md, section 4).
//
// Quantisation: f_k = max(1, round-half-even(p_k * 2^16)); the sum is then
// brought to exactly 2^16 as if one unit at a time were taken from (surplus)
// or given to (deficit) the currently largest frequency, the lowest slot
// among equals.  The kernel does not loop over units; it uses that loop's
// closed form.  A surplus E never touches a frequency at some level while one
// above it remains, and at each level it lowers the slots in slot order, so
// the result is: every frequency above T becomes T, T the smallest level
// whose removal sum(max(0, f - T)) is at most E, and the remaining
// E - removal units come one each from the lowest slots at T.  A deficit goes
// whole to the first largest slot, which stays the largest after each unit.
//
// Gaussian row of scale s (half-width c = ceil(s * z) for a standard-normal
// quantile z): slot k = 0..2c holds v = k - c with mass
// Phi((v + 1/2) / s) - Phi((v - 1/2) / s), the escape slot the mass of both
// tails, 2 Phi(-(c + 1/2) / s), with Phi(x) = erfc(-x / sqrt 2) / 2 in double
// precision; offset -c, length 2c + 3, entries past the length 2^16.
#include "rans_internal.hpp"

#pragma clang fp contract(off)

namespace rans {
namespace {

// one workgroup per row, so the widest row sets the time: 16 waves share it
constexpr int kTabThreads = 1024;
constexpr int kTabWaves = kTabThreads / kWave;
constexpr int kMaxRowSlots = RANS_MAX_STRIDE - 1;   // pmf entries of one row (cdf has one more)

__device__ inline double std_normal_cdf(double x)
{
    return 0.5 * erfc(-x * 0.70710678118654752440);
}

__device__ inline uint32_t block_sum(uint32_t v, uint32_t *red)
{
    for (int o = kWave / 2; o > 0; o >>= 1)
        v += __shfl_xor(v, o);
    __syncthreads();   // red may still be read by the previous reduction
    if ((threadIdx.x & (kWave - 1)) == 0)
        red[threadIdx.x / kWave] = v;
    __syncthreads();
    uint32_t t = 0;
    for (int i = 0; i < kTabWaves; ++i)
        t += red[i];
    return t;
}

// exclusive scan of v in thread order
__device__ inline uint32_t block_exclusive_scan(uint32_t v, uint32_t *red)
{
    const int lane = threadIdx.x & (kWave - 1);
    uint32_t inc = v;
    for (int o = 1; o < kWave; o <<= 1) {
        const uint32_t u = __shfl_up(inc, o);
        if (lane >= o)
            inc += u;
    }
    __syncthreads();
    if (lane == kWave - 1)
        red[threadIdx.x / kWave] = inc;
    __syncthreads();
    uint32_t before = 0;
    for (int i = 0; i < (int)(threadIdx.x / kWave); ++i)
        before += red[i];
    return before + inc - v;
}

__device__ inline unsigned long long block_max(unsigned long long v, unsigned long long *red)
{
    for (int o = kWave / 2; o > 0; o >>= 1) {
        const unsigned long long u = __shfl_xor(v, o);
        v = u > v ? u : v;
    }
    __syncthreads();
    if ((threadIdx.x & (kWave - 1)) == 0)
        red[threadIdx.x / kWave] = v;
    __syncthreads();
    unsigned long long t = 0;
    for (int i = 0; i < kTabWaves; ++i)
        t = red[i] > t ? red[i] : t;
    return t;
}

__global__ __launch_bounds__(kTabThreads) void table_rows_kernel(TableArgs a)
{
    __shared__ int32_t f[kMaxRowSlots];
    __shared__ uint32_t red[kTabWaves];
    __shared__ unsigned long long red64[kTabWaves];
    const int r = blockIdx.x;
    const int tid = threadIdx.x;
    int32_t *row = a.cdf + (int64_t)r * a.cdf_stride;

    // ---- row size (the same for every thread of the block) ------------------
    const bool gauss = a.scales != nullptr;
    double s = 0.0;
    int32_t c = 0;
    int m;
    bool ok;
    if (gauss) {
        s = a.scales[r];
        ok = s > 0.0;   // false for NaN
        const double cw = ok ? ceil(s * a.tail_z) : 0.0;
        ok = ok && 2.0 * cw + 3.0 <= (double)a.cdf_stride;
        c = ok ? (int32_t)cw : 0;
        m = 2 * c + 2;   // 2c + 1 symbols and the escape slot
    } else {
        m = a.pmf_lengths[r];
        ok = m >= 2 && m <= a.pmf_stride && m + 1 <= a.cdf_stride;
    }
    if (!ok) {
        if (tid == 0) {
            a.status[r] = RANS_E_TABLE;
            a.lengths[r] = 0;
        }
        return;
    }

    // ---- rounded frequencies, raised to 1 ------------------------------------
    // Gaussian: slot k's lower bin edge is Phi((k - c - 1/2) / s) and its
    // upper edge the lower edge of slot k + 1, taken from the next lane (a
    // wave's last lane evaluates its own); k - c +- 1/2 are exact, so both
    // are the same doubles as Phi((v +- 1/2) / s).  Slot m - 1 (the escape)
    // supplies the top edge of slot m - 2 and holds the two tails itself.
    uint32_t bad = 0;
    const int lane = tid & (kWave - 1);
    for (int k0 = 0; k0 < m; k0 += kTabThreads) {   // the same trip count in every lane
        const int k = k0 + tid;
        double p = 0.0;
        if (!gauss) {
            if (k < m)
                p = a.pmf[(int64_t)r * a.pmf_stride + k];
        } else {
            const double lo = k < m ? std_normal_cdf(((double)(k - c) - 0.5) / s) : 0.0;
            double hi = __shfl_down(lo, 1);
            if (lane == kWave - 1 && k + 1 < m)
                hi = std_normal_cdf(((double)(k + 1 - c) - 0.5) / s);
            p = k == m - 1 ? 2.0 * std_normal_cdf(-((double)c + 0.5) / s) : hi - lo;
        }
        if (k >= m)
            continue;
        if (!(p >= 0.0 && p <= 1.0)) {
            bad = 1;
            p = 0.0;
        }
        const int32_t q = (int32_t)rint(p * 65536.0);   // half to even
        f[k] = q < 1 ? 1 : q;
    }
    if (block_sum(bad, red)) {
        if (tid == 0) {
            a.status[r] = RANS_E_TABLE;
            a.lengths[r] = 0;
        }
        return;
    }

    // ---- bring the sum to 2^16 (thread t owns slots [k0, k1)) ---------------
    const int per = (m + kTabThreads - 1) / kTabThreads;
    const int k0 = min(m, tid * per), k1 = min(m, k0 + per);
    uint32_t sum = 0;
    int32_t lmax = 0;
    int lk = k0;
    for (int k = k0; k < k1; ++k) {
        sum += (uint32_t)f[k];
        if (f[k] > lmax) {
            lmax = f[k];
            lk = k;
        }
    }
    // at most 16383 slots of at most 65536: the sum fits 31 bits
    const int32_t excess = (int32_t)block_sum(sum, red) - 65536;
    if (excess != 0) {
        // the largest frequency, and its first slot
        const unsigned long long key = ((unsigned long long)(uint32_t)lmax << 32) |
                                       (unsigned long long)(0xFFFFFFFFu - (uint32_t)lk);
        const unsigned long long best = block_max(key, red64);
        if (excess < 0) {
            if (tid == 0)
                f[0xFFFFFFFFu - (uint32_t)best] -= excess;
        } else {
            // smallest level T with sum(max(0, f - T)) <= excess; T = 1 removes
            // S - m >= excess, so T exists in [1, max]
            int lo = 1, hi = (int)(best >> 32);
            while (lo < hi) {
                const int mid = (lo + hi) >> 1;
                uint32_t cost = 0;
                for (int k = k0; k < k1; ++k)
                    cost += f[k] > mid ? (uint32_t)(f[k] - mid) : 0u;
                if (block_sum(cost, red) <= (uint32_t)excess)
                    hi = mid;
                else
                    lo = mid + 1;
            }
            const int T = lo;
            uint32_t cost = 0, at = 0;
            for (int k = k0; k < k1; ++k) {
                cost += f[k] > T ? (uint32_t)(f[k] - T) : 0u;
                at += f[k] >= T ? 1u : 0u;
            }
            const uint32_t rest = (uint32_t)excess - block_sum(cost, red);
            // rest > 0 only when T >= 2 (T = 1 removes exactly the surplus)
            uint32_t rank = block_exclusive_scan(at, red);
            for (int k = k0; k < k1; ++k)
                if (f[k] >= T) {
                    f[k] = rank < rest ? T - 1 : T;
                    ++rank;
                }
        }
        __syncthreads();
    }

    // ---- cumulative frequencies, then the row (coalesced) --------------------
    sum = 0;
    for (int k = k0; k < k1; ++k)
        sum += (uint32_t)f[k];
    uint32_t run = block_exclusive_scan(sum, red);
    for (int k = k0; k < k1; ++k) {
        run += (uint32_t)f[k];
        f[k] = (int32_t)run;   // now cdf entry k + 1
    }
    __syncthreads();
    for (int k = tid; k < a.cdf_stride; k += kTabThreads)
        row[k] = k == 0 ? 0 : (k <= m ? f[k - 1] : 65536);
    if (tid == 0) {
        a.lengths[r] = m + 1;
        if (gauss)
            a.offsets[r] = -c;
        a.status[r] = RANS_OK;
    }
}

}  // namespace

hipError_t launch_table_rows(const TableArgs &a, hipStream_t s)
{
    hipLaunchKernelGGL(table_rows_kernel, dim3(a.num_tables), dim3(kTabThreads), 0, s, a);
    return hipGetLastError();
}

}  // namespace rans
