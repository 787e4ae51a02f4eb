// rans_encode.hip -- fused lane encoder: rANS64 per lane, then a decoupled
// look-back scan of lane sizes, the container header and the compaction of
// every lane's words, all in one launch.
//
// Coding rules (kompressor README "Why"/"Credits": CompressAI's 64-bit
// ryg_rans-style coder; torch_ans "Usage" table: rans64 = 64-bit state,
// 32-bit words, 16-bit frequencies; torch_ans "Low-level API Reference":
// indexed tables, coded range [offset, offset+len-2), zig-zag bypass):
//   REG(start, f):  if x >= f*2^47: spill low word, x >>= 32;
//                   x = floor(x/f)*2^16 + (x mod f) + start
//   BITS(b):        if x >= 2^59: spill low word, x >>= 32;  x = 16x + b
//   an escaped symbol is REG(escape slot), BITS(nb), BITS(g_0..g_{nb-1})
//   a lane's puts are applied last to first starting from x = 2^31.
//
// Mapping to gfx950: one lane of a wavefront owns one rANS lane, with its
// 64-bit state in a VGPR pair; the packed u16 CDF rows and row metadata are
// staged once per workgroup into LDS; a lane spills words backwards into its
// own scratch segment.  Waves take tickets in arrival order, publish their
// word total, look back over earlier tickets for their offset (no grid-wide
// barrier, no second launch), then write their header entries and copy
// their lanes' words into the contiguous container.
#include "rans_internal.hpp"

namespace rans {

namespace {

constexpr uint64_t kFlagAggregate = 1ull << 62;
constexpr uint64_t kFlagInclusive = 2ull << 62;
constexpr uint64_t kFlagValueMask = (1ull << 62) - 1;
constexpr uint32_t kSpinLimit = 1u << 26;

__device__ inline void record_error(WsHeader *hdr, int code)
{
    atomicCAS(&hdr->err, 0, code);
}

struct Spill {
    uint32_t *top;      // one past the lane's scratch segment
    uint32_t count;     // words spilled so far
    uint32_t cap;       // segment size (keeps 2 words for the final state)
    bool overflow;

    __device__ inline void put(uint32_t w)
    {
        if (count + 2 < cap)
            top[-1 - (int64_t)count] = w;
        else
            overflow = true;
        ++count;
    }
};

// q = floor(x / f), r = x mod f for x < f * 2^47, f in [1, 65535].
// The quotient estimate comes from one fp64 division; x/f < 2^47 and the
// relative error of (double)x / (double)f is below 2^-51, so the truncated
// estimate is within one of q and a single exact integer correction fixes it.
__device__ inline uint64_t reg_step(uint64_t x, uint32_t start, uint32_t f)
{
    double qd = (double)x / (double)f;
    uint64_t q = (uint64_t)qd;
    int64_t r = (int64_t)(x - q * (uint64_t)f);
    if (r < 0) {
        q -= 1;
        r += f;
    } else if (r >= (int64_t)f) {
        q += 1;
        r -= f;
    }
    return (q << kPrecision) + (uint64_t)r + start;
}

__device__ inline void put_reg(uint64_t &x, uint32_t start, uint32_t f, Spill &sp)
{
    if (x >= ((uint64_t)f << (63 - kPrecision))) {
        sp.put((uint32_t)x);
        x >>= 32;
    }
    x = reg_step(x, start, f);
}

__device__ inline void put_bits(uint64_t &x, uint32_t b, Spill &sp)
{
    if (x >= (1ull << (63 - kBypassBits))) {
        sp.put((uint32_t)x);
        x >>= 32;
    }
    x = (x << kBypassBits) | b;
}

__device__ inline uint32_t wave_inclusive_scan(uint32_t v, uint32_t lane)
{
    for (int off = 1; off < kWave; off <<= 1) {
        uint32_t o = __shfl_up(v, off, kWave);
        if (lane >= (uint32_t)off)
            v += o;
    }
    return v;
}

template <int TPB>
__global__ __launch_bounds__(TPB) void encode_kernel(EncodeArgs a)
{
    extern __shared__ __align__(16) uint8_t lds[];
    __shared__ int s_last;

    WsHeader *hdr = reinterpret_cast<WsHeader *>(a.ws);
    const uint8_t *tab = a.ws + ws_tables_offset();
    uint64_t *flags = reinterpret_cast<uint64_t *>(a.ws + ws_flags_offset());
    uint32_t *scratch = reinterpret_cast<uint32_t *>(a.ws + ws_scratch_offset(a.lanes));
    const uint32_t tid = threadIdx.x;
    const uint32_t lane = tid & (kWave - 1);
    const uint32_t L = a.lanes;
    const uint32_t nwork = (uint32_t)ws_flag_count(L);

    // ---- tables -> LDS -------------------------------------------------------
    int herr = 0;
    if (hdr->magic != kMagic || hdr->num_tables != (uint32_t)a.num_tables)
        herr = RANS_E_ARG;
    else if (!hdr->enc_ok)
        herr = RANS_E_TABLE_SIZE;
    const uint32_t K = (uint32_t)a.num_tables;
    const uint32_t nbytes = herr ? 0u : hdr->enc_bytes;
    {
        const uint4 *src = reinterpret_cast<const uint4 *>(tab);
        uint4 *dst = reinterpret_cast<uint4 *>(lds);
        for (uint32_t i = tid; i < nbytes / 16; i += TPB)
            dst[i] = src[i];
    }
    __syncthreads();
    const RowMeta *meta = reinterpret_cast<const RowMeta *>(lds);
    const uint16_t *cdf16 = reinterpret_cast<const uint16_t *>(lds + align_up(16ull * K, 16));
    int bad = 0;
    if (!herr)
        for (uint32_t r = tid; r < K; r += TPB)
            bad |= (meta[r].mv & kRowInvalid) ? 1 : 0;
    bad = __syncthreads_or(bad);
    if (!herr && bad)
        herr = RANS_E_TABLE;
    if (herr && blockIdx.x == 0 && tid == 0)
        record_error(hdr, herr);

    if (!herr) {
        // ---- ticket: which 64 lanes this wave codes ---------------------------
        uint32_t t = 0;
        if (lane == 0)
            t = atomicAdd(&hdr->ticket, 1u);
        t = __shfl(t, 0, kWave);
        if (t < nwork) {
            const uint32_t j = t * kWave + lane;
            uint32_t words = 0;
            uint32_t *seg_top = nullptr;
            int lerr = 0;
            if (j < L) {
                const uint64_t b = lane_begin(a.n, L, j);
                const uint64_t e = lane_begin(a.n, L, j + 1);
                Spill sp;
                sp.top = scratch + 2 * e + 4ull * (j + 1);
                sp.count = 0;
                sp.cap = (uint32_t)(2 * (e - b) + 4);
                sp.overflow = false;
                uint64_t x = kStateLow;
                for (uint64_t i = e; i > b;) {
                    --i;
                    const int32_t s = a.symbols[i];
                    int32_t r = a.indexes[i];
                    if ((uint32_t)r >= K) {
                        lerr = RANS_E_INDEX;
                        r = 0;
                    }
                    const RowMeta m = meta[r];
                    const uint32_t mv = m.mv;
                    const int64_t v = (int64_t)s - (int64_t)m.offset;
                    const bool esc = (uint64_t)v >= (uint64_t)mv;
                    const uint32_t slot = esc ? mv : (uint32_t)v;
                    const uint32_t start = cdf16[m.cdf_base + slot];
                    const uint32_t f = ((uint32_t)cdf16[m.cdf_base + slot + 1] - start) & 0xFFFFu;
                    if (esc) {
                        uint64_t raw = v < 0 ? (uint64_t)(-2 * v - 1) : (uint64_t)(2 * (v - (int64_t)mv));
                        if (raw >= (1ull << 31)) {
                            lerr = RANS_E_SYMBOL_RANGE;
                            raw = 0;
                        }
                        const uint32_t bits = raw ? 64u - (uint32_t)__clzll(raw) : 0u;
                        const uint32_t nb = (bits + kBypassBits - 1) / kBypassBits;
                        for (uint32_t g = nb; g-- > 0;)
                            put_bits(x, (uint32_t)(raw >> (kBypassBits * g)) & 15u, sp);
                        put_bits(x, nb, sp);
                    }
                    put_reg(x, start, f, sp);
                }
                if (sp.overflow) {
                    lerr = lerr ? lerr : RANS_E_CAPACITY;
                    sp.count = sp.cap - 2;
                }
                sp.top[-2 - (int64_t)sp.count] = (uint32_t)x;
                sp.top[-1 - (int64_t)sp.count] = (uint32_t)(x >> 32);
                words = sp.count + 2;
                seg_top = sp.top;
            }
            if (lerr)
                record_error(hdr, lerr);

            // ---- wave scan and look-back over earlier tickets ---------------------
            const uint32_t incl = wave_inclusive_scan(words, lane);
            const uint64_t agg = __shfl(incl, kWave - 1, kWave);
            uint64_t prefix = 0;
            if (lane == 0) {
                if (t == 0) {
                    __hip_atomic_store(&flags[t], kFlagInclusive | agg, __ATOMIC_RELEASE,
                                       __HIP_MEMORY_SCOPE_AGENT);
                } else {
                    __hip_atomic_store(&flags[t], kFlagAggregate | agg, __ATOMIC_RELEASE,
                                       __HIP_MEMORY_SCOPE_AGENT);
                    uint32_t k = t;
                    uint32_t spins = 0;
                    while (k > 0) {
                        const uint64_t fv = __hip_atomic_load(&flags[k - 1], __ATOMIC_ACQUIRE,
                                                              __HIP_MEMORY_SCOPE_AGENT);
                        if ((fv >> 62) == 0) {
                            if (++spins > kSpinLimit) {   // never expected: bail out, flag it
                                record_error(hdr, RANS_E_HIP);
                                break;
                            }
                            __builtin_amdgcn_s_sleep(1);
                            continue;
                        }
                        prefix += fv & kFlagValueMask;
                        if ((fv >> 62) == 2)
                            break;
                        --k;
                    }
                    __hip_atomic_store(&flags[t], kFlagInclusive | (prefix + agg), __ATOMIC_RELEASE,
                                       __HIP_MEMORY_SCOPE_AGENT);
                }
                if (t == nwork - 1) {
                    hdr->total_words = prefix + agg;
                    a.stream[0] = L;
                }
            }
            prefix = __shfl(prefix, 0, kWave);

            // ---- header entry and compaction --------------------------------------
            if (j < L) {
                const uint64_t end = prefix + incl;
                a.stream[1 + j] = (uint32_t)end;
                const uint64_t dst = 1ull + L + end - words;
                const uint32_t *src = seg_top - words;
                for (uint32_t k = 0; k < words; ++k)
                    if (dst + k < a.capacity)
                        a.stream[dst + k] = src[k];
            }
        }
    }

    // ---- completion: the last block publishes status and cleans up -------------
    __syncthreads();
    if (tid == 0) {
        __threadfence();
        const uint32_t old = atomicAdd(&hdr->done, 1u);
        s_last = (old == gridDim.x - 1) ? 1 : 0;
    }
    __syncthreads();
    if (s_last) {
        __threadfence();
        if (!herr)
            for (uint32_t k = tid; k < nwork; k += TPB)
                flags[k] = 0;
        if (tid == 0) {
            const uint64_t total = 1ull + L + hdr->total_words;
            int err = hdr->err;
            if (!err && total > a.capacity)
                err = RANS_E_CAPACITY;
            *a.status = err;
            *a.stream_words = herr ? 0ull : total;
            hdr->err = 0;
            hdr->ticket = 0;
            hdr->total_words = 0;
            hdr->done = 0;
            __threadfence();
        }
    }
}

template <int TPB>
hipError_t launch_encode_t(const EncodeArgs &a, hipStream_t s)
{
    static const hipError_t attr = hipFuncSetAttribute(
        reinterpret_cast<const void *>(&encode_kernel<TPB>),
        hipFuncAttributeMaxDynamicSharedMemorySize, (int)kTableBudget);
    if (attr != hipSuccess)
        return attr;
    const uint32_t blocks = (uint32_t)((a.lanes + TPB - 1) / TPB);
    hipLaunchKernelGGL(encode_kernel<TPB>, dim3(blocks), dim3(TPB), kTableBudget, s, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_encode(const EncodeArgs &a, hipStream_t s)
{
    const uint32_t t = coding_block_threads(a.lanes);
    if (t <= 256)
        return launch_encode_t<256>(a, s);
    if (t <= 512)
        return launch_encode_t<512>(a, s);
    return launch_encode_t<1024>(a, s);
}

}  // namespace rans
