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

constexpr int kRound = 8;   // positions per lane between memory phases

// Spilled words of one lane.  Word k of the lane (k-th spill) belongs at
// top[-1 - k] in global scratch; until the next memory phase it waits in the
// lane's LDS ring (kRingWords words), or is stored directly if the ring is full.
struct Spill {
    uint32_t *top;      // one past the lane's scratch segment
    uint32_t *ring;     // ring slot 0 of this lane (slots are `stride` words apart)
    uint32_t stride;    // threads per block
    uint32_t count;     // words spilled so far
    uint32_t flushed;   // words [0, flushed) are in global scratch (or stored directly)
    uint32_t cap;       // segment size (keeps 2 words for the final state)
    bool overflow;

    __device__ inline void put(uint32_t w)
    {
        if (count + 2 >= cap) {
            overflow = true;
        } else if (count - flushed < kRingWords) {
            ring[(count % kRingWords) * stride] = w;
        } else {
            top[-1 - (int64_t)count] = w;
        }
        ++count;
    }

    // Move the ring's words to global scratch.  Always eight stores (a fixed
    // count keeps the compiler's wait counts exact): slots without a word
    // write filler to not-yet-used positions of the lane's segment, which are
    // rewritten later by spills or the final state, or never copied out.
    __device__ inline void flush()
    {
        // words at or past cap - 2 were never kept (overflow, reported)
        const uint32_t upto = min(min(count, flushed + kRingWords), cap - 2);
#pragma unroll
        for (uint32_t k = 0; k < kRingWords; ++k) {
            const uint32_t idx = flushed + k;
            const uint32_t at = idx < upto ? idx : min(idx, cap - 1);
            top[-1 - (int64_t)at] = ring[(idx % kRingWords) * stride];
        }
        flushed = count;
    }
};

// Reciprocal of f in fp64 for the quotient estimate: the hardware estimate
// refined by two Newton-Raphson steps r <- r + r(1 - f r), which square the
// relative error each time (from about 2^-23 to far below the 2^-52 of the
// final rounding).
__device__ inline double reciprocal(uint32_t f)
{
    const double fd = (double)f;
    double r = __builtin_amdgcn_rcp(fd);
    double e = __builtin_fma(-fd, r, 1.0);
    r = __builtin_fma(r, e, r);
    e = __builtin_fma(-fd, r, 1.0);
    return __builtin_fma(r, e, r);
}

// x <- floor(x/f)*2^16 + (x mod f) + start, for x < f * 2^47.
// q = round(x * (1/f)) is read from the mantissa of fma(x, 1/f, 2^52); with
// x/f < 2^47 and a relative error below 2^-50 the estimate is floor(x/f) or
// one more, so one exact correction on the low 32 bits of x - q*f (which lie
// in [-f, f)) gives the true quotient and remainder.
__device__ inline uint64_t reg_step(uint64_t x, uint32_t start, uint32_t f, double rcp)
{
    const double xd = __builtin_fma((double)(uint32_t)(x >> 32), 4294967296.0,
                                    (double)(uint32_t)x);
    const double t = __builtin_fma(xd, rcp, 4503599627370496.0);   // 2^52
    uint64_t q = (uint64_t)__double_as_longlong(t) & ((1ull << 52) - 1);
    int32_t r = (int32_t)((uint32_t)x - (uint32_t)q * f);
    if (r < 0) {
        q -= 1;
        r += (int32_t)f;
    }
    return (q << kPrecision) + (uint32_t)r + start;
}

__device__ inline void put_reg(uint64_t &x, uint32_t start, uint32_t f, double rcp, Spill &sp)
{
    if (x >= ((uint64_t)f << (63 - kPrecision))) {
        sp.put((uint32_t)x);
        x >>= 32;
    }
    x = reg_step(x, start, f, rcp);
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

// The puts of one symbol, applied last to first; returns a status code.
__device__ __forceinline__ int encode_symbol(int32_t s, int32_t r, uint64_t &x, Spill &sp,
                                             const RowMeta *meta, const uint16_t *cdf16,
                                             uint32_t K)
{
    int err = 0;
    if ((uint32_t)r >= K) {
        err = RANS_E_INDEX;
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
            err = err ? err : RANS_E_SYMBOL_RANGE;
            raw = 0;
        }
        const uint32_t bits = raw ? 64u - (uint32_t)__clzll(raw) : 0u;
        const uint32_t nb = (bits + kBypassBits - 1) / kBypassBits;
        for (uint32_t g = nb; g-- > 0;)
            put_bits(x, (uint32_t)(raw >> (kBypassBits * g)) & 15u, sp);
        put_bits(x, nb, sp);
    }
    put_reg(x, start, f, reciprocal(f), sp);
    return err;
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
    stage_tables<TPB>(lds, tab, nbytes);
    __syncthreads();
    const RowMeta *meta = reinterpret_cast<const RowMeta *>(lds);
    const uint16_t *cdf16 = reinterpret_cast<const uint16_t *>(lds + align_up(16ull * K, 16));
    uint32_t *ring = reinterpret_cast<uint32_t *>(lds + kTableBudget) + tid;
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
                sp.ring = ring;
                sp.stride = TPB;
                sp.count = 0;
                sp.flushed = 0;
                sp.cap = (uint32_t)(2 * (e - b) + 4);
                sp.overflow = false;
                uint64_t x = kStateLow;
                const uint64_t nj = e - b;
                const uint64_t kl = nj ? nj - 1 : 0;     // last position offset
                // Positions are coded last to first.  Symbols and indexes of
                // round r+1 are requested in the memory phase before round r,
                // so they are one round old when the state chain reads them.
                // Two symbol/index buffers used in turn (no register copies
                // between rounds): a buffer is refilled in the memory phase right
                // after its round and read again two rounds later.  Every memory
                // phase issues the same global accesses in the same order (8
                // spill stores, 16 loads) and the prologue runs two such phases
                // too, so the compiler's wait counts only ever cover requests
                // that are at least a round old.  Empty lanes (n may be 0 with
                // null arrays) read a dummy word of the workspace header.
                const int32_t *syp = nj ? a.symbols : reinterpret_cast<const int32_t *>(hdr->pad0);
                const int32_t *ixp = nj ? a.indexes : reinterpret_cast<const int32_t *>(hdr->pad0);
                const uint64_t p_hi = nj ? e - 1 : 0;
                int32_t sa[kRound], ia[kRound], sb[kRound], ib[kRound];
                auto load_next = [&](int32_t (&sym)[kRound], int32_t (&idx)[kRound], uint64_t k) {
#pragma unroll
                    for (int u = 0; u < kRound; ++u) {
                        const uint64_t p = p_hi - min(k + u, kl);
                        sym[u] = syp[p];
                        idx[u] = ixp[p];
                    }
                    __builtin_amdgcn_sched_barrier(0);
                };
                auto round = [&](int32_t (&sym)[kRound], int32_t (&idx)[kRound], uint64_t k0) {
#pragma unroll
                    for (int u = 0; u < kRound; ++u) {
                        if (k0 + u < nj) {
                            const int ec = encode_symbol(sym[u], idx[u], x, sp, meta, cdf16, K);
                            lerr = lerr ? lerr : ec;
                        }
                    }
                    __builtin_amdgcn_sched_barrier(0);
                    // ---- memory phase ----
                    sp.flush();
                    __builtin_amdgcn_sched_barrier(0);
                    load_next(sym, idx, k0 + 2 * kRound);
                };
                // prologue: two phases of the same shape (the empty flushes write
                // filler to the lane's first spill slot, rewritten later)
                sp.flush();
                __builtin_amdgcn_sched_barrier(0);
                load_next(sa, ia, 0);
                sp.flush();
                __builtin_amdgcn_sched_barrier(0);
                load_next(sb, ib, kRound);
                // both rounds always run (positions past the lane are skipped
                // inside), so every path back to the loop head passes both phases
                for (uint64_t k0 = 0; k0 < nj; k0 += 2 * kRound) {
                    round(sa, ia, k0);
                    round(sb, ib, k0 + kRound);
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
                    a.stream[0] = L;
                    __hip_atomic_store(&hdr->total_words, prefix + agg, __ATOMIC_RELEASE,
                                       __HIP_MEMORY_SCOPE_AGENT);
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
    const uint32_t lds_bytes = coding_lds_bytes(TPB);
    static const hipError_t attr = hipFuncSetAttribute(
        reinterpret_cast<const void *>(&encode_kernel<TPB>),
        hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds_bytes);
    if (attr != hipSuccess)
        return attr;
    const uint32_t blocks = (uint32_t)((a.lanes + TPB - 1) / TPB);
    hipLaunchKernelGGL(encode_kernel<TPB>, dim3(blocks), dim3(TPB), lds_bytes, s, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_encode(const EncodeArgs &a, hipStream_t s)
{
    if (coding_block_threads(a.lanes) <= 256)
        return launch_encode_t<256>(a, s);
    return launch_encode_t<512>(a, s);
}

}  // namespace rans
