// rans_decode.hip -- lane decoder: one rANS64 state per wavefront lane,
// symbols read first to last, the symbol of each step found through the
// LDS bucket lookup (one 8-byte read in the common case) with a binary
// search over the LDS row as fallback.
//
// Decoding rules (the inverse of the puts in rans_encode.hip; decode reads
// the lane's words in order):
//   cum = x mod 2^16; slot s with cdf[s] <= cum < cdf[s+1];
//   x = f * (x >> 16) + cum - cdf[s]; if x < 2^31: x = (x << 32) | next word
//   escape slot -> 4-bit gets: count nb (15 = continue), then nb raw groups,
//   least significant first; odd raw -> -(raw>>1)-1, even -> (raw>>1)+mv
// (kompressor BENCHMARKS.md section 4 names the lookup as the decoder's cost:
// CompressAI scans the row linearly, kompressor binary-searches it; torch_ans
// "Usage" describes the inverse-CDF table keyed by the low state bits.)
// A lane must end at x = 2^31 with all of its words consumed, otherwise the
// call reports RANS_E_CORRUPT; reads never leave the lane's header extent.
//
// Memory schedule.  A lane works in rounds of kRound symbols.  Global memory
// is touched only between rounds, in straight-line code: the indexes of the
// round after next are requested, the finished round's symbols are stored,
// and kRefill stream words are requested for the lane's word ring in LDS.
// Every loaded register is first read one round after its load was issued,
// so the state chain inside a round never waits on global memory.  The ring
// (kRingWords words per lane) supplies renormalisation words; the next one
// is kept in a register.  Should a lane drain its ring within one round
// (long bypass runs), it reads the word straight from global memory.
#include "rans_internal.hpp"

namespace rans {

namespace {

constexpr int kRound = 8;        // symbols per lane between memory phases
constexpr uint32_t kRefill = 4;  // words requested per lane per memory phase

__device__ inline void record_error(WsHeader *hdr, int code)
{
    atomicCAS(&hdr->err, 0, code);
}

// Per-lane stream words: [0, count) of the lane, ring slots in LDS.
struct Words {
    const uint32_t *w;   // the lane's words in global memory
    uint32_t *ring;      // ring slot 0 of this lane (slots are `stride` words apart)
    uint32_t stride;     // threads per block
    uint32_t count;      // words in the lane
    uint32_t pos;        // next word to consume
    uint32_t filled;     // words [.., filled) have been written to the ring
    uint32_t next;       // ring word at pos (valid when pos < filled)

    __device__ inline uint32_t slot(uint32_t p) const { return (p % kRingWords) * stride; }

    // x < 2^31 after a step means the encoder spilled a word there.
    __device__ inline bool refill(uint64_t &x)
    {
        if (x < kStateLow) {
            if (pos >= count)
                return false;
            if (pos < filled) {
                x = (x << 32) | next;
            } else {
                // ring drained: read the word from global memory here, so the
                // wait for it stays on this rare path
                const uint32_t direct = w[pos];
                __builtin_amdgcn_s_waitcnt(0);
                x = (x << 32) | direct;
            }
            ++pos;
        }
        next = ring[slot(pos)];
        return true;
    }
};

// One decoding step of one lane; writes the symbol to `out`; returns a status.
__device__ __forceinline__ int decode_symbol(int32_t r, uint64_t &x, Words &wd,
                                             const RowMeta *meta, const uint16_t *cdf16,
                                             const uint64_t *lut, uint32_t shift, uint32_t K,
                                             int32_t &out)
{
    if ((uint32_t)r >= K)
        return RANS_E_INDEX;
    const RowMeta m = meta[r];
    const uint32_t cum = (uint32_t)x & (kTotal - 1);
    const uint64_t ent = lut[m.lut_base + (cum >> shift)];
    const uint32_t s0 = (uint32_t)ent & 0xFFFFu;
    const uint32_t s1 = (uint32_t)(ent >> 16) & 0xFFFFu;
    const uint32_t e1 = (uint32_t)(ent >> 32) & 0xFFFFu;
    uint32_t slot, start, f;
    if (cum >= s0 && cum <= e1) {
        const bool second = cum >= s1;
        slot = (uint32_t)(ent >> 48) + (second ? 1u : 0u);
        start = second ? s1 : s0;
        f = second ? e1 + 1 - s1 : s1 - s0;
    } else {
        // value(lo) <= cum < value(hi), with value(mv + 1) = 65536
        const uint16_t *row = cdf16 + m.cdf_base;
        uint32_t lo = 0, hi = m.mv + 1;
        while (hi - lo > 1) {
            const uint32_t mid = (lo + hi) >> 1;
            if ((uint32_t)row[mid] <= cum)
                lo = mid;
            else
                hi = mid;
        }
        slot = lo;
        start = row[lo];
        const uint32_t nxt = (lo == m.mv) ? kTotal : (uint32_t)row[lo + 1];
        f = nxt - start;
    }
    x = (uint64_t)f * (x >> kPrecision) + (cum - start);
    if (!wd.refill(x))
        return RANS_E_CORRUPT;
    int64_t value = slot;
    if (slot == m.mv) {
        uint32_t t = (uint32_t)x & 15u;
        x >>= kBypassBits;
        bool ok = wd.refill(x);
        uint32_t nb = t;
        while (ok && t == 15u && nb <= 8u) {
            t = (uint32_t)x & 15u;
            x >>= kBypassBits;
            ok = wd.refill(x);
            nb += t;
        }
        uint64_t raw = 0;
        if (ok && nb <= 8u) {
            for (uint32_t g = 0; g < nb && ok; ++g) {
                raw |= (uint64_t)((uint32_t)x & 15u) << (kBypassBits * g);
                x >>= kBypassBits;
                ok = wd.refill(x);
            }
        }
        if (!ok || nb > 8u || raw >= (1ull << 31))
            return RANS_E_CORRUPT;
        value = (raw & 1) ? -(int64_t)(raw >> 1) - 1 : (int64_t)(raw >> 1) + m.mv;
    }
    const int64_t sym = value + m.offset;
    if (sym < INT32_MIN || sym > INT32_MAX)
        return RANS_E_CORRUPT;
    out = (int32_t)sym;
    return 0;
}

template <int TPB>
__global__ __launch_bounds__(TPB) void decode_kernel(DecodeArgs a)
{
    extern __shared__ __align__(16) uint8_t lds[];
    __shared__ int s_last;

    WsHeader *hdr = reinterpret_cast<WsHeader *>(a.ws);
    const uint8_t *tab = a.ws + ws_tables_offset();
    const uint32_t tid = threadIdx.x;
    const uint32_t L = a.lanes;

    int herr = 0;
    if (hdr->magic != kMagic || hdr->num_tables != (uint32_t)a.num_tables)
        herr = RANS_E_ARG;
    else if (!hdr->dec_ok)
        herr = RANS_E_TABLE_SIZE;
    const uint32_t K = (uint32_t)a.num_tables;
    const uint32_t nbytes = herr ? 0u : hdr->dec_bytes;
    const uint32_t q = hdr->lut_q;
    stage_tables<TPB>(lds, tab, nbytes);
    __syncthreads();
    const RowMeta *meta = reinterpret_cast<const RowMeta *>(lds);
    const uint32_t meta_bytes = (uint32_t)align_up(16ull * K, 16);
    const uint16_t *cdf16 = reinterpret_cast<const uint16_t *>(lds + meta_bytes);
    const uint64_t *lut = reinterpret_cast<const uint64_t *>(
        lds + meta_bytes + align_up(2ull * hdr->total_len, 16));
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

    const uint32_t j = blockIdx.x * TPB + tid;
    if (!herr && j < L) {
        int lerr = 0;
        const uint64_t beg_w = j ? a.stream[j] : 0u;
        const uint64_t end_w = a.stream[1 + j];
        if (a.stream[0] != L || end_w < beg_w + 2 || 1ull + L + end_w > a.capacity) {
            lerr = RANS_E_CORRUPT;
        } else {
            Words wd;
            wd.w = a.stream + 1 + L + beg_w;
            wd.ring = ring;
            wd.stride = TPB;
            wd.count = (uint32_t)(end_w - beg_w);
            const uint32_t last_w = wd.count - 1;
            uint64_t x = (uint64_t)wd.w[0] | ((uint64_t)wd.w[1] << 32);
            // first ring fill: words [2, 2 + kRingWords)
            {
                uint32_t v[kRingWords];
#pragma unroll
                for (uint32_t k = 0; k < kRingWords; ++k)
                    v[k] = wd.w[min(2 + k, last_w)];
#pragma unroll
                for (uint32_t k = 0; k < kRingWords; ++k)
                    ring[((2 + k) % kRingWords) * TPB] = v[k];
            }
            wd.pos = 2;
            wd.filled = min(wd.count, 2u + kRingWords);
            wd.next = ring[wd.slot(2)];
            uint32_t pend[kRefill];
            uint32_t pend_at = wd.filled;

            const uint64_t b = lane_begin(a.n, L, j);
            const uint64_t e = lane_begin(a.n, L, j + 1);
            const uint64_t last_i = e > b ? e - 1 : b;
            const uint32_t shift = kPrecision - q;
            // Two index buffers used in turn (no register copies between rounds):
            // a buffer is refilled in the memory phase right after its round
            // and read again two rounds later.  Every memory phase issues the
            // same global accesses in the same order (8 stores, 8 index loads,
            // kRefill word loads), and the prologue runs two such phases too, so
            // the compiler's wait counts only ever cover requests that are at
            // least a round old.  Empty lanes (n may be 0 with null arrays) use
            // a dummy word of the workspace header instead.
            const bool any = e > b;
            const int32_t *ixp = any ? a.indexes : reinterpret_cast<const int32_t *>(hdr->pad0);
            int32_t *sdp = any ? a.symbols : reinterpret_cast<int32_t *>(hdr->pad0);
            const uint64_t ix0 = any ? b : 0, ixl = any ? last_i : 0;
            int32_t ia[kRound], ib[kRound], out[kRound];
#pragma unroll
            for (int u = 0; u < kRound; ++u)
                out[u] = 0;
            // last to first with clamped positions: filler stores to the lane's
            // last position precede its true value
            // (a phase after the lane's last symbol stores to a dummy word)
            int32_t *dummy = reinterpret_cast<int32_t *>(hdr->pad0);
            auto store_out = [&](uint64_t i0) {
                int32_t *base = i0 < e ? sdp : dummy;
                const uint64_t lim = i0 < e ? ixl : 0;
#pragma unroll
                for (int u = kRound - 1; u >= 0; --u)
                    base[min(i0 + u, lim)] = out[u];
            };
            auto load_next = [&](int32_t (&idx)[kRound], uint64_t ip) {
#pragma unroll
                for (int u = 0; u < kRound; ++u)
                    idx[u] = ixp[min(ip + u, ixl)];
#pragma unroll
                for (uint32_t k = 0; k < kRefill; ++k)
                    pend[k] = wd.w[min(wd.filled + k, last_w)];
                pend_at = wd.filled;
                __builtin_amdgcn_sched_barrier(0);
            };
            auto ring_refill = [&]() {
                if (pend_at == wd.filled && wd.filled + kRefill <= wd.pos + kRingWords) {
#pragma unroll
                    for (uint32_t k = 0; k < kRefill; ++k)
                        ring[((wd.filled + k) % kRingWords) * TPB] = pend[k];
                    wd.filled = min(wd.count, wd.filled + kRefill);
                }
                if (wd.filled < wd.pos)   // the lane outran its ring via direct reads
                    wd.filled = wd.pos;
                wd.next = ring[wd.slot(wd.pos)];
            };
            auto round = [&](int32_t (&idx)[kRound], uint64_t i0) {
#pragma unroll
                for (int u = 0; u < kRound; ++u) {
                    out[u] = 0;
                    if (i0 + u < e && !lerr)
                        lerr = decode_symbol(idx[u], x, wd, meta, cdf16, lut, shift, K, out[u]);
                }
                __builtin_amdgcn_sched_barrier(0);
                // ---- memory phase ----
                ring_refill();
                store_out(i0);
                __builtin_amdgcn_sched_barrier(0);
                load_next(idx, i0 + 2 * kRound);
            };
            // prologue: two phases of the same shape (zeros go to the lane's
            // first positions and are overwritten by the true symbols later)
            store_out(ix0);
            __builtin_amdgcn_sched_barrier(0);
            load_next(ia, ix0);
            store_out(ix0);
            __builtin_amdgcn_sched_barrier(0);
            load_next(ib, ix0 + kRound);
            // both rounds always run (symbols past the lane end are skipped inside),
            // so every path back to the loop head passes both memory phases
            for (uint64_t i0 = b; i0 < e && !lerr; i0 += 2 * kRound) {
                round(ia, i0);
                round(ib, i0 + kRound);
            }
            if (!lerr && (x != kStateLow || wd.pos != wd.count))
                lerr = RANS_E_CORRUPT;
        }
        if (lerr)
            record_error(hdr, lerr);
    }

    // ---- completion: the last block publishes status and cleans up -------------
    __syncthreads();
    if (tid == 0) {
        __threadfence();
        const uint32_t old = atomicAdd(&hdr->done, 1u);
        s_last = (old == gridDim.x - 1) ? 1 : 0;
    }
    __syncthreads();
    if (s_last && tid == 0) {
        __threadfence();
        *a.status = hdr->err;
        hdr->err = 0;
        hdr->done = 0;
        __threadfence();
    }
}

template <int TPB>
hipError_t launch_decode_t(const DecodeArgs &a, hipStream_t s)
{
    const uint32_t lds_bytes = coding_lds_bytes(TPB);
    static const hipError_t attr = hipFuncSetAttribute(
        reinterpret_cast<const void *>(&decode_kernel<TPB>),
        hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds_bytes);
    if (attr != hipSuccess)
        return attr;
    const uint32_t blocks = (uint32_t)((a.lanes + TPB - 1) / TPB);
    hipLaunchKernelGGL(decode_kernel<TPB>, dim3(blocks), dim3(TPB), lds_bytes, s, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_decode(const DecodeArgs &a, hipStream_t s)
{
    if (coding_block_threads(a.lanes) <= 256)
        return launch_decode_t<256>(a, s);
    return launch_decode_t<512>(a, s);
}

}  // namespace rans
