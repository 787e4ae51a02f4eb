// rans_decode.hip -- lane decoder: one rANS64 state per wavefront lane,
// symbols read first to last, the symbol of each step found through the
// bucket lookup (the bucket's first slot, then one 8-byte read of the next
// slot starts) with a short search of the bucket's slots as fallback.
//
// Decoding rules (the inverse of the puts in rans_encode.hip; decode reads
// the lane's words in order):
//   cum = x mod 2^16; slot s with cdf[s] <= cum < cdf[s+1];
//   x = f * (x >> 16) + cum - cdf[s]; if x < 2^31: x = (x << 32) | next word
//   escape slot -> 4-bit gets: count nb, then nb raw groups, least
//   significant first; odd raw -> -(raw>>1)-1, even -> (raw>>1)+mv
// (kompressor BENCHMARKS.md section 4 names the lookup as the decoder's cost:
// CompressAI scans the row linearly, kompressor binary-searches it; torch_ans
// "Usage" describes the inverse-CDF table keyed by the low state bits.)
// A lane must end at x = 2^31 with all of its words consumed, otherwise the
// call reports RANS_E_CORRUPT; reads never leave the lane's header extent.
//
// The lane count comes from the container's first word (a stream carries its
// own length bookkeeping: torch_ans "Parallel ANS stream"), so the launch
// cannot depend on it: the grid is at most one block per CU, and each block
// loops over the work units the lane count gives it.
//
// Per-symbol work.  The common step -- cum within three slots of the
// bucket's first slot, an ordinary slot, the renormalisation word already in
// the LDS ring -- is straight-line code.  Two ways to handle the rest:
//  * waves of few lanes (the latency-bound regime) decode a whole round of
//    kRound symbols speculatively, with no branch at all, and collect in one
//    flag whether any step left the common case; only then (rarely) do the
//    lanes concerned redo the round step by step;
//  * waves of many lanes, where some lane leaves the common case in most
//    rounds, commit each step at once, and lanes outside it redo that step
//    on the slow path, entered only when some lane of the wave needs it.
//
// Memory schedule.  A lane works in rounds of kRound symbols.  Global memory
// is touched only between rounds: the indexes of the round after next and
// kRefill stream words for the lane's word ring in LDS are requested, then
// the finished round's symbols are stored.  Every loaded register is first
// read two rounds after its load was issued (a round takes about as long as
// a loaded memory round trip), so the state chain inside a round never waits
// on global memory.  Should a lane drain its ring (long bypass runs), it
// reads the word straight from global memory.
#include <type_traits>

#include "rans_lookup.hpp"

namespace rans {

namespace {

constexpr int kRound = 8;        // symbols per lane between memory phases
constexpr uint32_t kRefill = 4;  // words requested per lane per memory phase
constexpr uint32_t kNoStore = 0x80000000u;   // a buffer offset past every buffer
constexpr uint32_t kMaxDecWaves = 2048;      // lanes are spread over at most this many waves
constexpr uint32_t kDecTPB = 8 * kWave;      // one block shape: eight waves, two per SIMD
constexpr uint32_t kSpecLanes = 4;           // waves of at most this many lanes decode speculatively

__device__ inline void record_error(WsHeader *hdr, int code)
{
    atomicCAS(&hdr->err, 0, code);
}

// Per-lane stream words: [0, count) of the lane, ring slots in LDS.
template <int TPB>
struct Words {
    const uint32_t *w;   // the lane's words in global memory
    uint32_t ring;       // LDS address of this lane's ring slot 0 (slots are TPB words apart)
    uint32_t count;      // words in the lane
    uint32_t pos;        // next word to consume
    uint32_t filled;     // words [.., filled) have been written to the ring
    uint32_t next;       // ring word at pos (valid when pos < filled)

    __device__ inline uint32_t slot(uint32_t p) const { return ring | ((p % kDecRing) * (4 * TPB)); }
    __device__ inline uint32_t at(uint32_t p) const { return lds_load<uint32_t>(slot(p)); }
    __device__ inline void put(uint32_t p, uint32_t v) const { lds_store<uint32_t>(slot(p), v); }

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
        next = at(pos);
        return true;
    }
};


template <class Tab>
__device__ inline uint32_t cdfm1_at(const Tab &tab, const RowMeta &m, uint32_t k)
{
    return tab.template load<uint16_t>(m.base + 2 * k);
}

// Slow step of one lane, from the state before the step.  `slot`, `f` and
// `rr` come from the lookup window; `beyond` says cum lies past it.  The
// lanes in here are few, so the code keeps to straight-line work with a
// handful of wave-uniform branches:
//  * past the window, the search walks the bucket's slots up to first[b+1]
//    (the escape slot mv for the last bucket), eight slot starts per LDS
//    round trip;
//  * the renormalisation word and an escape's groups need at most three
//    words (after the step x >= 2^31, and nb <= 8 groups of 4 bits follow),
//    read from the ring when it holds them, else on the checked path;
//  * out-of-range values and bad indexes are reported.
// Writes the symbol to `out`; returns a status.
template <class WordsT, class Tab>
__device__ __forceinline__ int decode_slow(int32_t r, const RowMeta &m, uint32_t bucket,
                                           bool beyond, uint32_t slot, uint32_t f, uint32_t rr,
                                           uint64_t &x, WordsT &wd, const DecTables &t,
                                           const Tab &tab, int32_t &out)
{
    if ((uint32_t)r >= t.K)
        return RANS_E_INDEX;
    const uint32_t mv = m.mvf & 0xFFFFu;
    const uint32_t cum = (uint32_t)x & (kTotal - 1);
    if (__ballot(beyond) != 0) {
        uint32_t lo = slot;   // value(lo) <= cum
        const uint32_t hi = (bucket + 1 < (1u << t.q))
                                ? tab.template load<uint16_t>((m.lut & ~kRowInvalid) + 2 * (bucket + 1))
                                : mv;
        // the slot is the last k in [lo, hi] with value(k) <= cum
        uint32_t c;
        do {
            c = 0;
#pragma unroll
            for (uint32_t k = 1; k <= 8; ++k) {
                const uint32_t v = cdfm1_at(tab, m, min(lo + k, hi));
                c += (lo + k <= hi && cum > v) ? 1u : 0u;
            }
            lo += c;
        } while (c == 8 && lo < hi);
        const uint32_t sm1 = cdfm1_at(tab, m, lo), em1 = cdfm1_at(tab, m, lo + 1);
        if (beyond) {
            slot = lo;
            f = (em1 - sm1) & 0xFFFFu;
            rr = (cum - sm1 - 1) & 0xFFFFu;
        }
    }
    x = (uint64_t)f * (x >> kPrecision) + rr;
    int64_t value = slot;
    int err = 0;
    if (wd.pos + 3 <= wd.filled) {
        // the next three words are in the ring
        uint32_t q0 = wd.next, q1 = wd.at(wd.pos + 1), q2 = wd.at(wd.pos + 2);
        uint32_t used = 0;
        auto renorm = [&]() {
            const bool need = x < kStateLow;
            x = need ? ((x << 32) | q0) : x;
            q0 = need ? q1 : q0;
            q1 = need ? q2 : q1;
            used += need ? 1u : 0u;
        };
        renorm();
        if (slot == mv) {
            uint32_t nb = (uint32_t)x & 15u;
            x >>= kBypassBits;
            renorm();
            if (nb > 8u) {   // raw < 2^31 needs at most 8 groups
                err = RANS_E_CORRUPT;
                nb = 0;
            }
            uint32_t raw = 0;
            for (uint32_t k = 0; k < nb; ++k) {
                raw |= ((uint32_t)x & 15u) << (kBypassBits * k);
                x >>= kBypassBits;
                renorm();
            }
            if (raw >= (1u << 31))
                err = RANS_E_CORRUPT;
            value = (raw & 1) ? -(int64_t)(raw >> 1) - 1 : (int64_t)(raw >> 1) + mv;
        }
        wd.pos += used;
    } else {
        // near the end of the ring (or of the lane): one word at a time
        if (!wd.refill(x))
            return RANS_E_CORRUPT;
        if (slot == mv) {
            const uint32_t nb = (uint32_t)x & 15u;
            x >>= kBypassBits;
            if (!wd.refill(x) || nb > 8u)
                return RANS_E_CORRUPT;
            uint64_t raw = 0;
            for (uint32_t k = 0; k < nb; ++k) {
                raw |= (uint64_t)((uint32_t)x & 15u) << (kBypassBits * k);
                x >>= kBypassBits;
                if (!wd.refill(x))
                    return RANS_E_CORRUPT;
            }
            if (raw >= (1ull << 31))
                return RANS_E_CORRUPT;
            value = (raw & 1) ? -(int64_t)(raw >> 1) - 1 : (int64_t)(raw >> 1) + mv;
        }
    }
    const int64_t sym = value + m.offset;
    if (sym < INT32_MIN || sym > INT32_MAX)
        err = RANS_E_CORRUPT;
    out = (int32_t)sym;
    return err;
}

// One decoding step of one lane, committed at once.  Lanes outside the common
// case (past the window, escape or out-of-range value, renormalisation word
// not in the ring, bad index) redo the step on the slow path.  A bad row
// index arrives with a fast bound of 0.
template <class WordsT, class Tab>
__device__ __forceinline__ void decode_step(int32_t r, const RowMeta &m, uint64_t &x, WordsT &wd,
                                            const DecTables &t, const Tab &tab, int32_t &out,
                                            int &lerr)
{
    const Lookup s = lookup_step(m, x, t, tab);
    const bool need = s.xn < kStateLow;
    const bool slow = s.beyond | (s.slot >= (m.mvf >> 16)) | (need & (wd.pos >= wd.filled));
    const uint64_t x0 = x;
    const uint32_t pos0 = wd.pos;
    x = need ? ((s.xn << 32) | wd.next) : s.xn;
    wd.pos = pos0 + (need ? 1u : 0u);
    out = (int32_t)(s.slot + (uint32_t)m.offset);
    if (__builtin_expect(__ballot(slow) != 0, 0)) {
        if (slow) {
            x = x0;
            wd.pos = pos0;
            const int ec = decode_slow(r, m, s.bucket, s.beyond, s.slot, s.f, s.rr, x, wd, t, tab,
                                       out);
            lerr = lerr ? lerr : ec;
        }
    }
    wd.next = wd.at(wd.pos);
}

// One speculative step: the common case applied with no branch; `bad` gathers
// every reason the result might be wrong (a word read past the ring's filled
// part is caught once per round, from the final position).
template <int TPB, class Tab>
__device__ __forceinline__ void decode_step_spec(const RowMeta &m, uint64_t &x, Words<TPB> &wd,
                                                 const DecTables &t, const Tab &tab, int32_t &out,
                                                 bool &bad)
{
    const Lookup s = lookup_step(m, x, t, tab);
    const bool need = s.xn < kStateLow;
    x = need ? ((s.xn << 32) | wd.next) : s.xn;
    wd.pos += need ? 1u : 0u;
    out = (int32_t)(s.slot + (uint32_t)m.offset);
    bad = bad | s.beyond | (s.slot >= (m.mvf >> 16));
    wd.next = wd.at(wd.pos);
}

// Everything one wave does for one work unit group: units u0 .. u0 + lpw - 1
// (lane j's pieces u = j * 2^pl + s), one per wavefront lane.
template <bool SPLIT, class Tab>
__device__ __forceinline__ void decode_wave(const DecodeArgs &a, const Tab &tab, const DecTables &t,
                                            uint32_t L, uint32_t lpw, uint32_t u0)
{
    constexpr int TPB = kDecTPB;
    // the speculative rounds are built for LDS tables only (a set read from
    // the workspace takes the per-step form)
    constexpr bool kSpeculate = std::is_same<Tab, LdsTab>::value;
    WsHeader *hdr = reinterpret_cast<WsHeader *>(a.ws);
    const uint32_t K = t.K;
    const uint32_t tid = threadIdx.x;
    const uint32_t lane = tid & (kWave - 1);
    const uint32_t ring = decode_ring_base(TPB) + 4 * tid;
    const uint32_t pl = SPLIT ? a.pieces_log2 : 0u;
    // the wave's unit range is the same in every lane: kept in scalar
    // registers, so are the buffer descriptors built from it (the compiler
    // cannot see that across the unit-group loop)
    u0 = __builtin_amdgcn_readfirstlane(u0);
    lpw = __builtin_amdgcn_readfirstlane(lpw);
    L = __builtin_amdgcn_readfirstlane(L);
    const uint32_t LV = L << pl;
    const uint32_t u = u0 + lane;
    const uint32_t j = u >> pl;                 // the unit's lane
    const uint32_t ps = u & ((1u << pl) - 1);   // and piece
    const bool spec = lpw <= kSpecLanes;        // wave-uniform
    // first position of unit v (v = LV gives n)
    auto unit_begin = [&](uint32_t v) -> uint64_t {
        const uint32_t lj = v >> pl;
        const uint64_t lb = lane_begin(a.n, L, lj);
        return lj < L ? piece_begin(lb, lane_begin(a.n, L, lj + 1), pl, v & ((1u << pl) - 1)) : lb;
    };
    // the wave's index and symbol spans, and its stream words, as buffers
    const uint32_t u1 = min(u0 + lpw, LV);
    const uint64_t bw = unit_begin(u0), ew = unit_begin(u1);
    const Rsrc ridx = make_rsrc(a.indexes + bw, (uint32_t)(4 * (ew - bw)));
    const Rsrc rout = make_rsrc(a.symbols + bw, (uint32_t)(4 * (ew - bw)));
    const uint32_t jw = u0 >> pl;   // the wave's first lane
    // the wave's first word (scalar, so the stream's buffer descriptor is)
    const uint64_t wbase = jw ? (uint32_t)__builtin_amdgcn_readfirstlane(a.stream[jw]) : 0u;
    const uint64_t wavail = a.capacity - 1 - L;
    const uint64_t wbytes = wbase < wavail ? rsrc_bytes(4 * (wavail - wbase)) : 0;
    const Rsrc rstr = make_rsrc(a.stream + 1 + L + (wbase < wavail ? wbase : 0), (uint32_t)wbytes);
    if (!(lane < lpw && u < LV))
        return;
    int lerr = 0;
    const uint64_t beg_w = j ? a.stream[j] : 0u;
    const uint64_t end_w = a.stream[1 + j];
    // the piece's start and end: word offset in the lane and state (piece 0
    // starts after the flushed state; the last piece ends at the start state
    // with every word read)
    const uint32_t W = (uint32_t)(end_w - beg_w);
    const uint32_t *rec = a.split_meta + 3ull * ((uint64_t)((1u << pl) - 1) * j + ps);
    uint32_t left0 = W - 2, left1 = 0;
    if (ps)
        left0 = rec[-1];
    if (ps + 1 < (1u << pl))
        left1 = rec[2];
    const bool bad_rec = left0 > W - 2 || left1 > left0;
    if (end_w < beg_w + 2 || 1ull + L + end_w > a.capacity || beg_w < wbase || bad_rec) {
        lerr = RANS_E_CORRUPT;
    } else {
        Words<TPB> wd;
        wd.w = a.stream + 1 + L + beg_w;
        wd.ring = ring;
        wd.count = W;
        const uint32_t o = W - left0;   // the piece's first unread word
        const uint32_t lw = (uint32_t)(4 * (beg_w - wbase));   // the lane's words in rstr
        // words o-2, o-1 (piece 0: the final state) and [o, o + kDecRing): the
        // first ring fill
        const uint32_t lo = lw + 4 * (o - 2);
        const u32x4 w0 = buf_load4(rstr, lo), w1 = buf_load4(rstr, lo + 16);
        const u32x4 w2 = buf_load4(rstr, lo + 32);
        uint64_t x = ps ? ((uint64_t)rec[-3] | ((uint64_t)rec[-2] << 32))
                        : ((uint64_t)w0[0] | ((uint64_t)w0[1] << 32));
        const uint64_t x_end =
            ps + 1 < (1u << pl) ? ((uint64_t)rec[0] | ((uint64_t)rec[1] << 32)) : kStateLow;
        {
            static_assert(kDecRing == 8, "ring fill below assumes 8 slots");
            const uint32_t v[kDecRing] = {w0[2], w0[3], w1[0], w1[1], w1[2], w1[3], w2[0], w2[1]};
#pragma unroll
            for (uint32_t k = 0; k < kDecRing; ++k)
                wd.put(o + k, v[k]);
        }
        wd.pos = o;
        wd.filled = min(wd.count, o + kDecRing);
        wd.next = wd.at(o);
        // Ring refills: kRefill words a round, requested two memory phases
        // before they are put into the ring (pa serves the rounds that use
        // ia, pb those that use ib), so a round never waits on a request of
        // the round before.  req is the next word to request; a phase asks
        // for [req, req + 4) only while req - pos <= 4, which keeps the four
        // ring slots it will overwrite consumed by the time it lands.  A
        // request that does not land at `filled` (the lane drained its ring
        // and read ahead directly) is dropped, and requests restart there.
        uint32_t pa[kRefill], pb[kRefill];
        uint32_t pa_at = ~0u, pb_at = ~0u, req = wd.filled;

        const uint64_t b = unit_begin(u);
        const uint64_t e = unit_begin(u + 1);
        const uint32_t nj = (uint32_t)(e - b);
        const uint32_t ob = (uint32_t)(4 * (b - bw));   // the lane's first position
        // Two index buffers used in turn (no register copies between rounds):
        // a buffer is refilled in the memory phase right after its round and
        // read again two rounds later.  Every memory phase issues the same
        // global accesses in the same order (8 stores, 8 index loads, kRefill
        // word loads), and the prologue runs two such phases too, so the
        // compiler's wait counts only ever cover requests that are at least a
        // round old.  Loads past the wave's span read 0; stores meant for
        // nothing use kNoStore.
        int32_t ia[kRound], ib[kRound], out[2 * kRound];
#pragma unroll
        for (int k = 0; k < 2 * kRound; ++k)
            out[k] = 0;
        // The round's symbols: a full round (every lane of the wave) as two
        // 16-byte stores, a partial one (a lane's last round) a word per
        // position, stores past the lane's end going nowhere.  Full rounds
        // carry no per-word address work; the wait counts merged from the
        // rare partial branch cost less than the eight extra stores (6% on
        // the 1080p latent at 4096 lanes).
        // The symbols of a pair of rounds (positions k0 .. k0+15), stored
        // after the second: 64 bytes per lane at once, which halves the
        // partial-line writes of 32-byte pieces.
        auto store_pair = [&](uint32_t k0) {
            if (__builtin_expect(__all(k0 + 2 * kRound <= nj), 1)) {
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    buf_store4(rout, ob + 4 * k0 + 16 * q,
                               u32x4{(uint32_t)out[4 * q], (uint32_t)out[4 * q + 1],
                                     (uint32_t)out[4 * q + 2], (uint32_t)out[4 * q + 3]});
            } else {
#pragma unroll
                for (int k = 0; k < 2 * kRound; ++k)
                    buf_store(rout, k0 + k < nj ? ob + 4 * (k0 + k) : kNoStore, 0, out[k]);
            }
        };
        // indexes of positions k .. k+7 and kRefill stream words: 16-byte
        // loads, the same three in every phase (past the wave's span or the
        // stream they read 0; a phase that requests no words loads at
        // kNoStore, past every buffer)
        static_assert(kRefill == 4, "one 16-byte load of stream words");
        auto load_next = [&](int32_t (&idx)[kRound], uint32_t (&pend)[kRefill], uint32_t &pend_at,
                             uint32_t k) {
            const bool ask = req - wd.pos <= kRefill;
            const u32x4 i0 = buf_load4(ridx, ob + 4 * k), i1 = buf_load4(ridx, ob + 4 * k + 16);
            const u32x4 w = buf_load4(rstr, ask ? lw + 4 * req : kNoStore);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                idx[q] = (int32_t)i0[q];
                idx[4 + q] = (int32_t)i1[q];
                pend[q] = w[q];
            }
            pend_at = ask ? req : ~0u;
            req += ask ? kRefill : 0u;
            __builtin_amdgcn_sched_barrier(0);
        };
        auto ring_refill = [&](const uint32_t (&pend)[kRefill], uint32_t pend_at) {
            if (pend_at == wd.filled) {
#pragma unroll
                for (uint32_t k = 0; k < kRefill; ++k)
                    wd.put(wd.filled + k, pend[k]);
                wd.filled = min(wd.count, wd.filled + kRefill);
            } else if (pend_at != ~0u) {
                req = max(wd.filled, wd.pos);   // requests no longer contiguous: restart
            }
            if (wd.filled < wd.pos) {   // the lane outran its ring via direct reads
                wd.filled = wd.pos;
                req = max(req, wd.pos);
            }
            wd.next = wd.at(wd.pos);
        };
        auto round = [&](auto second, int32_t (&idx)[kRound], uint32_t (&pend)[kRefill],
                         uint32_t &pend_at, uint32_t k0) {
            constexpr int o = decltype(second)::value ? kRound : 0;   // the round's out[] half
            // row metadata; an index outside [0, K) reads row K-1 with a fast
            // bound of 0 (its step then reports the index), which only a round
            // holding such an index has to arrange
            RowMeta m[kRound];
            uint32_t imax = (uint32_t)idx[0];
#pragma unroll
            for (int k = 1; k < kRound; ++k)
                imax = max(imax, (uint32_t)idx[k]);
            if (__builtin_expect(__ballot(imax >= K) == 0, 1)) {
#pragma unroll
                for (int k = 0; k < kRound; ++k)
                    m[k] = tab.meta((uint32_t)idx[k]);
            } else {
#pragma unroll
                for (int k = 0; k < kRound; ++k) {
                    m[k] = tab.meta(min((uint32_t)idx[k], K - 1));
                    if ((uint32_t)idx[k] >= K)
                        m[k].mvf = 0;
                }
            }
            // A round lies wholly inside every lane of the wave, or not.  Waves
            // of few lanes first decode a whole round speculatively; the
            // per-step form then runs only for the lanes where that went
            // wrong (bad), or for every lane when the round was not
            // speculated (many lanes a wave, or a partial round).
            const bool full = __all(k0 + kRound <= nj);
            bool general = true;
            if constexpr (kSpeculate) {
                if (spec && full) {
                    const uint64_t x0 = x;
                    const uint32_t pos0 = wd.pos, next0 = wd.next;
                    bool bad = false;
#pragma unroll
                    for (int k = 0; k < kRound; ++k)
                        decode_step_spec<TPB>(m[k], x, wd, t, tab, out[o + k], bad);
                    bad = bad | (wd.pos > wd.filled);   // read a ring slot not yet filled
                    if (bad) {
                        x = x0;
                        wd.pos = pos0;
                        wd.next = next0;
                    }
                    general = bad;
                }
            }
            if (__builtin_expect(__ballot(general) != 0, !kSpeculate || !spec || !full)) {
#pragma unroll
                for (int k = 0; k < kRound; ++k) {
                    if (general) {
                        out[o + k] = 0;
                        if (k0 + k < nj && !lerr)
                            decode_step(idx[k], m[k], x, wd, t, tab, out[o + k], lerr);
                    }
                }
            }
            __builtin_amdgcn_sched_barrier(0);
            ring_refill(pend, pend_at);
            // the phase's loads go out before its stores: a full round stores
            // 16 bytes twice, a partial one word by word, and a later wait
            // for these loads then never has to cover those stores
            load_next(idx, pend, pend_at, k0 + 2 * kRound);
            if constexpr (decltype(second)::value)
                store_pair(k0 - kRound);
            __builtin_amdgcn_sched_barrier(0);
        };
        // prologue: two phases of the same shape (stores to nothing)
#pragma unroll
        for (int p = 0; p < 2; ++p) {
            if (p)
                load_next(ib, pb, pb_at, kRound);
            else
                load_next(ia, pa, pa_at, 0);
            __builtin_amdgcn_sched_barrier(0);
        }
        // both rounds always run (symbols past the lane end are skipped inside),
        // so every path back to the loop head passes both memory phases
        for (uint32_t k0 = 0; k0 < nj && !lerr; k0 += 2 * kRound) {
            round(std::false_type{}, ia, pa, pa_at, k0);
            round(std::true_type{}, ib, pb, pb_at, k0 + kRound);
        }
        if (!lerr && (x != x_end || wd.pos != W - left1))
            lerr = RANS_E_CORRUPT;
    }
    if (lerr)
        record_error(hdr, lerr);
}

// ---- one decoding wave per CU (at most 2048 lanes) ------------------------------
//
// With at most 2048 lanes, 8 lanes or fewer go to each CU, and one wave
// decodes them all: its time is that of the lanes' chains of dependent
// lookups, and every other instruction it issues lengthens them.  So the
// block's other waves do the state-independent work around the chains:
//  * waves 1 and 2 load each step's row index and write the row's metadata
//    (an index outside [0, K) gets row K-1's with a fast bound of 0, whose
//    step then reports the index) into entry buffers, one chunk of 32 steps
//    ahead of the decoding wave, and store the decoded symbols of the chunk
//    two behind it from LDS to memory, 16 bytes a lane;
//  * wave 3 keeps each lane's next 128 stream words in an LDS FIFO: at every
//    handover it is told how far the lane has read, and refills the slots of
//    words read before;
//  * waves 4 to 7 (on the SIMDs of waves 0 to 3) only take part in the
//    barriers.
// A round inside every lane is decoded with no branch first; a lane that
// met a step outside the common case takes up again from the state before
// it, step by step.  Measured against eight decoding waves of few lanes
// each: 151 against 167 us at 2048 lanes of the 1080p latent, 254 against
// 334 us at 1024; at 4096 lanes (16 a wave) the eight waves were 2% faster,
// and there the eight-wave form is kept.
// One barrier per chunk, at the start of the decoding wave's last round of a
// chunk (that round's entries are already in registers), hands over the next
// chunk's entries, the words filled since the last handover, and the symbols
// of the chunk before last.  The decoding wave takes each step as decode_step
// does (committed at once; lanes outside the common case redo it on the slow
// path), so a word the FIFO does not hold yet is read from memory there.
constexpr uint32_t kPdMaxLanes = 2048;
constexpr uint32_t kPdLanes = 16;                              // lanes of a group, at most
constexpr uint32_t kPdChainWaves = 1;                          // decoding waves a block
constexpr uint32_t kPdChainLanes = kPdLanes / kPdChainWaves;   // lanes of a decoding wave
constexpr uint32_t kPdChunkRounds = 4;
constexpr uint32_t kPdChunk = kPdChunkRounds * kRound;   // steps per chunk
constexpr uint32_t kPdFifo = 128;                        // words per lane
constexpr uint32_t kPdEntryBuf = kPdChunk * kPdLanes * 16;
constexpr uint32_t kPdOutBuf = kPdChunk * kPdLanes * 4;
// the region after the table set: [entries x2 | symbols x3 | fifo | positions]
constexpr uint32_t kPdOut = 2 * kPdEntryBuf;
constexpr uint32_t kPdFifoOff = kPdOut + 3 * kPdOutBuf;
constexpr uint32_t kPdPos = kPdFifoOff + kPdFifo * kPdLanes * 4;
constexpr uint32_t kPdBytes = kPdPos + 4 * kPdLanes;
static_assert(lanes_per_wave_for(kPdMaxLanes, kCodingCUs) <= kPdLanes, "decoding wave too wide");
static_assert((kPdChunk / 4) * kPdLanes == 2 * kWave, "one quad of steps per entry producer");
static_assert(kPdChunkRounds % 2 == 0, "rounds run in pairs");
static_assert(kDecTPB == 8 * kWave && kPdChainWaves + 3 <= 8, "decoding, producing and waiting waves");
static_assert(kPdLanes % kPdChainWaves == 0, "lanes split evenly over the decoding waves");

// The lane's words in the FIFO: word p in slot p mod kPdFifo; [.., filled)
// hold words (the interface of Words, for decode_step and decode_slow).
struct PdWords {
    const uint32_t *w;   // the lane's words in global memory
    uint32_t fifo;       // LDS address of this lane's slot 0 (slots are kPdLanes words apart)
    uint32_t count;      // words in the lane
    uint32_t pos;        // next word to consume
    uint32_t filled;     // words [.., filled) are in the FIFO
    uint32_t next;       // FIFO word at pos (valid when pos < filled)

    __device__ inline uint32_t slot(uint32_t p) const { return fifo + (p % kPdFifo) * (4 * kPdLanes); }
    __device__ inline uint32_t at(uint32_t p) const { return lds_load<uint32_t>(slot(p)); }
    __device__ inline bool refill(uint64_t &x)
    {
        if (x < kStateLow) {
            if (pos >= count)
                return false;
            if (pos < filled) {
                x = (x << 32) | next;
            } else {
                const uint32_t direct = w[pos];
                __builtin_amdgcn_s_waitcnt(0);
                x = (x << 32) | direct;
            }
            ++pos;
        }
        next = at(pos);
        return true;
    }
};

// Lane j of a group: positions [b, b + nj), payload words [beg_w, beg_w + W)
// (header entries checked as in decode_wave).
struct PdLane {
    uint64_t b, beg_w;
    uint32_t nj, W;
    bool ok;
};

// Decode one group of lanes j0 .. j0 + lpw - 1 with the block's eight waves;
// P is the LDS address of the region after the table set.
__device__ __forceinline__ void decode_pc_group(const DecodeArgs &a, const DecTables &t,
                                                uint32_t L, uint32_t lpw, uint32_t grp, uint32_t P)
{
    WsHeader *hdr = reinterpret_cast<WsHeader *>(a.ws);
    const uint32_t K = t.K;
    const uint32_t tid = threadIdx.x;
    const uint32_t lane = tid & (kWave - 1);
    const uint32_t wave = __builtin_amdgcn_readfirstlane(tid / kWave);
    const uint32_t j0 = __builtin_amdgcn_readfirstlane(grp * lpw);
    const uint32_t j1 = min(j0 + lpw, L);
    // the group's positions and stream words, as buffers
    const uint64_t bw = lane_begin(a.n, L, j0), ew = lane_begin(a.n, L, j1);
    const Rsrc ridx = make_rsrc(a.indexes + bw, (uint32_t)(4 * (ew - bw)));
    const Rsrc rout = make_rsrc(a.symbols + bw, (uint32_t)(4 * (ew - bw)));
    const uint64_t wbase = j0 ? (uint32_t)__builtin_amdgcn_readfirstlane(a.stream[j0]) : 0u;
    const uint64_t wavail = a.capacity - 1 - L;
    const uint64_t wbytes = wbase < wavail ? rsrc_bytes(4 * (wavail - wbase)) : 0;
    const Rsrc rstr = make_rsrc(a.stream + 1 + L + (wbase < wavail ? wbase : 0), (uint32_t)wbytes);
    // rounds of the longest lane, and chunks
    const uint32_t nr = (uint32_t)(((a.n + L - 1) / L + kRound - 1) / kRound);
    const uint32_t nch = (nr + kPdChunkRounds - 1) / kPdChunkRounds;
    // roles: decoding waves [0, cw), entry waves cw and cw+1, the FIFO wave
    // cw+2, the rest only take part in the barriers
    constexpr uint32_t cw = kPdChainWaves;
    const bool chain = wave < cw;
    const uint32_t p = tid - cw * kWave;   // producer thread
    // this thread's lane: the decoding wave's lane, or the producers' l
    // (a decoding wave's lanes past its share alias lanes of it, and only read)
    const uint32_t l = chain ? kPdChainLanes * wave + (lane & (kPdChainLanes - 1)) : p % kPdLanes;
    const uint32_t j = j0 + l;
    const bool act = (chain ? lane < kPdChainLanes : wave < cw + 3) && l < lpw && j < L;
    PdLane ln{};
    if (act) {
        ln.b = lane_begin(a.n, L, j);
        ln.nj = (uint32_t)(lane_begin(a.n, L, j + 1) - ln.b);
        const uint64_t beg_w = j ? a.stream[j] : 0u;
        const uint64_t end_w = a.stream[1 + j];
        ln.ok = !(end_w < beg_w + 2 || 1ull + L + end_w > a.capacity || beg_w < wbase);
        ln.beg_w = beg_w;
        ln.W = ln.ok ? (uint32_t)(end_w - beg_w) : 2u;
    }
    auto entry_at = [&](uint32_t chunk, uint32_t s, uint32_t ll) {
        return P + (chunk & 1u) * kPdEntryBuf + (s * kPdLanes + ll) * 16;
    };
    auto out_at = [&](uint32_t chunk, uint32_t s, uint32_t ll) {   // lane-major
        return P + kPdOut + (chunk % 3u) * kPdOutBuf + (ll * kPdChunk + s) * 4;
    };
    const uint32_t pos_at = P + kPdPos + 4 * l;

    if (chain) {
        // ---- a decoding wave --------------------------------------------------
        int lerr = (act && !ln.ok) ? RANS_E_CORRUPT : 0;
        const bool live = act && ln.ok;
        PdWords wd;
        wd.w = a.stream + 1 + L + ln.beg_w;
        wd.fifo = P + kPdFifoOff + 4 * l;
        wd.count = ln.W;
        wd.pos = 2;
        wd.filled = min(ln.W, 2 + kPdFifo);
        wd.next = 0;
        uint64_t x = kStateLow;
        if (live)
            x = (uint64_t)wd.w[0] | ((uint64_t)wd.w[1] << 32);   // the flushed state
        uint32_t pub = 2;   // the position published at the last handover
        const uint32_t el = l & (kPdLanes - 1);
        auto load_round = [&](u32x4 (&E)[kRound], uint32_t g) {
            const uint32_t s0 = (g % kPdChunkRounds) * kRound;
#pragma unroll
            for (int u = 0; u < kRound; ++u)
                E[u] = lds_load<u32x4>(entry_at(g / kPdChunkRounds, s0 + u, el));
        };
        auto meta_of = [](const u32x4 &e) {
            RowMeta m;
            m.base = e[0];
            m.offset = (int32_t)e[1];
            m.mvf = e[2];
            m.lut = e[3];
            return m;
        };
        // (a bad index arrives with mvf 0: its step reports it)
        auto row_of = [&](const RowMeta &m) -> int32_t { return (m.mvf & 0xFFFFu) ? 0 : (int32_t)K; };
        // One round.  A round inside every lane is first decoded with no
        // branch, each lane noting its first step outside the common case
        // (past the lookup window, an escape or a value out of int32's
        // range, a word the FIFO does not hold yet); such a lane then takes
        // up again from the state before that step, step by step as
        // decode_step does.  A lane's last, partial round goes step by step
        // from the start.  The round's symbols go to LDS as 32 bytes a lane.
        auto round = [&](const u32x4 (&E)[kRound], uint32_t g) {
            const uint32_t k0 = g * kRound;
            const uint32_t c = g / kPdChunkRounds, s0 = (g % kPdChunkRounds) * kRound;
            int32_t o[kRound];
            if (__all(k0 + kRound <= ln.nj)) {
                uint64_t xs[kRound];
                uint32_t ps[kRound];
                uint32_t first_bad = kRound;
#pragma unroll
                for (int u = 0; u < kRound; ++u) {
                    xs[u] = x;
                    ps[u] = wd.pos;
                    const RowMeta m = meta_of(E[u]);
                    const Lookup sl = lookup_step(m, x, t, LdsTab{});
                    const bool need = sl.xn < kStateLow;
                    const bool bad = sl.beyond | (sl.slot >= (m.mvf >> 16)) |
                                     (need & (wd.pos >= wd.filled));
                    first_bad = (bad & (first_bad == kRound)) ? (uint32_t)u : first_bad;
                    x = need ? ((sl.xn << 32) | wd.next) : sl.xn;
                    wd.pos += need ? 1u : 0u;
                    o[u] = (int32_t)(sl.slot + (uint32_t)m.offset);
                    wd.next = wd.at(wd.pos);
                }
                if (__builtin_expect(__ballot(first_bad < kRound) != 0, 0)) {
                    if (first_bad < kRound) {
#pragma unroll
                        for (int u = 0; u < kRound; ++u) {
                            x = first_bad == (uint32_t)u ? xs[u] : x;
                            wd.pos = first_bad == (uint32_t)u ? ps[u] : wd.pos;
                        }
                        wd.next = wd.at(wd.pos);
                    }
#pragma unroll
                    for (int u = 0; u < kRound; ++u)
                        if (first_bad <= (uint32_t)u)
                            decode_step(row_of(meta_of(E[u])), meta_of(E[u]), x, wd, t, LdsTab{},
                                        o[u], lerr);
                }
            } else {
#pragma unroll
                for (int u = 0; u < kRound; ++u) {
                    o[u] = 0;
                    if (k0 + u < ln.nj)
                        decode_step(row_of(meta_of(E[u])), meta_of(E[u]), x, wd, t, LdsTab{},
                                    o[u], lerr);
                }
            }
            const uint32_t oa = out_at(c, s0, l);
            lds_store<u32x4>(oa, u32x4{(uint32_t)o[0], (uint32_t)o[1], (uint32_t)o[2], (uint32_t)o[3]});
            lds_store<u32x4>(oa + 16, u32x4{(uint32_t)o[4], (uint32_t)o[5], (uint32_t)o[6], (uint32_t)o[7]});
        };
        const uint32_t nr2 = (nr + 1) & ~1u;
        u32x4 E0[kRound], E1[kRound];
        auto handover = [&]() {
            if (act)
                lds_store<uint32_t>(pos_at, wd.pos);
            __syncthreads();
            // the FIFO now holds the words filled since the handover before
            wd.filled = min(ln.W, pub + kPdFifo);
            pub = wd.pos;
            wd.next = wd.at(wd.pos);
        };
        auto step = [&](const u32x4 (&E)[kRound], u32x4 (&En)[kRound], uint32_t g) {
            if (g % kPdChunkRounds == kPdChunkRounds - 1 && g + 1 < nr2)
                handover();
            load_round(En, g + 1);
            if (live)
                round(E, g);
        };
        if (nr2 > 0) {
            if (act)
                lds_store<uint32_t>(pos_at, 2u);
            __syncthreads();   // chunk 0 and the first words are ready
            wd.next = wd.at(2);
            load_round(E0, 0);
        }
        for (uint32_t g = 0; g < nr2; g += 2) {
            step(E0, E1, g);
            step(E1, E0, g + 1);
        }
        __syncthreads();   // the producers' last barrier
        if (live && !lerr && (x != kStateLow || wd.pos != ln.W))
            lerr = RANS_E_CORRUPT;
        if (lerr)
            record_error(hdr, lerr);
    } else if (wave < cw + 2) {
        // ---- entries and symbol stores ---------------------------------------
        const uint32_t q = p / kPdLanes;   // steps 4q .. 4q+3 of a chunk
        auto fill_entries = [&](uint32_t c) {
            if (!act)
                return;
            const uint32_t k = c * kPdChunk + 4 * q;
            const u32x4 iv = buf_load4(ridx, (uint32_t)(4 * (ln.b - bw)) + 4 * k);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const uint32_t idx = iv[e];
                u32x4 m = lds_load<u32x4>(16 * min(idx, K - 1));
                if (idx >= K)
                    m[2] = 0u;   // fast bound and escape slot 0
                lds_store<u32x4>(entry_at(c, 4 * q + e, l), m);
            }
        };
        auto store_symbols = [&](uint32_t c) {
            if (!act || !ln.ok)
                return;
            const uint32_t k = c * kPdChunk + 4 * q;
            if (k >= ln.nj)
                return;
            const u32x4 v = lds_load<u32x4>(out_at(c, 4 * q, l));
            const uint32_t ob = (uint32_t)(4 * (ln.b - bw)) + 4 * k;
            if (k + 4 <= ln.nj) {
                buf_store4(rout, ob, v);
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    if (k + e < ln.nj)
                        buf_store(rout, ob + 4 * e, 0, (int32_t)v[e]);
            }
        };
        if (nch > 0) {
            fill_entries(0);
            __syncthreads();
            for (uint32_t c = 0; c < nch; ++c) {
                if (c + 1 < nch)
                    fill_entries(c + 1);
                if (c >= 2)
                    store_symbols(c - 2);
                if (c + 1 < nch)
                    __syncthreads();
            }
        }
        __syncthreads();   // the decoding wave is done
        if (nch >= 2)
            store_symbols(nch - 2);
        if (nch >= 1)
            store_symbols(nch - 1);
    } else if (wave == cw + 2) {
        // ---- stream words into the FIFO ----------------------------------------
        const uint32_t sub = (p - 2 * kWave) / kPdLanes;   // four threads a lane
        const bool mine = act && ln.ok;
        uint32_t filled = 2;   // words [2, filled) are in the FIFO
        const uint32_t lw = (uint32_t)(4 * (ln.beg_w - wbase));   // the lane's words in rstr
        const uint32_t fifo = P + kPdFifoOff + 4 * l;
        // words [filled, target): sixteen a pass (four per thread), four
        // passes' loads issued before any of their FIFO writes
        auto fill_words = [&](uint32_t target) {
            while (filled < target) {
                u32x4 v[4];
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    const uint32_t w0 = filled + 16 * k + 4 * sub;
                    v[k] = w0 < target ? buf_load4(rstr, lw + 4 * w0) : u32x4{0u, 0u, 0u, 0u};
                }
#pragma unroll
                for (int k = 0; k < 4; ++k)
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const uint32_t w = filled + 16 * k + 4 * sub + e;
                        if (w < target)
                            lds_store<uint32_t>(fifo + (w % kPdFifo) * (4 * kPdLanes), v[k][e]);
                    }
                filled = min(target, filled + 64);
            }
        };
        if (mine)
            fill_words(min(ln.W, 2 + kPdFifo));
        if (nch > 0) {
            __syncthreads();
            for (uint32_t c = 0; c + 1 < nch; ++c) {
                // the slots of words the lane had read at the handover
                if (mine)
                    fill_words(min(ln.W, lds_load<uint32_t>(pos_at) + kPdFifo));
                __syncthreads();
            }
        }
        __syncthreads();
    } else {
        // ---- waves 4 to 7: the barriers only ---------------------------------------
        if (nch > 0) {
            __syncthreads();
            for (uint32_t c = 0; c + 1 < nch; ++c)
                __syncthreads();
        }
        __syncthreads();
    }
}

template <bool SPLIT>
__global__ __launch_bounds__(kDecTPB) void decode_kernel(DecodeArgs a)
{
    constexpr int TPB = kDecTPB;
    extern __shared__ __align__(16) uint8_t lds[];
    // block bookkeeping after the table set and before the rings: [0] flag OR, [1] last block
    uint32_t *misc = reinterpret_cast<uint32_t *>(lds + kDecTableBudget);

    WsHeader *hdr = reinterpret_cast<WsHeader *>(a.ws);
    const uint8_t *tab = a.ws + ws_dec_offset();
    const uint32_t tid = threadIdx.x;

    int herr = 0;
    if (hdr->magic != kMagic || hdr->num_tables != (uint32_t)a.num_tables ||
        hdr->cdf_stride != (uint32_t)a.stride)
        herr = RANS_E_ARG;
    else if (lds_address_of(lds) != 0)   // table offsets are used as LDS addresses
        herr = RANS_E_HIP;
    // the lane count from the container (header word 0), checked against the
    // readable words and, with split records, against the record array
    const uint32_t pl = SPLIT ? a.pieces_log2 : 0u;
    const uint32_t L = (uint32_t)__builtin_amdgcn_readfirstlane(a.stream[0]);
    if (!herr && (L == 0 || L > RANS_MAX_LANES || 1ull + L > a.capacity))
        herr = RANS_E_CORRUPT;
    if (!herr && SPLIT && 3ull * L * ((1u << pl) - 1) > a.split_words)
        herr = RANS_E_ARG;
    const uint32_t K = (uint32_t)a.num_tables;
    const bool in_lds = hdr->dec_lds != 0;
    DecTables t;
    t.q = hdr->lut_q;
    t.shift = kPrecision - t.q;
    t.K = K;

    // Work units: lane j's pieces u = j * 2^pl + s (one piece per lane
    // without split records), spread thin over waves (lpw units a wave).
    // With at most one wave per block in use, every block codes one wave
    // (its other waves only help stage the tables); beyond, all eight code.
    // Wave w of the grid takes unit groups w, w + G*cw, ...  Whole lanes on
    // a staged table set that leaves room for its buffers, at most 4096 of
    // them, take the one-decoding-wave form instead (decode_pc_group): a
    // group of up to 16 lanes per block, blocks taking groups b, b + G, ...
    const uint32_t LV = herr ? 0u : (L << pl);
    const uint32_t pd_base = (__builtin_amdgcn_readfirstlane(hdr->dec_bytes) + 15u) & ~15u;
    const bool pc = !SPLIT && !herr && in_lds && L <= kPdMaxLanes &&
                    pd_base + kPdBytes <= decode_lds_bytes(TPB);
    const uint32_t lpw = pc ? lanes_per_wave_for(LV, kCodingCUs) : lanes_per_wave_for(LV, kMaxDecWaves);
    const uint32_t nw = (LV + lpw - 1) / lpw;
    const uint32_t G = gridDim.x;
    const uint32_t cw = (pc || nw <= G) ? 1u : (uint32_t)(TPB / kWave);
    const bool block_work = (uint64_t)blockIdx.x * cw < nw;
    stage_tables<TPB>(lds, tab, (!herr && block_work && in_lds) ? hdr->dec_bytes : 0u);
    __syncthreads();
    int bad = 0;
    if (!herr && block_work) {
        const GlobalTab gt{tab};
        for (uint32_t r = tid; r < K; r += TPB)
            bad |= ((in_lds ? lds_meta(r) : gt.meta(r)).lut & kRowInvalid) ? 1 : 0;
    }
    if (tid == 0)
        misc[0] = 0u;
    __syncthreads();
    bad = block_or(&misc[0], bad);
    if (!herr && bad)
        herr = RANS_E_TABLE;
    if (herr && blockIdx.x == 0 && tid == 0)
        record_error(hdr, herr);

    // coding waves are 0 .. cw-1; the wave index and herr are the same in
    // every lane, and scalar they keep the buffer descriptors and loops uniform
    const uint32_t wave = __builtin_amdgcn_readfirstlane(tid / kWave);
    herr = __builtin_amdgcn_readfirstlane(herr);
    if (!herr && pc) {
        for (uint32_t w = blockIdx.x; w < nw; w += G) {
            const DecodeArgs al = fresh_kernel_args<DecodeArgs>();
            decode_pc_group(al, t, L, lpw, w, pd_base);
        }
    } else if (!herr && wave < cw) {
        const uint32_t first = blockIdx.x * cw + wave, step = G * cw;
        // The arguments are read afresh for every unit group: hoisted out of
        // the loop, they would stay live across the whole coding body and
        // crowd out its scalar registers.
        if (in_lds) {
            for (uint32_t w = first; w < nw; w += step) {
                const DecodeArgs al = fresh_kernel_args<DecodeArgs>();
                decode_wave<SPLIT>(al, LdsTab{}, t, L, lpw, w * lpw);
            }
        } else {
            for (uint32_t w = first; w < nw; w += step) {
                const DecodeArgs al = fresh_kernel_args<DecodeArgs>();
                decode_wave<SPLIT>(al, GlobalTab{al.ws + ws_dec_offset()}, t, L, lpw, w * lpw);
            }
        }
    }

    // ---- completion: the last block publishes status and cleans up -------------
    __syncthreads();
    if (tid == 0) {
        __threadfence();
        const uint32_t old = atomicAdd(&hdr->done, 1u);
        misc[1] = (old == gridDim.x - 1) ? 1u : 0u;
    }
    __syncthreads();
    if (misc[1] && tid == 0) {
        __threadfence();
        *a.status = hdr->err;
        hdr->err = 0;
        hdr->done = 0;
        __threadfence();
    }
}

// Compute units of the current device (the grid has at most one block per CU).
uint32_t device_cus()
{
    static uint32_t cached[64] = {};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64)
        return kCodingCUs;
    if (!cached[dev]) {
        int v = 0;
        if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
            v <= 0)
            v = (int)kCodingCUs;
        cached[dev] = (uint32_t)v;
    }
    return cached[dev];
}

template <bool SPLIT>
hipError_t launch_decode_t(const DecodeArgs &a, hipStream_t s)
{
    const uint32_t lds_bytes = decode_lds_bytes(kDecTPB);
    static const hipError_t attr = hipFuncSetAttribute(
        reinterpret_cast<const void *>(&decode_kernel<SPLIT>),
        hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds_bytes);
    if (attr != hipSuccess)
        return attr;
    // A valid container holds at least two words per lane after its header,
    // which bounds the lane count by the readable words; more blocks than
    // that many work units would find nothing to do.
    uint64_t units_max = a.capacity > 3 ? (a.capacity - 1) / 3 : 1;
    if (units_max > RANS_MAX_LANES)
        units_max = RANS_MAX_LANES;
    units_max <<= a.pieces_log2;
    const uint32_t cus = device_cus();
    const uint32_t blocks = units_max < cus ? (uint32_t)units_max : cus;
    hipLaunchKernelGGL((decode_kernel<SPLIT>), dim3(blocks), dim3(kDecTPB), lds_bytes, s, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_decode(const DecodeArgs &a, hipStream_t s)
{
    // decoding split pieces is its own instantiation (the plain decoder
    // carries none of the piece bookkeeping)
    if (a.pieces_log2 > 0)
        return launch_decode_t<true>(a, s);
    return launch_decode_t<false>(a, s);
}

}  // namespace rans
