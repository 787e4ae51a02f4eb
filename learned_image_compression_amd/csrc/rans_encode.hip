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
// 64-bit state in a VGPR pair; row metadata and per-slot (start, f) pairs are
// staged once per workgroup into LDS; a lane spills words backwards into its
// own scratch segment.  Waves are numbered in block order, publish their
// word total, look back over earlier waves for their offset (no grid-wide
// barrier, no second launch), then write their header entries and copy
// their lanes' words into the contiguous container.
//
// Per-symbol work.  A lane codes in rounds of kRound positions.  Everything
// that does not depend on the state -- row metadata, the slot's pair, the
// reciprocal of f, whether the symbol is an ordinary one -- is computed for
// the whole round first.  When every lane of the wave has a full round of
// ordinary symbols, the state chain runs with no branch and no LDS access.
// Otherwise the same chain runs with one wave-uniform test per position:
// where some lane escapes, those lanes first put the value's groups and
// count and take the escape slot's pair; padding positions and bad indexes
// take an identity step.  Spilled words go to the lane's LDS ring either
// way.  Only a lane near the end of its scratch segment, or a round holding
// a split cut, redoes its round with the checked puts.
//
// Memory schedule.  Global memory is touched only between rounds, in
// straight-line code with a fixed number of accesses: the round's candidate
// words are stored (a symbol that spilled nothing stores to a position that
// a later word overwrites, or to the lane's last scratch word), and the
// symbols and indexes of the round after next are requested.  A loaded
// register is first read a round after its load was issued, so the state
// chain never waits on global memory.
#include "rans_coding.hpp"

#include <type_traits>

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
constexpr uint32_t kNoStore = 0x80000000u;   // a buffer offset past every buffer

// Encoder tables: [meta | pairs], pair = start | f << 16, in LDS from address
// 0 or in the workspace (rans_internal.hpp: LdsTab, GlobalTab).

// Spill state of one lane.  Word k of the lane (its k-th spill) belongs at
// byte offset top - 4 - 4k of the wave's scratch buffer.  During a round the
// spilled words wait in the lane's LDS ring (slot i holds the round's i-th
// word; slots are TPB words apart); the memory phase stores them.
template <int TPB>
struct Spill {
    Rsrc scr;           // the wave's scratch segments
    uint32_t *ring;     // the lane's ring slot 0
    uint32_t top;       // byte offset one past the lane's segment
    uint32_t cb;        // 4 * words spilled so far
    uint32_t cb0;       // cb at the start of the round
    uint32_t capb;      // 4 * segment size (the last 2 words hold the final state)
    bool overflow;

    __device__ inline uint32_t *slot(uint32_t i) const { return ring + i * TPB; }

    // Spill the low word when `spill`.  The ring slot is written either way
    // (a slot past the round's words is never stored), so there is no branch.
    __device__ inline void put_if(bool spill, uint32_t w)
    {
        overflow = overflow | (spill & (cb + 8 >= capb));
        *slot(min((cb - cb0) >> 2, kEncRing - 1)) = w;
        cb += spill ? 4u : 0u;
    }

    // Store the round's words (ring slots 0 .. n-1) to positions
    // cb0/4 .. cb0/4 + n - 1, i.e. descending byte offsets from
    // top - 4 - cb0.  Slots 0..7 are always stored, as two 16-byte stores
    // (slots past n hold stale words for positions that later words or the
    // final state overwrite); a round of more than 8 words, or a lane near
    // the end of its segment, stores word by word.
    __device__ inline void store_round()
    {
        const uint32_t n = (cb - cb0) >> 2;
        uint32_t r[8];
#pragma unroll
        for (int i = 0; i < 8; ++i)
            r[i] = *slot(i);
        const bool whole = cb0 + 32 <= capb;
        // (a round that spilled nothing sends both stores past the buffer,
        // where they are dropped: no write traffic for it)
        const uint32_t off = (whole & (n > 0)) ? top - cb0 - 32 : kNoStore;
        buf_store4(scr, off, u32x4{r[7], r[6], r[5], r[4]});
        buf_store4(scr, off + 16, u32x4{r[3], r[2], r[1], r[0]});
        if (__builtin_expect(__ballot(!whole | (n > 8)) != 0, 0)) {
            for (uint32_t i = whole ? 8u : 0u; i < n; ++i)
                if (cb0 + 4 * i + 8 < capb)
                    buf_store(scr, top - 4 - cb0 - 4 * i, 0, (int32_t)*slot(i));
        }
        cb0 = cb;
    }
};

// The puts of one symbol that come before its REG put (applied last to
// first: an escaped value's groups, then its group count), and the (start, f)
// pair of the slot its REG put codes; the row index is in range.  Returns a
// status code.
template <int TPB, class Tab>
__device__ __forceinline__ int encode_prefix(int32_t s, const RowMeta m, const Tab &tab, uint64_t &x,
                                             Spill<TPB> &sp, uint32_t &pair)
{
    int err = 0;
    const uint32_t mv = m.mvf & 0xFFFFu;
    const int64_t v = (int64_t)s - (int64_t)m.offset;
    const bool esc = (uint64_t)v >= (uint64_t)mv;
    uint64_t raw = v < 0 ? (uint64_t)(-2 * v - 1) : (uint64_t)(2 * (v - (int64_t)mv));
    if (esc && raw >= (1ull << 31)) {
        err = RANS_E_SYMBOL_RANGE;
        raw = 0;
    }
    // BITS puts: groups nb-1 .. 0, then the count nb (none for ordinary values)
    const uint32_t bits = raw ? 64u - (uint32_t)__clzll(raw) : 0u;
    const uint32_t nb = esc ? (bits + kBypassBits - 1) / kBypassBits : 0u;
    auto put_bits = [&](uint32_t b) {
        const bool spill = x >= (1ull << (63 - kBypassBits));
        sp.put_if(spill, (uint32_t)x);
        x = spill ? (x >> 32) : x;
        x = (x << kBypassBits) | b;
    };
    for (uint32_t g = nb; g-- > 0;)
        put_bits((uint32_t)(raw >> (kBypassBits * g)) & 15u);
    if (esc)
        put_bits(nb);
    pair = tab.template load<uint32_t>(m.base + 4 * (esc ? mv : (uint32_t)v));
    return err;
}

// All puts of one symbol off the common path (an escaped value, or a lane
// near the end of its segment), applied last to first; the row index is in
// range.  Returns a status code.
template <int TPB, class Tab>
__device__ __forceinline__ int encode_slow(int32_t s, const RowMeta m, const Tab &tab, uint64_t &x,
                                           Spill<TPB> &sp)
{
    uint32_t pr;
    const int err = encode_prefix<TPB>(s, m, tab, x, sp, pr);
    const uint32_t f = pr >> 16;
    const bool spill = x >= ((uint64_t)f << (63 - kPrecision));
    sp.put_if(spill, (uint32_t)x);
    x = spill ? (x >> 32) : x;
    x = reg_step(x, pr & 0xFFFFu, f, reciprocal(f));
    return err;
}

// The coding of lane j (positions [b, e)), last position to first, into its
// scratch segment; returns the lane's word count (flushed state included) and
// its first error.
struct LaneResult {
    uint32_t words;
    int err;
};

// PAIR: the symbols and indexes of two rounds are loaded together, 64 bytes
// per lane and array, into one of two alternating 16-entry buffers (for
// waves of many lanes, whose lines the L2 would otherwise drop between one
// 32-byte round and the next); else one round's 32 bytes at a time.
template <int TPB, class Tab, bool PAIR>
__device__ __forceinline__ LaneResult encode_lane(const EncodeArgs &a, const Tab &tab, uint32_t K,
                                                  uint32_t L, uint32_t j, uint64_t bw, Rsrc rsym,
                                                  Rsrc ridx, Spill<TPB> sp)
{
    int lerr = 0;
    uint32_t words = 0;
    const uint64_t b = lane_begin(a.n, L, j);
    const uint64_t e = lane_begin(a.n, L, j + 1);
    const uint32_t nj = (uint32_t)(e - b);
    sp.cb = 0;
    sp.cb0 = 0;
    sp.capb = 4 * (2 * nj + 4);
    sp.overflow = false;
    uint64_t x = kStateLow;
    // Rounds are aligned to the lane's first position: step k codes
    // position b + R8 - 1 - k, where R8 is nj rounded up to whole rounds,
    // and the steps below pad = R8 - nj (past the lane's end) are no
    // positions.  A round's window of positions then never starts before
    // the lane (so never before the wave's buffer), and the loads need no
    // clamping branch.
    const uint32_t R8 = (nj + kRound - 1) / kRound * kRound;
    const uint32_t pad = R8 - nj;
    auto valid = [&](uint32_t k) { return k >= pad && k < R8; };
    // Split records: the next cut to record (cuts are met last to
    // first) and the step k = R8 - 1 - (c - b) at which position c
    // is coded; a round holding it takes the per-position path,
    // which records the state and the words emitted so far right
    // after that position.
    const uint32_t npieces = 1u << a.pieces_log2;
    int32_t cut_s = (int32_t)npieces - 1;
    auto cut_step = [&](int32_t s) -> uint32_t {
        return R8 - 1 - (uint32_t)(piece_begin(b, e, a.pieces_log2, (uint32_t)s) - b);
    };
    uint32_t cut_k = (npieces > 1 && nj > 0) ? cut_step(cut_s) : ~0u;
    auto record_cut = [&]() {
        uint32_t *m = a.split_meta + 3ull * ((uint64_t)(npieces - 1) * j + cut_s - 1);
        m[0] = (uint32_t)x;
        m[1] = (uint32_t)(x >> 32);
        m[2] = sp.cb >> 2;
        --cut_s;
        cut_k = (cut_s >= 1 && nj > 0) ? cut_step(cut_s) : ~0u;
    };
    // byte offset, in the wave's buffers, of the first position of the
    // lane's last whole window (steps R8 - 8 .. R8 - 1); a window of later
    // steps lies past the lane's end (its loads read the next lane's values
    // or, past the wave's buffer, zeros: only for steps that are no
    // positions)
    const uint32_t pbase = (uint32_t)(4 * (b - bw));
    int32_t sa[kRound], ia[kRound], sb[kRound], ib[kRound];
    // Symbols and indexes of steps k .. k+7: two 16-byte loads each, always
    // the same four loads in the same order, so that the compiler's wait
    // counts cover exactly the requests that are a round old or older.
    // Rounds past the lane (k >= R8) reload its first window: they code
    // nothing.
    auto load_next = [&](int32_t (&sym)[kRound], int32_t (&idx)[kRound], uint32_t k) {
        // (an empty lane loads at its own position: in the buffer, or past it)
        const uint32_t kc = R8 >= kRound ? min(k, R8 - kRound) : 0u;
        const uint32_t lo = R8 >= kRound ? pbase + 4 * (R8 - kRound - kc) : pbase;
        const u32x4 s0 = buf_load4(rsym, lo), s1 = buf_load4(rsym, lo + 16);
        const u32x4 i0 = buf_load4(ridx, lo), i1 = buf_load4(ridx, lo + 16);
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            sym[7 - u] = (int32_t)s0[u];
            sym[3 - u] = (int32_t)s1[u];
            idx[7 - u] = (int32_t)i0[u];
            idx[3 - u] = (int32_t)i1[u];
        }
        __builtin_amdgcn_sched_barrier(0);
    };
    auto store_words = [&]() { sp.store_round(); };
    // State-independent values of one round (positions k0 .. k0+7,
    // last to first): the slot's (start, f), the reciprocal of f,
    // whether the position holds an ordinary symbol of a valid row,
    // and the round's symbols and indexes for the general puts.
    struct Pre {
        uint32_t start[kRound], f[kRound];
        double rcp[kRound];
        int32_t sym[kRound], idx[kRound];
        uint32_t fast;   // bit u: position u is fast (one register, not eight lane masks)
    };
    // Written phase by phase across the round's positions (all metadata
    // reads, then all pair reads, then each step of the reciprocal for all
    // eight), so that the eight independent chains interleave instead of
    // each waiting on its own latencies in turn.
    auto pre = [&](const int32_t (&sym)[kRound], const int32_t (&idx)[kRound], uint32_t k0,
                   Pre &P) {
        RowMeta m[kRound];
#pragma unroll
        for (int u = 0; u < kRound; ++u)
            m[u] = tab.meta(min((uint32_t)idx[u], K - 1));
        uint32_t pr[kRound];
        P.fast = 0;
#pragma unroll
        for (int u = 0; u < kRound; ++u) {
            const uint32_t mv = m[u].mvf & 0xFFFFu;
            // s - offset wraps mod 2^32 into [0, mv) only on rows whose
            // fast bound is 0
            const uint32_t w = (uint32_t)sym[u] - (uint32_t)m[u].offset;
            const bool fast = (w < (m[u].mvf >> 16)) & ((uint32_t)idx[u] < K) & valid(k0 + u);
            P.fast |= fast ? (1u << u) : 0u;
            pr[u] = tab.template load<uint32_t>(m[u].base + 4 * min(w, mv));
            P.sym[u] = sym[u];
            P.idx[u] = idx[u];
        }
        double fd[kRound], e[kRound];
#pragma unroll
        for (int u = 0; u < kRound; ++u) {
            P.start[u] = pr[u] & 0xFFFFu;
            P.f[u] = pr[u] >> 16;
            fd[u] = (double)P.f[u];
        }
        // the reciprocal of reciprocal(): the hardware estimate and two
        // Newton-Raphson steps, each applied to all positions in turn
#pragma unroll
        for (int u = 0; u < kRound; ++u)
            P.rcp[u] = __builtin_amdgcn_rcp(fd[u]);
#pragma unroll
        for (int it = 0; it < 2; ++it) {
#pragma unroll
            for (int u = 0; u < kRound; ++u)
                e[u] = __builtin_fma(-fd[u], P.rcp[u], 1.0);
#pragma unroll
            for (int u = 0; u < kRound; ++u)
                P.rcp[u] = __builtin_fma(P.rcp[u], e[u], P.rcp[u]);
        }
    };
    // Steps k .. k+15 (two rounds) into a pair buffer: 64 contiguous bytes
    // per array, whose reverse order is the steps' order.  A window that
    // starts before the wave's buffer (the offset wraps) reads 0; one that
    // starts before the lane reads the previous lane's values: only for
    // steps that are no positions.
    auto load_pair = [&](int32_t (&sym)[2 * kRound], int32_t (&idx)[2 * kRound], uint32_t k) {
        const uint32_t lo = pbase + 4 * (R8 - 2 * kRound - k);
        u32x4 sv[4], iv[4];
#pragma unroll
        for (int q = 0; q < 4; ++q)
            sv[q] = buf_load4(rsym, lo + 16 * q);
#pragma unroll
        for (int q = 0; q < 4; ++q)
            iv[q] = buf_load4(ridx, lo + 16 * q);
#pragma unroll
        for (int q = 0; q < 4; ++q)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                sym[15 - 4 * q - e] = (int32_t)sv[q][e];
                idx[15 - 4 * q - e] = (int32_t)iv[q][e];
            }
        __builtin_amdgcn_sched_barrier(0);
    };
    // One round of positions k0 .. k0+7 on P, with the next round's
    // state-independent work (from sym/idx into Pn) in the same
    // straight-line block, where it fills the chain's latency.  The
    // chain assumes every position fast; a round where that is not so
    // for some lane (an escape, a bad index, a lane end, a lane near
    // the end of its segment) is redone from its start state with
    // the general puts.  The round's loads follow its stores: the symbols
    // and indexes of the round three ahead into the buffer just used, or
    // (PAIR) whatever `mem` issues.
    auto round = [&](const Pre &P, uint32_t k0, int32_t (&sym)[kRound], int32_t (&idx)[kRound],
                     Pre &Pn, auto &&mem) {
        // room for three words per position: the fast steps need no check
        const bool room = sp.cb + 4 * (2 + 3 * kRound) < sp.capb;
        const uint64_t x0 = x;
        const uint32_t cb_start = sp.cb;
        pre(sym, idx, k0 + kRound, Pn);
        if (__builtin_expect(__all(P.fast == (1u << kRound) - 1), 1)) {
#pragma unroll
            for (int u = 0; u < kRound; ++u) {
                const bool need = (uint32_t)(x >> 32) >= (P.f[u] << (31 - kPrecision));
                *sp.slot((sp.cb - sp.cb0) >> 2) = (uint32_t)x;
                sp.cb += need ? 4u : 0u;
                x = need ? (x >> 32) : x;
                x = reg_step(x, P.start[u], P.f[u], P.rcp[u]);
            }
        } else {
            // Some lane holds a position off the common path.  Per
            // position, the lanes concerned (a wave-uniform branch, taken
            // only where one of them is) put an escape's groups and count
            // and take the slot pair of its REG put; a position that is no
            // position (padding before the lane's first round is full, a
            // round past its end) or holds a bad index takes the identity
            // step start 0, f = 2^16 (x unchanged, never renormalised).
            // Every spilled word goes to the ring (at most 3 a position).
#pragma unroll
            for (int u = 0; u < kRound; ++u) {
                uint32_t st = P.start[u], fu = P.f[u];
                double ru = P.rcp[u];
                const bool off = ((P.fast >> u) & 1u) == 0u;
                if (__ballot(off) != 0) {
                    if (off) {
                        st = 0u;
                        fu = kTotal;
                        ru = 1.0 / kTotal;
                        if (valid(k0 + u)) {
                            if ((uint32_t)P.idx[u] < K) {
                                uint32_t pr;
                                const int ec = encode_prefix<TPB>(P.sym[u], tab.meta(P.idx[u]),
                                                                  tab, x, sp, pr);
                                lerr = lerr ? lerr : ec;
                                st = pr & 0xFFFFu;
                                fu = pr >> 16;
                                ru = reciprocal(fu);
                            } else {
                                lerr = lerr ? lerr : RANS_E_INDEX;
                            }
                        }
                    }
                }
                const bool need = (uint32_t)(x >> 32) >= (fu << (31 - kPrecision));
                *sp.slot(min((sp.cb - sp.cb0) >> 2, kEncRing - 1)) = (uint32_t)x;
                sp.cb += need ? 4u : 0u;
                x = need ? (x >> 32) : x;
                x = reg_step(x, st, fu, ru);
            }
        }
        // A lane near the end of its segment (whose spills need checks), or
        // a round holding a split cut, redoes the round from its start.
        if (__builtin_expect(!__all(room & (cut_k >= k0 + kRound)), 0)) {
            x = x0;
            sp.cb = cb_start;
            // the fast step is committed where it applies; the other
            // lanes take the slow puts
#pragma unroll
            for (int u = 0; u < kRound; ++u) {
                const bool fast = ((P.fast >> u) & 1u) & room;
                const bool need = (uint32_t)(x >> 32) >= (P.f[u] << (31 - kPrecision));
                const uint64_t xn =
                    reg_step(need ? (x >> 32) : x, P.start[u], P.f[u], P.rcp[u]);
                *sp.slot(min((sp.cb - sp.cb0) >> 2, kEncRing - 1)) = (uint32_t)x;
                sp.cb += (fast & need) ? 4u : 0u;
                x = fast ? xn : x;
                const bool slow = !fast & valid(k0 + u);
                if (__builtin_expect(__ballot(slow) != 0, 0)) {
                    if (slow) {
                        int ec = RANS_E_INDEX;
                        if ((uint32_t)P.idx[u] < K)
                            ec = encode_slow<TPB>(P.sym[u], tab.meta(P.idx[u]), tab, x, sp);
                        lerr = lerr ? lerr : ec;
                    }
                }
                while (cut_k == k0 + u)   // (cuts may share a position)
                    record_cut();
            }
        }
        __builtin_amdgcn_sched_barrier(0);
        // ---- memory phase: this round's words, then its loads
        store_words();
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (PAIR)
            mem();
        else
            load_next(sym, idx, k0 + 3 * kRound);
    };
    Pre pa, pb;
    if constexpr (PAIR) {
        // pair buffers: rounds 0-1 in (s0, i0), 2-3 in (s1, i1); a pair is
        // loaded by the second round of the pair before the one that
        // first reads it (two rounds ahead), into the buffer just freed
        int32_t s0[2 * kRound], i0[2 * kRound], s1[2 * kRound], i1[2 * kRound];
        auto half = [](int32_t (&v)[2 * kRound], int h) -> int32_t (&)[kRound] {
            return *reinterpret_cast<int32_t (*)[kRound]>(v + kRound * h);
        };
        auto none = [] {};
        store_words();
        __builtin_amdgcn_sched_barrier(0);
        load_pair(s0, i0, 0);
        load_pair(s1, i1, 2 * kRound);
        pre(half(s0, 0), half(i0, 0), 0, pa);
        for (uint32_t k0 = 0; k0 < R8; k0 += 4 * kRound) {
            round(pa, k0, half(s0, 1), half(i0, 1), pb, none);
            round(pb, k0 + kRound, half(s1, 0), half(i1, 0), pa,
                  [&] { load_pair(s0, i0, k0 + 4 * kRound); });
            if (k0 + 2 * kRound >= R8)   // (this lane's rounds are done)
                break;
            round(pa, k0 + 2 * kRound, half(s1, 1), half(i1, 1), pb, none);
            round(pb, k0 + 3 * kRound, half(s0, 0), half(i0, 0), pa,
                  [&] { load_pair(s1, i1, k0 + 6 * kRound); });
        }
    } else {
        // prologue: three phases of the same shape (their stores carry
        // stale ring words to positions that later words overwrite);
        // rounds 0 and 1 are loaded, round 0 prepared, round 2 loaded
        store_words();
        __builtin_amdgcn_sched_barrier(0);
        load_next(sa, ia, 0);
        store_words();
        __builtin_amdgcn_sched_barrier(0);
        load_next(sb, ib, kRound);
        pre(sa, ia, 0, pa);
        __builtin_amdgcn_sched_barrier(0);
        store_words();
        __builtin_amdgcn_sched_barrier(0);
        load_next(sa, ia, 2 * kRound);
        // both rounds always run (positions past the lane are skipped
        // inside), so every path back to the loop head passes both phases
        for (uint32_t k0 = 0; k0 < R8; k0 += 2 * kRound) {
            round(pa, k0, sb, ib, pb, [] {});
            round(pb, k0 + kRound, sa, ia, pa, [] {});
        }
    }
    while (cut_s >= 1)   // an empty lane: every cut holds the start state
        record_cut();
    if (sp.overflow) {
        lerr = lerr ? lerr : RANS_E_CAPACITY;
        sp.cb = sp.capb - 8;
    }
    buf_store(sp.scr, sp.top - 8 - sp.cb, 0, (int32_t)(uint32_t)x);
    buf_store(sp.scr, sp.top - 4 - sp.cb, 0, (int32_t)(uint32_t)(x >> 32));
    // (the final state is stored after every memory phase)
    words = sp.cb / 4 + 2;
    return LaneResult{words, lerr};
}

// Lane j coded from tables read in the workspace (a set over the LDS budget):
// the same puts as above, one position at a time, each spilled word stored
// straight to the lane's scratch segment.  A short loop with few registers,
// so that the round-based form keeps its register budget to itself.
template <int TPB>
__device__ __forceinline__ LaneResult encode_lane_simple(const EncodeArgs &a, const GlobalTab &tab,
                                                         uint32_t K, uint32_t L, uint32_t j,
                                                         uint64_t bw, Rsrc rsym, Rsrc ridx,
                                                         const Spill<TPB> &sp)
{
    int lerr = 0;
    const uint64_t b = lane_begin(a.n, L, j), e = lane_begin(a.n, L, j + 1);
    const uint32_t nj = (uint32_t)(e - b);
    const uint32_t capb = 4 * (2 * nj + 4);   // the last 2 words hold the final state
    uint32_t cb = 0;
    bool overflow = false;
    uint64_t x = kStateLow;
    // word k of the lane goes to byte offset top - 4 - 4k
    auto renorm = [&](bool spill) {
        if (spill) {
            overflow = overflow | (cb + 8 >= capb);
            if (cb + 8 < capb)
                buf_store(sp.scr, sp.top - 4 - cb, 0, (int32_t)(uint32_t)x);
            cb += 4;
            x >>= 32;
        }
    };
    const uint32_t pl = a.pieces_log2, npieces = 1u << pl;
    int32_t cut_s = (int32_t)npieces - 1;
    auto record_cut = [&]() {
        uint32_t *m = a.split_meta + 3ull * ((uint64_t)(npieces - 1) * j + cut_s - 1);
        m[0] = (uint32_t)x;
        m[1] = (uint32_t)(x >> 32);
        m[2] = cb >> 2;
        --cut_s;
    };
    for (uint32_t k = 0; k < nj; ++k) {
        const uint64_t c = e - 1 - k;   // positions are coded last to first
        const uint32_t off = (uint32_t)(4 * (c - bw));
        const int32_t sym = buf_load(rsym, off, 0), r = buf_load(ridx, off, 0);
        if ((uint32_t)r >= K) {
            lerr = lerr ? lerr : RANS_E_INDEX;
        } else {
            const RowMeta m = tab.meta((uint32_t)r);
            const uint32_t mv = m.mvf & 0xFFFFu;
            const int64_t v = (int64_t)sym - (int64_t)m.offset;
            const bool esc = (uint64_t)v >= (uint64_t)mv;
            uint64_t raw = v < 0 ? (uint64_t)(-2 * v - 1) : (uint64_t)(2 * (v - (int64_t)mv));
            if (esc && raw >= (1ull << 31)) {
                lerr = lerr ? lerr : RANS_E_SYMBOL_RANGE;
                raw = 0;
            }
            const uint32_t bits = raw ? 64u - (uint32_t)__clzll(raw) : 0u;
            const uint32_t nb = esc ? (bits + kBypassBits - 1) / kBypassBits : 0u;
            // BITS puts: groups nb-1 .. 0, then the count nb (k = nb); then the REG put
            for (uint32_t k = 0; k < nb + (esc ? 1u : 0u); ++k) {
                const uint32_t b4 = k == nb ? nb : (uint32_t)(raw >> (kBypassBits * (nb - 1 - k))) & 15u;
                renorm(x >= (1ull << (63 - kBypassBits)));
                x = (x << kBypassBits) | b4;
            }
            const uint32_t pr = tab.template load<uint32_t>(m.base + 4 * (esc ? mv : (uint32_t)v));
            const uint32_t f = pr >> 16;
            renorm(x >= ((uint64_t)f << (63 - kPrecision)));
            x = reg_step(x, pr & 0xFFFFu, f, reciprocal(f));
        }
        while (cut_s >= 1 && piece_begin(b, e, pl, (uint32_t)cut_s) == c)   // (cuts may share a position)
            record_cut();
    }
    while (cut_s >= 1)   // an empty lane: every cut holds the start state
        record_cut();
    if (overflow) {
        lerr = lerr ? lerr : RANS_E_CAPACITY;
        cb = capb - 8;
    }
    buf_store(sp.scr, sp.top - 8 - cb, 0, (int32_t)(uint32_t)x);
    buf_store(sp.scr, sp.top - 4 - cb, 0, (int32_t)(uint32_t)(x >> 32));
    return LaneResult{cb / 4 + 2, lerr};
}

// The buffers of the wave coding lanes j0 .. j1-1, and lane j's spill state:
// the wave's symbols and indexes, and its lanes' scratch segments (lane j
// owns words [2 b_j + 4 j, 2 e_j + 4 (j+1)) of the scratch area).
template <int TPB>
struct WaveBufs {
    Rsrc rsym, ridx;
    uint64_t bw;
    Spill<TPB> sp;
};

template <int TPB>
__device__ __forceinline__ WaveBufs<TPB> wave_bufs(const EncodeArgs &a, uint32_t L, uint32_t j0,
                                                   uint32_t j1, uint32_t j)
{
    extern __shared__ __align__(16) uint8_t lds[];
    uint32_t *scratch = reinterpret_cast<uint32_t *>(a.ws + ws_scratch_offset(a.num_tables, a.stride));
    WaveBufs<TPB> w;
    w.bw = lane_begin(a.n, L, j0);
    const uint64_t ew = lane_begin(a.n, L, j1);
    w.rsym = make_rsrc(a.symbols + w.bw, (uint32_t)(4 * (ew - w.bw)));
    w.ridx = make_rsrc(a.indexes + w.bw, (uint32_t)(4 * (ew - w.bw)));
    const uint64_t sw0 = 2 * w.bw + 4ull * j0, sw1 = 2 * ew + 4ull * j1;
    w.sp.scr = make_rsrc(scratch + sw0, (uint32_t)(4 * (sw1 - sw0)));
    w.sp.ring = reinterpret_cast<uint32_t *>(lds + kEncTableBudget) + threadIdx.x;
    const uint64_t e = lane_begin(a.n, L, min(j + 1, L));
    w.sp.top = (uint32_t)(4 * (2 * e + 4ull * min(j + 1, L) - sw0));
    return w;
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

// Block start of both encode kernels: check the prepared workspace, stage the
// encoder table set into LDS (when it fits), and refuse a set with an invalid
// row.  `misc[0]` is a zeroed LDS word for the block OR.  Returns the call's
// error (the same in every lane; scalar, it keeps the buffer descriptors and
// loops after it uniform for the compiler).
template <int TPB>
__device__ __forceinline__ int encode_block_start(const EncodeArgs &a, WsHeader *hdr,
                                                  const uint8_t *tab, uint8_t *lds, uint32_t *misc,
                                                  bool &in_lds)
{
    const uint32_t tid = threadIdx.x;
    int herr = 0;
    if (hdr->magic != kMagic || hdr->num_tables != (uint32_t)a.num_tables ||
        hdr->cdf_stride != (uint32_t)a.stride)
        herr = RANS_E_ARG;
    else if (lds_address_of(lds) != 0)   // table offsets are used as LDS addresses
        herr = RANS_E_HIP;
    const uint32_t K = (uint32_t)a.num_tables;
    in_lds = hdr->enc_lds != 0;
    stage_tables<TPB>(lds, tab, (!herr && in_lds) ? hdr->enc_bytes : 0u);
    __syncthreads();
    int bad = 0;
    if (!herr) {
        const GlobalTab gt{tab};
        for (uint32_t r = tid; r < K; r += TPB)
            bad |= ((in_lds ? lds_meta(r) : gt.meta(r)).lut & kRowInvalid) ? 1 : 0;
    }
    __syncthreads();
    bad = block_or(&misc[0], bad);
    if (!herr && bad)
        herr = RANS_E_TABLE;
    if (herr && blockIdx.x == 0 && tid == 0)
        record_error(hdr, herr);
    return __builtin_amdgcn_readfirstlane(herr);
}

// After coding, coding wave t (lanes j0 + lane, `active` ones) publishes its
// word total, finds its offset by a look-back over earlier waves, writes its
// lanes' header entries and copies their words into the container.
template <int S>
__device__ __forceinline__ void publish_and_copy(const EncodeArgs &a, WsHeader *hdr,
                                                 uint64_t *flags, uint32_t t, uint32_t nwork,
                                                 uint32_t lane, uint32_t j, bool active,
                                                 const Spill<S> &sp, uint32_t words, int lerr)
{
    const uint32_t L = a.lanes;
    if (lerr)
        record_error(hdr, lerr);
    // The lane's first 64 words are read back from its scratch segment now:
    // their loads do not depend on the offset the look-back finds, and their
    // latency passes while it waits.
    const uint32_t src = sp.top - 4 * words;   // the lane's first word in sp.scr
    const uint32_t kt = words & ~3u;           // first word of the last, partial group
    u32x4 v0[16];
    uint32_t t0[3];
    if (active) {
#pragma unroll
        for (int i = 0; i < 16; ++i)
            if (4 * i + 4 <= words)
                v0[i] = buf_load4(sp.scr, src + 16 * i);
#pragma unroll
        for (int e = 0; e < 3; ++e)
            if (kt < 64 && kt + e < words)
                t0[e] = (uint32_t)buf_load(sp.scr, src + 4 * (kt + e), 0);
    }
    // (a compiler barrier: the loads would otherwise sink below the
    // look-back to where their values are used, and wait there)
    asm volatile("" ::: "memory");

    // ---- wave scan and look-back over earlier waves -----------------------
    // Every wave publishes its aggregate, then reads the flags of the 256
    // waves before it at once (four per wavefront lane): the nearest
    // inclusive flag ends the walk once every flag after it is
    // published, and the values up to it are summed across the wave.
    // (Inclusive flags spread one window per round trip when many
    // waves finish together, so the window is made wide.)
    // A flag carries all it says in its own 64 bits, so the flags are
    // relaxed device-scope atomics: no cache writeback or invalidation
    // per publication or poll (spinning waves would otherwise keep
    // flushing the L2 that the working waves read from).  Its look-back
    // waits only for waves of lower-numbered blocks.  Workgroups are
    // dispatched in index order, so those have all started and none of them
    // waits on this one (a per-wave ticket counter would guarantee the same
    // without relying on dispatch order, but its one contended atomic cost
    // about 10 us).
    const uint32_t incl = wave_inclusive_scan(words, lane);
    const uint64_t agg = __shfl(incl, kWave - 1, kWave);
    uint64_t prefix = 0;
    if (lane == 0)
        __hip_atomic_store(&flags[t], (t == 0 ? kFlagInclusive : kFlagAggregate) | agg,
                           __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (t > 0) {
        constexpr int kLook = 4;   // flags per lane per round trip
        constexpr uint32_t kWindow = kLook * kWave;
        int32_t k = (int32_t)t;   // this window covers waves k-1 .. k-kWindow
        uint32_t spins = 0;
        while (true) {
            // flag at distance d = 64 i + lane behind k
            uint64_t fv[kLook];
#pragma unroll
            for (int i = 0; i < kLook; ++i) {
                const int32_t p = k - 1 - (int32_t)(kWave * i + lane);
                fv[i] = p >= 0 ? __hip_atomic_load(&flags[p], __ATOMIC_RELAXED,
                                                   __HIP_MEMORY_SCOPE_AGENT)
                               : kFlagInclusive;
            }
            // the nearest inclusive flag (kWindow: none in this window)
            uint32_t dstar = kWindow;
#pragma unroll
            for (int i = kLook - 1; i >= 0; --i) {
                const uint64_t im = __ballot((fv[i] >> 62) == 2);
                if (im)
                    dstar = kWave * i + (uint32_t)__builtin_ctzll(im);
            }
            // every flag up to it must be published
            bool ready = true;
#pragma unroll
            for (int i = 0; i < kLook; ++i) {
                const uint64_t rm = __ballot((fv[i] >> 62) != 0);
                const uint32_t lo = kWave * i;
                const uint64_t need = dstar < lo ? 0ull
                                      : dstar >= lo + kWave - 1 ? ~0ull
                                                                : (2ull << (dstar - lo)) - 1;
                ready = ready & ((rm & need) == need);
            }
            if (!ready) {
                if (++spins > kSpinLimit) {   // never expected: bail out, flag it
                    if (lane == 0)
                        record_error(hdr, RANS_E_HIP);
                    break;
                }
                __builtin_amdgcn_s_sleep(1);
                continue;
            }
            uint64_t v = 0;
#pragma unroll
            for (int i = 0; i < kLook; ++i)
                v += (kWave * i + lane <= dstar) ? (fv[i] & kFlagValueMask) : 0;
            for (int off = 1; off < kWave; off <<= 1)
                v += __shfl_xor(v, off, kWave);
            prefix += v;
            if (dstar < kWindow)
                break;
            k -= (int32_t)kWindow;
        }
        if (lane == 0)
            __hip_atomic_store(&flags[t], kFlagInclusive | (prefix + agg), __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
    }
    if (lane == 0 && t == nwork - 1) {
        a.stream[0] = L;
        __hip_atomic_store(&hdr->total_words, prefix + agg, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
    }

    // ---- header entry and compaction --------------------------------------
    // The wave's lanes fill container words [1 + L + prefix, + agg); the
    // output buffer ends at the capacity, so nothing is written past it.
    // Each lane reads back only the scratch words it stored itself,
    // sixty-four per round trip (all loads issued before any store; the
    // first sixty-four above), and stores whole 16-byte groups of its own
    // words, then its last one to three words one by one.  Accesses are
    // masked per lane (a lane without words for a group sends no request).
    const uint64_t wbase =
        1ull + L + (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)prefix) +
        ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(prefix >> 32)) << 32);
    const uint64_t wroom = a.capacity > wbase ? a.capacity - wbase : 0;
    const Rsrc rout = make_rsrc(a.stream + (wroom ? wbase : 0),
                                rsrc_bytes(4 * wroom));
    if (active) {
        const uint64_t end = prefix + incl;
        a.stream[1 + j] = (uint32_t)end;
        const uint32_t ob = 4 * (incl - words);   // the lane's first word in rout
#pragma unroll
        for (int i = 0; i < 16; ++i)
            if (4 * i + 4 <= words)
                buf_store4(rout, ob + 16 * i, v0[i]);
#pragma unroll
        for (int e = 0; e < 3; ++e)
            if (kt < 64 && kt + e < words)
                buf_store(rout, ob + 4 * (kt + e), 0, (int32_t)t0[e]);
        for (uint32_t k0 = 64; k0 < words; k0 += 64) {
            u32x4 v[16];
            uint32_t tw[3];
#pragma unroll
            for (int i = 0; i < 16; ++i)
                if (k0 + 4 * i + 4 <= words)
                    v[i] = buf_load4(sp.scr, src + 4 * k0 + 16 * i);
            const bool tail = kt >= k0 && kt < k0 + 64;
#pragma unroll
            for (int e = 0; e < 3; ++e)
                if (tail && kt + e < words)
                    tw[e] = (uint32_t)buf_load(sp.scr, src + 4 * (kt + e), 0);
#pragma unroll
            for (int i = 0; i < 16; ++i)
                if (k0 + 4 * i + 4 <= words)
                    buf_store4(rout, ob + 4 * (k0 + 4 * i), v[i]);
#pragma unroll
            for (int e = 0; e < 3; ++e)
                if (tail && kt + e < words)
                    buf_store(rout, ob + 4 * (kt + e), 0, (int32_t)tw[e]);
        }
    }
}

// Block end of both encode kernels: the last block to finish publishes the
// status and the container length, and clears the bookkeeping (look-back
// flags, error, totals) for the next call.  `misc[1]` is an LDS word.
template <int TPB>
__device__ __forceinline__ void encode_block_end(const EncodeArgs &a, WsHeader *hdr,
                                                 uint64_t *flags, int herr, uint32_t nwork,
                                                 uint32_t *misc)
{
    const uint32_t tid = threadIdx.x;
    __syncthreads();
    if (tid == 0) {
        __threadfence();
        const uint32_t old = atomicAdd(&hdr->done, 1u);
        misc[1] = (old == gridDim.x - 1) ? 1u : 0u;
    }
    __syncthreads();
    if (misc[1]) {
        __threadfence();
        if (!herr)
            for (uint32_t k = tid; k < nwork; k += TPB)
                flags[k] = 0;
        if (tid == 0) {
            const uint64_t total = 1ull + a.lanes + hdr->total_words;
            int err = hdr->err;
            if (!err && total > a.capacity)
                err = RANS_E_CAPACITY;
            *a.status = err;
            *a.stream_words = herr ? 0ull : total;
            hdr->err = 0;
            hdr->total_words = 0;
            hdr->done = 0;
            __threadfence();
        }
    }
}

template <int TPB, int CW, bool PAIR>
__global__ __launch_bounds__(TPB) void encode_kernel(EncodeArgs a)
{
    extern __shared__ __align__(16) uint8_t lds[];
    // block bookkeeping after the table set and the rings: [0] flag OR, [1] last block
    uint32_t *misc = reinterpret_cast<uint32_t *>(lds + kEncTableBudget + kEncRing * 4 * TPB);

    WsHeader *hdr = reinterpret_cast<WsHeader *>(a.ws);
    const uint8_t *tab = a.ws + ws_enc_offset(a.num_tables, a.stride);
    uint64_t *flags = reinterpret_cast<uint64_t *>(a.ws + ws_flags_offset());
    const uint32_t tid = threadIdx.x;
    const uint32_t lane = tid & (kWave - 1);
    const uint32_t L = a.lanes;
    const uint32_t lpw = enc_lanes_per_wave(L);
    const uint32_t nwork = enc_waves(L);
    const uint32_t wave = __builtin_amdgcn_readfirstlane(tid / kWave);   // coding waves 0 .. CW-1
    const uint32_t K = (uint32_t)a.num_tables;

    if (tid == 0)
        misc[0] = 0u;
    bool in_lds;
    const int herr = encode_block_start<TPB>(a, hdr, tab, lds, misc, in_lds);
    if (!herr && wave < CW) {
        const uint32_t t = blockIdx.x * CW + wave;
        if (t < nwork) {
            // the wave codes lanes j0 .. j0 + lpw - 1, one per wavefront lane
            const uint32_t j0 = t * lpw, j1 = min(j0 + lpw, L);
            const uint32_t j = j0 + lane;
            const bool active = lane < lpw && j < L;
            const WaveBufs<TPB> wb = wave_bufs<TPB>(a, L, j0, j1, j);
            uint32_t words = 0;
            int lerr = 0;
            if (active) {
                const LaneResult lr =
                    in_lds ? encode_lane<TPB, LdsTab, PAIR>(a, LdsTab{}, K, L, j, wb.bw, wb.rsym,
                                                            wb.ridx, wb.sp)
                           : encode_lane_simple<TPB>(a, GlobalTab{tab}, K, L, j, wb.bw, wb.rsym,
                                                     wb.ridx, wb.sp);
                words = lr.words;
                lerr = lr.err;
            }
            publish_and_copy(a, hdr, flags, t, nwork, lane, j, active, wb.sp, words, lerr);
        }
    }
    encode_block_end<TPB>(a, hdr, flags, herr, nwork, misc);
}

// ---- one coding wave per CU --------------------------------------------------
//
// With at most 4096 lanes every CU holds a single coding wave of at most 16
// lanes, and the kernel takes as long as that wave's dependent chains.  The
// state-independent work of a position -- loading its symbol and index, the
// row metadata, the slot's (start, f), the reciprocal of f -- would run on the
// same wave at 16 of 64 threads.  Here the block's three other waves, on the
// CU's other SIMDs, do it for the coding wave: for every step of a chunk of
// 48 steps and every lane, they write one 16-byte entry to LDS,
//   an ordinary symbol of a valid row:  (1/f as fp64, f, start);
//   a step that is no position (padding, past the lane's end): the identity
//     step (2^-16, 2^16, 0), which leaves the state unchanged and never
//     renormalises;
//   anything else (an escape, a bad index, a row whose values may overflow
//     int32):  (symbol, index, 0, 0);
// and set, per step of the chunk, one bit when some lane's entry is of the
// last kind.  Two entry buffers alternate: one barrier per chunk hands a
// filled buffer to the coding wave and the one it has finished back to the
// producers.  The coding wave reads a round's entries during the round
// before and runs the state chain; at a step whose bit is set, the lanes
// concerned first put the escape's groups and count (a scalar test per step
// of such a round, nothing in the others).  Whether a lane may reach the end
// of its scratch segment, or holds a split cut, is asked once per chunk; only
// then is a round checked afterwards and redone with checked puts.  The
// puts, their order and the container are those of encode_lane.
constexpr uint32_t kPcLanes = 16;                           // lanes of a coding wave, at most
constexpr uint32_t kPcChunkRounds = 6;
constexpr uint32_t kPcChunk = kPcChunkRounds * kRound;      // steps per chunk
constexpr int kPcThreads = 4 * kWave;
constexpr uint32_t kPcRing = kEncTableBudget;               // the coding wave's word rings
constexpr uint32_t kPcEntries = kPcRing + kEncRing * 4 * kWave;
constexpr uint32_t kPcEntryBuf = kPcChunk * kPcLanes * 16;
constexpr uint32_t kPcMisc = kPcEntries + 2 * kPcEntryBuf;  // [0] flag OR, [1] last block,
                                                            // [2 + 2b, 3 + 2b] step bits of buffer b
constexpr uint32_t kPcEscBuf = kPcChunk * kPcLanes * 4;
constexpr uint32_t kPcEsc = kPcMisc + 32;                   // escaped values of three chunks
constexpr uint32_t kPcLdsBytes = kPcEsc + 3 * kPcEscBuf;
static_assert(kPcLdsBytes <= kLdsBytes, "encoder LDS over budget");
static_assert(kPcEntries % 16 == 0, "entries are 16-byte LDS accesses");
static_assert(lanes_per_wave_for(4096, kCodingCUs) <= kPcLanes, "coding wave too wide");
static_assert((kPcChunk / 4) * kPcLanes == kPcThreads - kWave, "one quad of steps per producer");
static_assert(kPcChunkRounds % 2 == 0, "rounds run in pairs");
static_assert(kPcChunk <= 64, "step bits of a chunk in two words");

__device__ inline uint32_t pc_entry(uint32_t buf, uint32_t step, uint32_t l)
{
    return kPcEntries + buf * kPcEntryBuf + (step * kPcLanes + l) * 16;
}
// Step `step` of chunk c, lane l: the zig-zag value + 1 of an escaped value
// whose entry is its escape slot's REG put, else 0.  Three buffers, as the
// producers fill chunk c+2 while the coding wave's last round of chunk c may
// still read chunk c's.
__device__ inline uint32_t pc_esc(uint32_t chunk, uint32_t step, uint32_t l)
{
    return kPcEsc + (chunk % 3u) * kPcEscBuf + (step * kPcLanes + l) * 4;
}
__device__ inline double entry_rcp(const u32x4 &e)
{
    return __builtin_bit_cast(double, (uint64_t)e[0] | ((uint64_t)e[1] << 32));
}

// Where lane j's steps lie: step k codes position b + R8 - 1 - k, R8 = the
// lane's length rounded up to whole rounds; steps below pad = R8 - nj and
// from R8 on are no positions.  pbase: byte offset of position b in the
// wave's buffers.
struct LaneSteps {
    uint64_t b, e;
    uint32_t nj, R8, pad, pbase;
};
__device__ inline LaneSteps lane_steps(uint64_t n, uint32_t L, uint32_t j, uint64_t bw)
{
    LaneSteps s;
    s.b = lane_begin(n, L, j);
    s.e = lane_begin(n, L, j + 1);
    s.nj = (uint32_t)(s.e - s.b);
    s.R8 = (s.nj + kRound - 1) / kRound * kRound;
    s.pad = s.R8 - s.nj;
    s.pbase = (uint32_t)(4 * (s.b - bw));
    return s;
}

// Producer input: the symbols and indexes of steps 4q .. 4q+3 of a chunk for
// one lane (positions c .. c+3 as one 16-byte load per array, c = the
// position of step 4q+3; a quad past the lane reads other lanes' values or
// zeros, only for steps that are no positions).
struct PcIn {
    u32x4 sv, iv;
};
__device__ inline PcIn pc_load(const LaneSteps &ls, Rsrc rsym, Rsrc ridx, uint32_t chunk,
                               uint32_t q)
{
    const uint32_t k4 = chunk * kPcChunk + 4 * q;
    const uint32_t off = ls.pbase + 4 * (ls.R8 - 4 - k4);   // (wraps past the buffer: reads 0)
    return PcIn{buf_load4(rsym, off), buf_load4(ridx, off)};
}

// Producer: the entries of those four steps of lane l, and their step bits.
__device__ __forceinline__ void pc_fill(const LaneSteps &ls, const PcIn &in, uint32_t K,
                                        uint32_t chunk, uint32_t q, uint32_t l,
                                        uint32_t *step_bits)
{
    const uint32_t buf = chunk & 1u;
    const uint32_t k4 = chunk * kPcChunk + 4 * q;
    uint32_t offs = 0;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const uint32_t k = k4 + u;
        const int32_t sym = (int32_t)in.sv[3 - u];
        const uint32_t idx = in.iv[3 - u];
        const RowMeta m = lds_meta(min(idx, K - 1));
        const uint32_t mv = m.mvf & 0xFFFFu;
        // s - offset wraps mod 2^32 into [0, mv) only on rows whose fast
        // bound is 0
        const uint32_t w = (uint32_t)sym - (uint32_t)m.offset;
        const bool fast = (w < (m.mvf >> 16)) & (idx < K);
        const uint32_t pr = lds_load<uint32_t>(m.base + 4 * min(w, mv));
        const uint32_t f = pr >> 16;
        const double r = reciprocal(f);
        const uint64_t rb = __builtin_bit_cast(uint64_t, r);
        const bool valid = k >= ls.pad && k < ls.R8;
        // an escaped value in range on a row whose values fit int32 (fast
        // bound mv): the entry is the escape slot's REG put (pr was read at
        // mv) and the value goes beside it
        const int64_t v = (int64_t)sym - (int64_t)m.offset;
        const uint64_t raw = v < 0 ? (uint64_t)(-2 * v - 1) : (uint64_t)(2 * (v - (int64_t)mv));
        const bool esc = !fast & (idx < K) & ((m.mvf >> 16) != 0u) & (raw < (1ull << 31));
        u32x4 ent;
        if (!valid)
            ent = u32x4{0u, 0x3EF00000u, kTotal, 0u};   // 2^-16, 2^16, 0
        else if (fast | esc)
            ent = u32x4{(uint32_t)rb, (uint32_t)(rb >> 32), f, pr & 0xFFFFu};
        else
            ent = u32x4{(uint32_t)sym, idx, 0u, 0u};
        offs |= (valid & !fast) ? (1u << u) : 0u;
        lds_store<u32x4>(pc_entry(buf, 4 * q + u, l), ent);
        lds_store<uint32_t>(pc_esc(chunk, 4 * q + u, l), (valid & esc) ? (uint32_t)raw + 1u : 0u);
    }
    if (offs)   // steps 4q .. 4q+3 are bits 4q % 32 .. of word 4q / 32
        __hip_atomic_fetch_or(&step_bits[2 * buf + (4 * q) / 32], offs << ((4 * q) % 32),
                              __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}

// Where the coding wave's puts send a lane's spilled words.  Every put
// offers the state's low word; it is kept when `spill` holds, and the next
// put overwrites it otherwise.  The room for three words a position is asked
// before a round, so neither sink checks it.
struct RingSink {      // the lane's LDS ring (a round starts at slot 0)
    uint32_t a;        // LDS address of the slot for the next word
    __device__ inline void put(bool spill, uint32_t w)
    {
        lds_store<uint32_t>(a, w);
        a += spill ? 4u * kWave : 0u;
    }
};
struct ScratchSink {   // straight to the lane's scratch segment
    Rsrc scr;
    uint32_t o;        // byte offset of the next word (words go downwards)
    __device__ inline void put(bool spill, uint32_t w)
    {
        buf_store(scr, o, 0, (int32_t)w);
        o -= spill ? 4u : 0u;
    }
};

// The BITS puts of an escaped value raw < 2^31, last to first: its groups
// nb-1 .. 0, then the count nb, as in encode_prefix; put(spill, w) offers
// the state's low word.
template <class Put>
__device__ __forceinline__ void put_escape_groups(uint32_t raw, uint64_t &x, Put &&put)
{
    const uint32_t nb = raw ? (32u - (uint32_t)__clz(raw) + kBypassBits - 1) / kBypassBits : 0u;
    auto put_bits = [&](uint32_t b) {
        const bool spill = x >= (1ull << (63 - kBypassBits));
        put(spill, (uint32_t)x);
        x = spill ? (x >> 32) : x;
        x = (x << kBypassBits) | b;
    };
    for (uint32_t g = nb; g-- > 0;)
        put_bits((raw >> (kBypassBits * g)) & 15u);
    put_bits(nb);
}

// The puts of an escaped value (its groups, then its count) before its REG
// put, as in encode_prefix, with each spilled word going to `sink`, and the
// (start, f) pair of the REG put's slot.
template <class Sink>
__device__ __forceinline__ int pc_prefix(int32_t s, const RowMeta m, uint64_t &x, Sink &sink,
                                         uint32_t &pair)
{
    int err = 0;
    const uint32_t mv = m.mvf & 0xFFFFu;
    const int64_t v = (int64_t)s - (int64_t)m.offset;
    const bool esc = (uint64_t)v >= (uint64_t)mv;
    uint64_t raw = v < 0 ? (uint64_t)(-2 * v - 1) : (uint64_t)(2 * (v - (int64_t)mv));
    if (esc && raw >= (1ull << 31)) {
        err = RANS_E_SYMBOL_RANGE;
        raw = 0;
    }
    const uint32_t bits = raw ? 64u - (uint32_t)__clzll(raw) : 0u;
    const uint32_t nb = esc ? (bits + kBypassBits - 1) / kBypassBits : 0u;
    auto put_bits = [&](uint32_t b) {
        const bool spill = x >= (1ull << (63 - kBypassBits));
        sink.put(spill, (uint32_t)x);
        x = spill ? (x >> 32) : x;
        x = (x << kBypassBits) | b;
    };
    for (uint32_t g = nb; g-- > 0;)
        put_bits((uint32_t)(raw >> (kBypassBits * g)) & 15u);
    if (esc)
        put_bits(nb);
    pair = lds_load<uint32_t>(m.base + 4 * (esc ? mv : (uint32_t)v));
    return err;
}

__global__ __launch_bounds__(kPcThreads) void encode_pc_kernel(EncodeArgs a)
{
    extern __shared__ __align__(16) uint8_t lds[];
    uint32_t *misc = reinterpret_cast<uint32_t *>(lds + kPcMisc);
    uint32_t *step_bits = misc + 2;

    WsHeader *hdr = reinterpret_cast<WsHeader *>(a.ws);
    const uint8_t *tab = a.ws + ws_enc_offset(a.num_tables, a.stride);
    uint64_t *flags = reinterpret_cast<uint64_t *>(a.ws + ws_flags_offset());
    const uint32_t tid = threadIdx.x;
    const uint32_t lane = tid & (kWave - 1);
    const uint32_t L = a.lanes;
    const uint32_t lpw = enc_lanes_per_wave(L);
    const uint32_t nwork = enc_waves(L);
    const uint32_t wave = __builtin_amdgcn_readfirstlane(tid / kWave);   // 0 codes, 1..3 produce
    const uint32_t K = (uint32_t)a.num_tables;
    const uint32_t t = blockIdx.x;
    const uint32_t j0 = t * lpw, j1 = min(j0 + lpw, L);
    // rounds of the longest lane (a lane holds floor or ceil of n / L
    // positions), and chunks
    const uint32_t nr = (uint32_t)(((a.n + L - 1) / L + kRound - 1) / kRound);
    const uint32_t nch = (nr + kPcChunkRounds - 1) / kPcChunkRounds;

    // producers: thread p fills steps 4q .. 4q+3 of lane l of every chunk; the
    // first chunk's loads are issued before the tables are staged
    const uint32_t p = tid - kWave;
    const uint32_t pl = p % kPcLanes, pq = p / kPcLanes;
    const bool mine = wave > 0 && t < nwork && pl < lpw && j0 + pl < L;
    const uint32_t pj = min(j0 + pl, L - 1);
    const WaveBufs<kWave> pwb = wave_bufs<kWave>(a, L, j0, j1, pj);
    const LaneSteps pls = lane_steps(a.n, L, pj, pwb.bw);
    PcIn in0{};
    if (mine && nch > 0)
        in0 = pc_load(pls, pwb.rsym, pwb.ridx, 0, pq);

    if (tid < 6)
        misc[tid] = 0u;
    bool in_lds;
    const int herr = encode_block_start<kPcThreads>(a, hdr, tab, lds, misc, in_lds);
    if (!herr && t < nwork) {
        if (wave == 0) {
            const uint32_t j = j0 + lane;
            const bool active = lane < lpw && j < L;
            const WaveBufs<kWave> wb = wave_bufs<kWave>(a, L, j0, j1, j);
            Spill<kWave> sp = wb.sp;
            uint32_t words = 0;
            int lerr = 0;
            if (!in_lds) {
                if (active) {
                    const LaneResult lr = encode_lane_simple<kWave>(a, GlobalTab{tab}, K, L, j,
                                                                    wb.bw, wb.rsym, wb.ridx, sp);
                    words = lr.words;
                    lerr = lr.err;
                }
            } else {
                const LaneSteps ls = lane_steps(a.n, L, j, wb.bw);
                const LdsTab tb{};
                uint64_t x = kStateLow;
                sp.cb = 0;
                sp.cb0 = 0;
                sp.capb = 4 * (2 * ls.nj + 4);
                sp.overflow = false;
                // split records, as in encode_lane
                const uint32_t npieces = 1u << a.pieces_log2;
                int32_t cut_s = (int32_t)npieces - 1;
                auto cut_step = [&](int32_t s) -> uint32_t {
                    return ls.R8 - 1 - (uint32_t)(piece_begin(ls.b, ls.e, a.pieces_log2, (uint32_t)s) - ls.b);
                };
                uint32_t cut_k = (npieces > 1 && ls.nj > 0) ? cut_step(cut_s) : ~0u;
                auto record_cut = [&]() {
                    uint32_t *m = a.split_meta + 3ull * ((uint64_t)(npieces - 1) * j + cut_s - 1);
                    m[0] = (uint32_t)x;
                    m[1] = (uint32_t)(x >> 32);
                    m[2] = sp.cb >> 2;
                    --cut_s;
                    cut_k = (cut_s >= 1 && ls.nj > 0) ? cut_step(cut_s) : ~0u;
                };
                const uint32_t ring_lds = kPcRing + 4 * lane;   // LDS address of ring slot 0
                const uint32_t el = lane & (kPcLanes - 1);       // this lane's entry column
                // A round is steps k0 .. k0+7 from its entries; `esc` holds
                // the round's step bits.  The round's puts, words to `sink`:
                // a round with no marked step, then one with some.
                auto puts_plain = [&](auto &sink, const u32x4 (&E)[kRound]) {
#pragma unroll
                    for (int u = 0; u < kRound; ++u) {
                        const uint32_t f = E[u][2];
                        const bool need = (uint32_t)(x >> 32) >= (f << (31 - kPrecision));
                        sink.put(need, (uint32_t)x);
                        x = need ? (x >> 32) : x;
                        x = reg_step(x, E[u][3], f, entry_rcp(E[u]));
                    }
                };
                // `sa`: the LDS address of the round's escaped values for
                // this lane (step u at sa + u * 4 * kPcLanes).
                auto puts = [&](auto &sink, const u32x4 (&E)[kRound], uint32_t esc, uint32_t sa) {
                    if (esc == 0u) {
                        puts_plain(sink, E);
                    } else {
                        // at a flagged step the lanes concerned put an escape's
                        // groups and count before the escape slot's REG put
                        // (in the entry); the lanes whose entry holds the
                        // symbol and index instead (a bad index, a row whose
                        // values might leave int32, a value out of range) take
                        // the whole symbol here, a bad index the identity step
#pragma unroll
                        for (int u = 0; u < kRound; ++u) {
                            uint32_t st = E[u][3], fu = E[u][2];
                            double ru = entry_rcp(E[u]);
                            if ((esc >> u) & 1u) {
                                if (fu != 0u) {
                                    const uint32_t e = lds_load<uint32_t>(sa + 4 * kPcLanes * u);
                                    if (e != 0u)
                                        put_escape_groups(e - 1u, x, [&](bool spill, uint32_t w) {
                                            sink.put(spill, w);
                                        });
                                } else {
                                    const int32_t sym = (int32_t)E[u][0];
                                    const uint32_t idx = E[u][1];
                                    st = 0u;
                                    fu = kTotal;
                                    ru = 1.0 / kTotal;
                                    if (idx < K) {
                                        uint32_t pr;
                                        const int ec = pc_prefix(sym, tb.meta(idx), x, sink, pr);
                                        lerr = lerr ? lerr : ec;
                                        st = pr & 0xFFFFu;
                                        fu = pr >> 16;
                                        ru = reciprocal(fu);
                                    } else {
                                        lerr = lerr ? lerr : RANS_E_INDEX;
                                    }
                                }
                            }
                            const bool need = (uint32_t)(x >> 32) >= (fu << (31 - kPrecision));
                            sink.put(need, (uint32_t)x);
                            x = need ? (x >> 32) : x;
                            x = reg_step(x, st, fu, ru);
                        }
                    }
                };
                // A round of a chunk where some lane could reach the end of
                // its segment or holds a cut (the other chunks' puts store
                // each word to the scratch segment at once): the words wait
                // in the LDS ring (from slot 0; the slot address advances a
                // slot per word), a lane near the end of its segment or at a
                // split cut redoes the round from its start with checked
                // puts, and the round's words are stored after.
                auto round_checked = [&](const u32x4 (&E)[kRound], uint32_t esc, uint32_t k0) {
                    const uint32_t sa = pc_esc(k0 / kPcChunk, k0 % kPcChunk, el);
                    const uint64_t x0 = x;
                    const uint32_t cb_start = sp.cb;
                    RingSink sink{ring_lds};
                    puts(sink, E, esc, sa);
                    sp.cb += (sink.a - ring_lds) / kWave;
                    {
                        // room for three words per position: the puts above
                        // need no check
                        const bool room = cb_start + 4 * (2 + 3 * kRound) < sp.capb;
                        if (__builtin_expect(!__all(room & (cut_k >= k0 + kRound)), 0)) {
                            x = x0;
                            sp.cb = cb_start;
#pragma unroll
                            for (int u = 0; u < kRound; ++u) {
                                const uint32_t f = E[u][2];
                                const bool off = f == 0u;
                                uint32_t e = 0u;   // an escaped value + 1
                                if ((esc >> u) & 1u)
                                    e = off ? 0u : lds_load<uint32_t>(sa + 4 * kPcLanes * u);
                                const bool fast = !off & room & (e == 0u);
                                const bool need = (uint32_t)(x >> 32) >= (f << (31 - kPrecision));
                                const uint64_t xn =
                                    reg_step(need ? (x >> 32) : x, E[u][3], f, entry_rcp(E[u]));
                                *sp.slot(min((sp.cb - sp.cb0) >> 2, kEncRing - 1)) = (uint32_t)x;
                                sp.cb += (fast & need) ? 4u : 0u;
                                x = fast ? xn : x;
                                if (__builtin_expect(__ballot(!fast) != 0, 0)) {
                                    if (!fast) {
                                        if (off) {
                                            int ec = RANS_E_INDEX;
                                            if (E[u][1] < K)
                                                ec = encode_slow<kWave>((int32_t)E[u][0],
                                                                        tb.meta(E[u][1]), tb, x, sp);
                                            lerr = lerr ? lerr : ec;
                                        } else {
                                            // an escaped value's groups and count,
                                            // then the REG put of the slot (or of
                                            // the identity), spills checked
                                            if (e != 0u)
                                                put_escape_groups(e - 1u, x,
                                                                  [&](bool spill, uint32_t w) {
                                                                      sp.put_if(spill, w);
                                                                  });
                                            const bool spill =
                                                x >= ((uint64_t)f << (63 - kPrecision));
                                            sp.put_if(spill, (uint32_t)x);
                                            x = spill ? (x >> 32) : x;
                                            x = reg_step(x, E[u][3], f, entry_rcp(E[u]));
                                        }
                                    }
                                }
                                while (cut_k == k0 + u)   // (cuts may share a position)
                                    record_cut();
                            }
                        }
                    }
                    __builtin_amdgcn_sched_barrier(0);
                    sp.store_round();
                    __builtin_amdgcn_sched_barrier(0);
                };
                // Entries of round g, read for every wavefront lane (lanes
                // past the wave's read another lane's, unused).
                // (round r of chunk c)
                auto load_round = [&](u32x4 (&E)[kRound], uint32_t c, uint32_t r) {
                    const uint32_t buf = c & 1u;
                    const uint32_t s0 = r * kRound;
#pragma unroll
                    for (int u = 0; u < kRound; ++u)
                        E[u] = lds_load<u32x4>(pc_entry(buf, s0 + u, el));
                };
                // step bits of chunk c (scalar), cleared for the producers'
                // next use of the buffer
                auto take_bits = [&](uint32_t c) -> uint64_t {
                    const uint32_t buf = c & 1u;
                    const uint32_t lo = __builtin_amdgcn_readfirstlane(step_bits[2 * buf]);
                    const uint32_t hi = __builtin_amdgcn_readfirstlane(step_bits[2 * buf + 1]);
                    if (lane == 0) {
                        step_bits[2 * buf] = 0u;
                        step_bits[2 * buf + 1] = 0u;
                    }
                    return (uint64_t)lo | ((uint64_t)hi << 32);
                };
                // A chunk's six rounds run unrolled, so that the round's
                // place in the chunk, its step bits and the handover are
                // fixed at compile time.  At the chunk's start the wave asks
                // whether any lane could reach the end of its segment (three
                // words a position) or holds a cut within the chunk.  Every
                // round requests the next one's entries (past the last:
                // unused reads); before the last round of a chunk the barrier
                // that hands over the next chunk comes first (that round's
                // entries are already in registers).  The last chunk runs
                // whole: its rounds past the longest lane hold identity
                // entries.
                u32x4 E0[kRound], E1[kRound];
                uint64_t bits = 0, bits_next = 0;
                auto step = [&](auto rc, const u32x4 (&E)[kRound], u32x4 (&En)[kRound],
                                uint32_t c, auto &&run_round) {
                    constexpr uint32_t r = decltype(rc)::value;
                    if constexpr (r + 1 == kPcChunkRounds) {
                        if (c + 1 < nch) {
                            __syncthreads();
                            bits_next = take_bits(c + 1);
                        }
                        load_round(En, c + 1, 0);
                    } else {
                        load_round(En, c, r + 1);
                    }
                    if (active)
                        run_round(E, (uint32_t)(bits >> (kRound * r)) & 0xFFu,
                                  (c * kPcChunkRounds + r) * kRound);
                };
                // the six rounds of chunk c, each run by run_round
                auto chunk = [&](uint32_t c, auto &&run_round) {
                    step(std::integral_constant<uint32_t, 0>{}, E0, E1, c, run_round);
                    step(std::integral_constant<uint32_t, 1>{}, E1, E0, c, run_round);
                    step(std::integral_constant<uint32_t, 2>{}, E0, E1, c, run_round);
                    step(std::integral_constant<uint32_t, 3>{}, E1, E0, c, run_round);
                    step(std::integral_constant<uint32_t, 4>{}, E0, E1, c, run_round);
                    step(std::integral_constant<uint32_t, 5>{}, E1, E0, c, run_round);
                };
                if (nch > 0) {
                    __syncthreads();   // chunk 0 is ready
                    bits = take_bits(0);
                    load_round(E0, 0, 0);
                }
                static_assert(kPcChunkRounds == 6, "the unrolled chunk below");
                for (uint32_t c = 0; c < nch; ++c) {
                    const bool ok = sp.cb + 4 * (2 + 3 * kPcChunk) < sp.capb &&
                                    cut_k >= (c + 1) * kPcChunk;
                    if (__all(ok | !active)) {
                        // every put of the chunk stores its word at once, and
                        // the segment's count is brought up to date after it
                        ScratchSink sink{sp.scr, sp.top - 4 - sp.cb};
                        chunk(c, [&](const u32x4 (&E)[kRound], uint32_t esc, uint32_t k0) {
                            if (esc == 0u)   // (one scalar test for the common round)
                                puts_plain(sink, E);
                            else
                                puts(sink, E, esc, pc_esc(c, k0 % kPcChunk, el));
                        });
                        sp.cb = sp.top - 4 - sink.o;
                        sp.cb0 = sp.cb;
                    } else {
                        chunk(c, round_checked);
                    }
                    bits = bits_next;
                }
                __syncthreads();   // the producers' last barrier
                if (active) {
                    while (cut_s >= 1)   // an empty lane: every cut holds the start state
                        record_cut();
                    if (sp.overflow) {
                        lerr = lerr ? lerr : RANS_E_CAPACITY;
                        sp.cb = sp.capb - 8;
                    }
                    buf_store(sp.scr, sp.top - 8 - sp.cb, 0, (int32_t)(uint32_t)x);
                    buf_store(sp.scr, sp.top - 4 - sp.cb, 0, (int32_t)(uint32_t)(x >> 32));
                    words = sp.cb / 4 + 2;
                }
            }
            publish_and_copy(a, hdr, flags, t, nwork, lane, j, active, sp, words, lerr);
        } else if (in_lds) {
            if (nch > 0) {
                if (mine)
                    pc_fill(pls, in0, K, 0, pq, pl, step_bits);
                __syncthreads();
                for (uint32_t c = 1; c < nch; ++c) {
                    if (mine)
                        pc_fill(pls, pc_load(pls, pwb.rsym, pwb.ridx, c, pq), K, c, pq, pl,
                                step_bits);
                    __syncthreads();
                }
            }
            __syncthreads();   // the coding wave's last barrier
        }
    }
    encode_block_end<kPcThreads>(a, hdr, flags, herr, nwork, misc);
}

template <int TPB, int CW, bool PAIR>
hipError_t launch_encode_t(const EncodeArgs &a, hipStream_t s)
{
    const uint32_t lds_bytes = encode_lds_bytes(TPB);
    static const hipError_t attr = hipFuncSetAttribute(
        reinterpret_cast<const void *>(&encode_kernel<TPB, CW, PAIR>),
        hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds_bytes);
    if (attr != hipSuccess)
        return attr;
    const uint32_t blocks = (enc_waves(a.lanes) + CW - 1) / CW;
    hipLaunchKernelGGL((encode_kernel<TPB, CW, PAIR>), dim3(blocks), dim3(TPB), lds_bytes, s, a);
    return hipGetLastError();
}

hipError_t launch_encode_pc(const EncodeArgs &a, hipStream_t s)
{
    static const hipError_t attr =
        hipFuncSetAttribute(reinterpret_cast<const void *>(&encode_pc_kernel),
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)kPcLdsBytes);
    if (attr != hipSuccess)
        return attr;
    hipLaunchKernelGGL(encode_pc_kernel, dim3(enc_waves(a.lanes)), dim3(kPcThreads), kPcLdsBytes,
                       s, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_encode(const EncodeArgs &a, hipStream_t s)
{
    // waves of 32 or more lanes load two rounds at a time (see encode_lane)
    const uint32_t waves = enc_waves(a.lanes);
    const bool pair = enc_lanes_per_wave(a.lanes) >= 32;
    if (coding_one_per_cu(waves))
        return launch_encode_pc(a, s);
    if (waves <= 4 * kCodingCUs)
        return pair ? launch_encode_t<4 * kWave, 4, true>(a, s)
                    : launch_encode_t<4 * kWave, 4, false>(a, s);
    return pair ? launch_encode_t<8 * kWave, 8, true>(a, s) : launch_encode_t<8 * kWave, 8, false>(a, s);
}

}  // namespace rans
