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
// ordinary symbols, the state chain runs with no branch and no LDS access:
// a symbol spills at most one word, which waits in a register together with
// its scratch position.  Other rounds take each escaped (or erroneous)
// symbol through the general puts, which store their words directly.
//
// Memory schedule.  Global memory is touched only between rounds, in
// straight-line code with a fixed number of accesses: the round's candidate
// words are stored (a symbol that spilled nothing stores to a position that
// a later word overwrites, or to the lane's last scratch word), and the
// symbols and indexes of the round after next are requested.  A loaded
// register is first read a round after its load was issued, so the state
// chain never waits on global memory.
#include "rans_coding.hpp"

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

// Encoder tables in LDS at address 0: [meta | pairs], pair = start | f << 16.
struct EncTables {
    uint32_t K;
};

__device__ inline uint32_t pair_of(const EncTables &, const RowMeta &m, uint32_t slot)
{
    return lds_load<uint32_t>(m.base + 4 * slot);
}

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
};

// The puts of one symbol off the common path (an escaped value, or a lane
// near the end of its segment), applied last to first; the row index is in
// range.  Returns a status code.
template <int TPB>
__device__ __forceinline__ int encode_slow(int32_t s, const RowMeta m, const EncTables &t,
                                           uint64_t &x, Spill<TPB> &sp)
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
    // the REG put of the slot
    const uint32_t pr = pair_of(t, m, esc ? mv : (uint32_t)v);
    const uint32_t f = pr >> 16;
    const bool spill = x >= ((uint64_t)f << (63 - kPrecision));
    sp.put_if(spill, (uint32_t)x);
    x = spill ? (x >> 32) : x;
    x = reg_step(x, pr & 0xFFFFu, f, reciprocal(f));
    return err;
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

template <int TPB, int CW>
__global__ __launch_bounds__(TPB) void encode_kernel(EncodeArgs a)
{
    extern __shared__ __align__(16) uint8_t lds[];
    // block bookkeeping after the table set and the rings: [0] flag OR, [1] last block
    uint32_t *misc = reinterpret_cast<uint32_t *>(lds + kEncTableBudget + kEncRing * 4 * TPB);

    WsHeader *hdr = reinterpret_cast<WsHeader *>(a.ws);
    const uint8_t *tab = a.ws + ws_enc_tables_offset();
    uint64_t *flags = reinterpret_cast<uint64_t *>(a.ws + ws_flags_offset());
    uint32_t *scratch = reinterpret_cast<uint32_t *>(a.ws + ws_scratch_offset(a.lanes));
    const uint32_t tid = threadIdx.x;
    const uint32_t lane = tid & (kWave - 1);
    const uint32_t L = a.lanes;
    const uint32_t lpw = enc_lanes_per_wave(L);
    const uint32_t nwork = enc_waves(L);

    // ---- tables -> LDS -------------------------------------------------------
    const uint32_t wave = __builtin_amdgcn_readfirstlane(tid / kWave);   // coding waves 0 .. CW-1
    int herr = 0;
    if (hdr->magic != kMagic || hdr->num_tables != (uint32_t)a.num_tables)
        herr = RANS_E_ARG;
    else if (!hdr->enc_ok)
        herr = RANS_E_TABLE_SIZE;
    else if (lds_address_of(lds) != 0)   // table offsets are used as LDS addresses
        herr = RANS_E_HIP;
    const uint32_t K = (uint32_t)a.num_tables;
    const uint32_t nbytes = herr ? 0u : hdr->enc_bytes;
    stage_tables<TPB>(lds, tab, nbytes);
    __syncthreads();
    EncTables et;
    et.K = K;
    int bad = 0;
    if (!herr)
        for (uint32_t r = tid; r < K; r += TPB)
            bad |= (lds_meta(r).lut & kRowInvalid) ? 1 : 0;
    if (tid == 0)
        misc[0] = 0u;
    __syncthreads();
    bad = block_or(&misc[0], bad);
    if (!herr && bad)
        herr = RANS_E_TABLE;
    if (herr && blockIdx.x == 0 && tid == 0)
        record_error(hdr, herr);

    // herr is the same in every lane; scalar, it keeps the buffer
    // descriptors and loops below uniform for the compiler
    herr = __builtin_amdgcn_readfirstlane(herr);
    if (!herr && wave < CW) {
        // Wave t codes lanes t*lpw ..; its look-back waits only for waves of
        // lower-numbered blocks.  Workgroups are dispatched in index order, so
        // those have all started and none of them waits on this one (a
        // per-wave ticket counter would guarantee the same without relying
        // on dispatch order, but its one contended atomic cost about 10 us).
        const uint32_t t = blockIdx.x * CW + wave;
        if (t < nwork) {
            // the wave codes lanes j0 .. j0 + lpw - 1, one per wavefront lane
            const uint32_t j0 = t * lpw, j1 = min(j0 + lpw, L);
            const uint32_t j = j0 + lane;
            const bool active = lane < lpw && j < L;
            // the wave's symbols and scratch segments, as buffers
            const uint64_t bw = lane_begin(a.n, L, j0), ew = lane_begin(a.n, L, j1);
            const Rsrc rsym = make_rsrc(a.symbols + bw, (uint32_t)(4 * (ew - bw)));
            const Rsrc ridx = make_rsrc(a.indexes + bw, (uint32_t)(4 * (ew - bw)));
            const uint64_t sw0 = 2 * bw + 4ull * j0, sw1 = 2 * ew + 4ull * j1;
            Spill<TPB> sp;
            sp.scr = make_rsrc(scratch + sw0, (uint32_t)(4 * (sw1 - sw0)));
            sp.ring = reinterpret_cast<uint32_t *>(lds + kEncTableBudget) + tid;
            sp.top = 0;
            uint32_t words = 0;
            int lerr = 0;
            if (active) {
                const uint64_t b = lane_begin(a.n, L, j);
                const uint64_t e = lane_begin(a.n, L, j + 1);
                const uint32_t nj = (uint32_t)(e - b);
                sp.top = (uint32_t)(4 * (2 * e + 4ull * (j + 1) - sw0));
                sp.cb = 0;
                sp.cb0 = 0;
                sp.capb = 4 * (2 * nj + 4);
                sp.overflow = false;
                uint64_t x = kStateLow;
                // Split records: the next cut to record (cuts are met last to
                // first) and the step k = nj - 1 - (c - b) at which position c
                // is coded; a round holding it takes the per-position path,
                // which records the state and the words emitted so far right
                // after that position.
                const uint32_t npieces = 1u << a.pieces_log2;
                int32_t cut_s = (int32_t)npieces - 1;
                auto cut_step = [&](int32_t s) -> uint32_t {
                    return nj - 1 - (uint32_t)(piece_begin(b, e, a.pieces_log2, (uint32_t)s) - b);
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
                // byte offsets of the lane's positions in the wave's buffers;
                // positions are coded last to first, clamped at the lane start
                const int32_t plast = (int32_t)(4 * (int64_t)(e - bw) - 4);
                const int32_t pfirst = (int32_t)(4 * (b - bw));
                int32_t sa[kRound], ia[kRound], sb[kRound], ib[kRound];
                // Symbols and indexes of positions k .. k+7: one 16-byte load per
                // four positions, or, when a window would start before the wave's
                // first symbol, one clamped load per position.
                auto load_next = [&](int32_t (&sym)[kRound], int32_t (&idx)[kRound], uint32_t k) {
                    const int32_t pk = plast - (int32_t)(4 * k);
                    if (__all(pk - 4 * (kRound - 1) >= 0)) {
                        const uint32_t lo = (uint32_t)(pk - 4 * (kRound - 1));
                        const u32x4 s0 = buf_load4(rsym, lo), s1 = buf_load4(rsym, lo + 16);
                        const u32x4 i0 = buf_load4(ridx, lo), i1 = buf_load4(ridx, lo + 16);
#pragma unroll
                        for (int u = 0; u < 4; ++u) {
                            sym[7 - u] = (int32_t)s0[u];
                            sym[3 - u] = (int32_t)s1[u];
                            idx[7 - u] = (int32_t)i0[u];
                            idx[3 - u] = (int32_t)i1[u];
                        }
                    } else {
#pragma unroll
                        for (int u = 0; u < kRound; ++u) {
                            const uint32_t off = (uint32_t)max(pk - 4 * u, pfirst);
                            sym[u] = buf_load(rsym, off, 0);
                            idx[u] = buf_load(ridx, off, 0);
                        }
                    }
                    __builtin_amdgcn_sched_barrier(0);
                };
                // The round's words (ring slots 0 .. n-1) go to positions
                // cb0/4 .. cb0/4 + n - 1, i.e. descending byte offsets from
                // top - 4 - cb0.  Slots 0..7 are always stored, as two 16-byte
                // stores (slots past n hold stale words for positions that later
                // words or the final state overwrite); a round of more than 8
                // words, or a lane near the end of its segment, stores word by
                // word.
                auto store_words = [&]() {
                    const uint32_t n = (sp.cb - sp.cb0) >> 2;
                    uint32_t r[8];
#pragma unroll
                    for (int i = 0; i < 8; ++i)
                        r[i] = *sp.slot(i);
                    const bool whole = sp.cb0 + 32 <= sp.capb;
                    const uint32_t off = whole ? sp.top - sp.cb0 - 32 : kNoStore;
                    buf_store4(sp.scr, off, u32x4{r[7], r[6], r[5], r[4]});
                    buf_store4(sp.scr, off + 16, u32x4{r[3], r[2], r[1], r[0]});
                    if (__builtin_expect(__ballot(!whole | (n > 8)) != 0, 0)) {
                        for (uint32_t i = whole ? 8u : 0u; i < n; ++i)
                            if (sp.cb0 + 4 * i + 8 < sp.capb)
                                buf_store(sp.scr, sp.top - 4 - sp.cb0 - 4 * i, 0, (int32_t)*sp.slot(i));
                    }
                    sp.cb0 = sp.cb;
                };
                // State-independent values of one round (positions k0 .. k0+7,
                // last to first): the slot's (start, f), the reciprocal of f,
                // whether the position holds an ordinary symbol of a valid row,
                // and the round's symbols and indexes for the general puts.
                struct Pre {
                    uint32_t start[kRound], f[kRound];
                    double rcp[kRound];
                    int32_t sym[kRound], idx[kRound];
                    bool fast[kRound];
                    bool all;   // every position of this lane is fast
                };
                auto pre = [&](const int32_t (&sym)[kRound], const int32_t (&idx)[kRound], uint32_t k0,
                               Pre &P) {
                    P.all = true;
#pragma unroll
                    for (int u = 0; u < kRound; ++u) {
                        const RowMeta m = lds_meta(min((uint32_t)idx[u], K - 1));
                        const uint32_t mv = m.mvf & 0xFFFFu;
                        // s - offset wraps mod 2^32 into [0, mv) only on rows whose
                        // fast bound is 0
                        const uint32_t w = (uint32_t)sym[u] - (uint32_t)m.offset;
                        P.fast[u] = (w < (m.mvf >> 16)) & ((uint32_t)idx[u] < K) & (k0 + u < nj);
                        P.all = P.all & P.fast[u];
                        const uint32_t pr = pair_of(et, m, min(w, mv));
                        P.start[u] = pr & 0xFFFFu;
                        P.f[u] = pr >> 16;
                        P.rcp[u] = reciprocal(P.f[u]);
                        P.sym[u] = sym[u];
                        P.idx[u] = idx[u];
                    }
                };
                // One round of positions k0 .. k0+7 on P, with the next round's
                // state-independent work (from sym/idx into Pn) in the same
                // straight-line block, where it fills the chain's latency.  The
                // chain assumes every position fast; a round where that is not so
                // for some lane (an escape, a bad index, a lane end, a lane near
                // the end of its segment) is redone from its start state with
                // the general puts.
                auto round = [&](const Pre &P, uint32_t k0, int32_t (&sym)[kRound],
                                 int32_t (&idx)[kRound], Pre &Pn) {
                    // room for three words per position: the fast steps need no check
                    const bool room = sp.cb + 4 * (2 + 3 * kRound) < sp.capb;
                    const uint64_t x0 = x;
                    const uint32_t cb_start = sp.cb;
                    pre(sym, idx, k0 + kRound, Pn);
#pragma unroll
                    for (int u = 0; u < kRound; ++u) {
                        const bool need = (uint32_t)(x >> 32) >= (P.f[u] << (31 - kPrecision));
                        *sp.slot((sp.cb - sp.cb0) >> 2) = (uint32_t)x;
                        sp.cb += need ? 4u : 0u;
                        x = need ? (x >> 32) : x;
                        x = reg_step(x, P.start[u], P.f[u], P.rcp[u]);
                    }
                    if (__builtin_expect(!__all(P.all & room & (cut_k >= k0 + kRound)), 0)) {
                        x = x0;
                        sp.cb = cb_start;
                        // the fast step is committed where it applies; the other
                        // lanes take the slow puts
#pragma unroll
                        for (int u = 0; u < kRound; ++u) {
                            const bool fast = P.fast[u] & room;
                            const bool need = (uint32_t)(x >> 32) >= (P.f[u] << (31 - kPrecision));
                            const uint64_t xn =
                                reg_step(need ? (x >> 32) : x, P.start[u], P.f[u], P.rcp[u]);
                            *sp.slot(min((sp.cb - sp.cb0) >> 2, kEncRing - 1)) = (uint32_t)x;
                            sp.cb += (fast & need) ? 4u : 0u;
                            x = fast ? xn : x;
                            const bool slow = !fast & (k0 + u < nj);
                            if (__builtin_expect(__ballot(slow) != 0, 0)) {
                                if (slow) {
                                    int ec = RANS_E_INDEX;
                                    if ((uint32_t)P.idx[u] < K)
                                        ec = encode_slow<TPB>(P.sym[u], lds_meta(P.idx[u]), et, x,
                                                              sp);
                                    lerr = lerr ? lerr : ec;
                                }
                            }
                            while (cut_k == k0 + u)   // (cuts may share a position)
                                record_cut();
                        }
                    }
                    __builtin_amdgcn_sched_barrier(0);
                    // ---- memory phase: this round's words, the symbols and
                    // indexes of the round three ahead into the buffer just used
                    store_words();
                    __builtin_amdgcn_sched_barrier(0);
                    load_next(sym, idx, k0 + 3 * kRound);
                };
                // prologue: three phases of the same shape (their stores carry
                // stale ring words to positions that later words overwrite);
                // rounds 0 and 1 are loaded, round 0 prepared, round 2 loaded
                Pre pa, pb;
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
                for (uint32_t k0 = 0; k0 < nj; k0 += 2 * kRound) {
                    round(pa, k0, sb, ib, pb);
                    round(pb, k0 + kRound, sa, ia, pa);
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
            }
            if (lerr)
                record_error(hdr, lerr);

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
            // flushing the L2 that the working waves read from).
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
            // sixty-four per round trip (all loads issued before any store),
            // and stores whole 16-byte groups of its own words, then its last
            // one to three words one by one.  Accesses are masked per lane
            // (a lane without words for a group sends no request).
            const uint64_t wbase = 1ull + L + __builtin_amdgcn_readfirstlane((uint32_t)prefix) +
                                   ((uint64_t)__builtin_amdgcn_readfirstlane((uint32_t)(prefix >> 32)) << 32);
            const uint64_t wroom = a.capacity > wbase ? a.capacity - wbase : 0;
            const Rsrc rout = make_rsrc(a.stream + (wroom ? wbase : 0),
                                        (uint32_t)min(4 * wroom, 1ull << 31));
            if (active) {
                const uint64_t end = prefix + incl;
                a.stream[1 + j] = (uint32_t)end;
                const uint32_t ob = 4 * (incl - words);   // the lane's first word in rout
                const uint32_t src = sp.top - 4 * words;
                const uint32_t kt = words & ~3u;   // first word of the last, partial group
                for (uint32_t k0 = 0; k0 < words; k0 += 64) {
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
    }

    // ---- completion: the last block publishes status and cleans up -------------
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
            const uint64_t total = 1ull + L + hdr->total_words;
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

template <int TPB, int CW>
hipError_t launch_encode_t(const EncodeArgs &a, hipStream_t s)
{
    const uint32_t lds_bytes = encode_lds_bytes(TPB);
    static const hipError_t attr = hipFuncSetAttribute(
        reinterpret_cast<const void *>(&encode_kernel<TPB, CW>),
        hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds_bytes);
    if (attr != hipSuccess)
        return attr;
    const uint32_t blocks = (enc_waves(a.lanes) + CW - 1) / CW;
    hipLaunchKernelGGL((encode_kernel<TPB, CW>), dim3(blocks), dim3(TPB), lds_bytes, s, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_encode(const EncodeArgs &a, hipStream_t s)
{
    const uint32_t waves = enc_waves(a.lanes);
    if (coding_one_per_cu(waves))
        return launch_encode_t<4 * kWave, 1>(a, s);
    if (waves <= 4 * kCodingCUs)
        return launch_encode_t<4 * kWave, 4>(a, s);
    return launch_encode_t<8 * kWave, 8>(a, s);
}

}  // namespace rans
