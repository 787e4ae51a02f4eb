// rans_decode.hip -- lane decoder: one rANS64 state per wavefront lane,
// symbols read first to last, the symbol of each step found through the
// LDS bucket lookup (the bucket's first slot, then one 8-byte read of the
// next slot starts) with a short search of the bucket's slots as fallback.
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
// Per-symbol work.  The common step -- cum within three slots of the
// bucket's first slot, an ordinary slot, the renormalisation word already in
// the LDS ring -- is straight-line code whose result is committed at once.
// Lanes outside it (cum further out, escape, drained ring, bad index) redo
// the step from the saved state in one out-of-line branch, entered only when
// some lane of the wave needs it.
//
// Memory schedule.  A lane works in rounds of kRound symbols.  Global memory
// is touched only between rounds, in straight-line code with a fixed number
// of accesses: the finished round's symbols are stored, the indexes of the
// round after next are requested, and kRefill stream words are requested for
// the lane's word ring in LDS.  Every loaded register is first read one
// round after its load was issued, so the state chain inside a round never
// waits on global memory.  Should a lane drain its ring within one round
// (long bypass runs), it reads the word straight from global memory.
#include "rans_internal.hpp"

namespace rans {

namespace {

constexpr int kRound = 8;        // symbols per lane between memory phases
constexpr uint32_t kRefill = 4;  // words requested per lane per memory phase
constexpr uint32_t kNoStore = 0x80000000u;   // a buffer offset past every buffer

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

// Decoder tables in LDS at address 0: [meta | cdfm1 | first].  cdfm1[k] =
// start(k) - 1 mod 2^16 (the terminal 65536 becomes 65535), so cum >= start(k)
// is cum > cdfm1[k] and f(k) = cdfm1[k+1] - cdfm1[k] mod 2^16.
struct DecTables {
    uint32_t q;              // 2^q buckets per row
    uint32_t shift;          // 16 - q: cumulative value -> bucket
    uint32_t K;
};

__device__ inline uint32_t cdfm1_at(const DecTables &, const RowMeta &m, uint32_t k)
{
    return lds_load<uint16_t>(m.base + 2 * k);
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
template <int TPB>
__device__ __forceinline__ int decode_slow(int32_t r, const RowMeta &m, uint32_t bucket,
                                           bool beyond, uint32_t slot, uint32_t f, uint32_t rr,
                                           uint64_t &x, Words<TPB> &wd, const DecTables &t,
                                           int32_t &out)
{
    if ((uint32_t)r >= t.K)
        return RANS_E_INDEX;
    const uint32_t mv = m.mvf & 0xFFFFu;
    const uint32_t cum = (uint32_t)x & (kTotal - 1);
    if (__ballot(beyond) != 0) {
        uint32_t lo = slot;   // value(lo) <= cum
        const uint32_t hi = (bucket + 1 < (1u << t.q))
                                ? lds_load<uint16_t>((m.lut & ~kRowInvalid) + 2 * (bucket + 1))
                                : mv;
        // the slot is the last k in [lo, hi] with value(k) <= cum
        uint32_t c;
        do {
            c = 0;
#pragma unroll
            for (uint32_t k = 1; k <= 8; ++k) {
                const uint32_t v = cdfm1_at(t, m, min(lo + k, hi));
                c += (lo + k <= hi && cum > v) ? 1u : 0u;
            }
            lo += c;
        } while (c == 8 && lo < hi);
        const uint32_t sm1 = cdfm1_at(t, m, lo), em1 = cdfm1_at(t, m, lo + 1);
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

// One decoding step of one lane.  The bucket's first slot fs and the four
// entries cdfm1[fs .. fs+3] (one 8-byte LDS read) resolve any cum that falls
// in slots fs .. fs+2; that result is committed for every lane, and lanes
// outside the common case (past the window, escape or out-of-range value,
// renormalisation word not in the ring, bad index) redo the step on the slow
// path.  A bad row index arrives with a fast bound of 0.
template <int TPB>
__device__ __forceinline__ void decode_step(int32_t r, const RowMeta &m, uint64_t &x, Words<TPB> &wd,
                                            const DecTables &t, int32_t &out, int &lerr)
{
    const uint32_t cum = (uint32_t)x & (kTotal - 1);
    const uint32_t xlo_m1 = (uint32_t)x - 1u;   // cum - 1 mod 2^16 in the low half
    const uint32_t bucket = cum >> t.shift;
    const uint32_t fs = lds_load<uint16_t>(m.lut + 2 * bucket);
    const uint64_t v = lds_load<uint64_t>(m.base + 2 * fs);
    const uint32_t wlo = (uint32_t)v, whi = (uint32_t)(v >> 32);   // cdfm1[fs..fs+1], [fs+2..fs+3]
    const bool c1 = cum > (wlo >> 16);
    const bool c2 = c1 & (cum > (whi & 0xFFFFu));
    const bool beyond = c2 & (cum > (whi >> 16));
    const uint32_t slot = fs + (c1 ? 1u : 0u) + (c2 ? 1u : 0u);
    // the slot's cdfm1 pair (start - 1, next start - 1) as one packed word;
    // f = its high half minus its low half and rr = cum - start, both mod
    // 2^16 (16-bit subtractions on the halves, upper bits cleared)
    const uint32_t pair = c2 ? whi : (c1 ? __builtin_amdgcn_alignbit(whi, wlo, 16) : wlo);
    uint32_t f, rr;
    asm("v_sub_u16_sdwa %0, %1, %1 dst_sel:WORD_0 dst_unused:UNUSED_PAD src0_sel:WORD_1 src1_sel:WORD_0"
        : "=v"(f) : "v"(pair));
    asm("v_sub_u16_sdwa %0, %1, %2 dst_sel:WORD_0 dst_unused:UNUSED_PAD src0_sel:WORD_0 src1_sel:WORD_0"
        : "=v"(rr) : "v"(xlo_m1), "v"(pair));
    // f * (x >> 16) + rr with x >> 16 < 2^48 split at bit 32
    const uint32_t xlo = (uint32_t)x, xhi = (uint32_t)(x >> 32);
    const uint32_t mid = __builtin_amdgcn_alignbit(xhi, xlo, 16);
    const uint64_t lo64 = (uint64_t)f * mid + rr;
    const uint32_t nhi = (uint32_t)(lo64 >> 32) + __umul24(f, xhi >> 16);
    const uint64_t xn = ((uint64_t)nhi << 32) | (uint32_t)lo64;
    const bool need = xn < kStateLow;
    const bool slow = beyond | (slot >= (m.mvf >> 16)) | (need & (wd.pos >= wd.filled));
    const uint64_t x0 = x;
    const uint32_t pos0 = wd.pos;
    x = need ? ((xn << 32) | wd.next) : xn;
    wd.pos = pos0 + (need ? 1u : 0u);
    out = (int32_t)(slot + (uint32_t)m.offset);
    if (__builtin_expect(__ballot(slow) != 0, 0)) {
        if (slow) {
            x = x0;
            wd.pos = pos0;
            const int ec = decode_slow<TPB>(r, m, bucket, beyond, slot, f, rr, x, wd, t, out);
            lerr = lerr ? lerr : ec;
        }
    }
    wd.next = wd.at(wd.pos);
}

template <int TPB, int CW, bool SPLIT>
__global__ __launch_bounds__(TPB) void decode_kernel(DecodeArgs a)
{
    extern __shared__ __align__(16) uint8_t lds[];
    // block bookkeeping after the table set and the rings: [0] flag OR, [1] last block
    uint32_t *misc = reinterpret_cast<uint32_t *>(lds + kDecTableBudget);

    WsHeader *hdr = reinterpret_cast<WsHeader *>(a.ws);
    const uint8_t *tab = a.ws + ws_tables_offset();
    const uint32_t tid = threadIdx.x;
    const uint32_t L = a.lanes;

    int herr = 0;
    if (hdr->magic != kMagic || hdr->num_tables != (uint32_t)a.num_tables)
        herr = RANS_E_ARG;
    else if (!hdr->dec_ok)
        herr = RANS_E_TABLE_SIZE;
    else if (lds_address_of(lds) != 0)   // table offsets are used as LDS addresses
        herr = RANS_E_HIP;
    const uint32_t K = (uint32_t)a.num_tables;
    const uint32_t nbytes = herr ? 0u : hdr->dec_bytes;
    const uint32_t q = hdr->lut_q;
    stage_tables<TPB>(lds, tab, nbytes);
    __syncthreads();
    DecTables t;
    t.q = q;
    t.shift = kPrecision - q;
    t.K = K;
    const uint32_t ring = decode_ring_base(TPB) + 4 * tid;
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

    // Work units: lane j's pieces u = j * 2^pl + s (one piece per lane
    // without split records).  The wave codes units u0 .. u0 + lpw - 1, one
    // per wavefront lane.
    const uint32_t pl = SPLIT ? a.pieces_log2 : 0u;
    const uint32_t LV = L << pl;
    const uint32_t lpw = dec_lanes_per_wave(LV);
    const uint32_t lane = tid & (kWave - 1);
    // coding waves are 0 .. CW-1; wave and herr are the same in every lane,
    // and scalar they keep the buffer descriptors and loops below uniform
    const uint32_t wave = __builtin_amdgcn_readfirstlane(tid / kWave);
    herr = __builtin_amdgcn_readfirstlane(herr);
    const uint32_t u0 = __builtin_amdgcn_readfirstlane((blockIdx.x * CW + wave) * lpw);
    const uint32_t u = u0 + lane;
    const uint32_t j = u >> pl;            // the unit's lane
    const uint32_t ps = u & ((1u << pl) - 1);   // and piece
    // first position of unit v (v = LV gives n)
    auto unit_begin = [&](uint32_t v) -> uint64_t {
        const uint32_t lj = v >> pl;
        const uint64_t lb = lane_begin(a.n, L, lj);
        return lj < L ? piece_begin(lb, lane_begin(a.n, L, lj + 1), pl, v & ((1u << pl) - 1)) : lb;
    };
    // the wave's index and symbol spans, and its stream words, as buffers
    if (!herr && wave < CW && u0 < LV) {
        const uint32_t u1 = min(u0 + lpw, LV);
        const uint64_t bw = unit_begin(u0), ew = unit_begin(u1);
        const Rsrc ridx = make_rsrc(a.indexes + bw, (uint32_t)(4 * (ew - bw)));
        const Rsrc rout = make_rsrc(a.symbols + bw, (uint32_t)(4 * (ew - bw)));
        const uint32_t jw = u0 >> pl;   // the wave's first lane
        // the wave's first word (scalar, so the stream's buffer descriptor is)
        const uint64_t wbase = jw ? (uint32_t)__builtin_amdgcn_readfirstlane(a.stream[jw]) : 0u;
        const uint64_t wavail = a.capacity - 1 - L;
        const uint64_t wbytes = wbase < wavail ? min(4 * (wavail - wbase), 1ull << 31) : 0;
        const Rsrc rstr = make_rsrc(a.stream + 1 + L + (wbase < wavail ? wbase : 0), (uint32_t)wbytes);
        if (lane < lpw && u < LV) {
            int lerr = 0;
            const uint64_t beg_w = j ? a.stream[j] : 0u;
            const uint64_t end_w = a.stream[1 + j];
            // the piece's start and end: word offset in the lane and state
            // (piece 0 starts after the flushed state; the last piece ends
            // at the start state with every word read)
            const uint32_t W = (uint32_t)(end_w - beg_w);
            const uint32_t *rec = a.split_meta + 3ull * ((uint64_t)((1u << pl) - 1) * j + ps);
            uint32_t left0 = W - 2, left1 = 0;
            if (ps)
                left0 = rec[-1];
            if (ps + 1 < (1u << pl))
                left1 = rec[2];
            const bool bad_rec = left0 > W - 2 || left1 > left0;
            if (a.stream[0] != L || end_w < beg_w + 2 || 1ull + L + end_w > a.capacity ||
                beg_w < wbase || bad_rec) {
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
                const uint64_t x_end = ps + 1 < (1u << pl) ? ((uint64_t)rec[0] | ((uint64_t)rec[1] << 32))
                                                           : kStateLow;
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
                uint32_t pend[kRefill];
                uint32_t pend_at = wd.filled;

                const uint64_t b = unit_begin(u);
                const uint64_t e = unit_begin(u + 1);
                const uint32_t nj = (uint32_t)(e - b);
                const uint32_t ob = (uint32_t)(4 * (b - bw));   // the lane's first position
                // Two index buffers used in turn (no register copies between
                // rounds): a buffer is refilled in the memory phase right after
                // its round and read again two rounds later.  Every memory phase
                // issues the same global accesses in the same order (8 stores, 8
                // index loads, kRefill word loads), and the prologue runs two
                // such phases too, so the compiler's wait counts only ever cover
                // requests that are at least a round old.  Loads past the
                // wave's span read 0; stores meant for nothing use kNoStore.
                int32_t ia[kRound], ib[kRound], out[kRound];
#pragma unroll
                for (int u = 0; u < kRound; ++u)
                    out[u] = 0;
                // a full round's symbols: two 16-byte stores; a partial round:
                // one store per position (stores past the lane's end go nowhere)
                auto store_full = [&](uint32_t k0) {
                    buf_store4(rout, ob + 4 * k0,
                               u32x4{(uint32_t)out[0], (uint32_t)out[1], (uint32_t)out[2], (uint32_t)out[3]});
                    buf_store4(rout, ob + 4 * k0 + 16,
                               u32x4{(uint32_t)out[4], (uint32_t)out[5], (uint32_t)out[6], (uint32_t)out[7]});
                };
                auto store_part = [&](uint32_t k0) {
#pragma unroll
                    for (int u = 0; u < kRound; ++u)
                        buf_store(rout, k0 + u < nj ? ob + 4 * (k0 + u) : kNoStore, 0, out[u]);
                };
                // indexes of positions k .. k+7 and kRefill stream words: 16-byte
                // loads (past the wave's span or the stream they read 0)
                static_assert(kRefill == 4, "one 16-byte load of stream words");
                auto load_next = [&](int32_t (&idx)[kRound], uint32_t k) {
                    const u32x4 i0 = buf_load4(ridx, ob + 4 * k), i1 = buf_load4(ridx, ob + 4 * k + 16);
                    const u32x4 w = buf_load4(rstr, lw + 4 * wd.filled);
#pragma unroll
                    for (int u = 0; u < 4; ++u) {
                        idx[u] = (int32_t)i0[u];
                        idx[4 + u] = (int32_t)i1[u];
                        pend[u] = w[u];
                    }
                    pend_at = wd.filled;
                    __builtin_amdgcn_sched_barrier(0);
                };
                auto ring_refill = [&]() {
                    if (pend_at == wd.filled && wd.filled + kRefill <= wd.pos + kDecRing) {
#pragma unroll
                        for (uint32_t k = 0; k < kRefill; ++k)
                            wd.put(wd.filled + k, pend[k]);
                        wd.filled = min(wd.count, wd.filled + kRefill);
                    }
                    if (wd.filled < wd.pos)   // the lane outran its ring via direct reads
                        wd.filled = wd.pos;
                    wd.next = wd.at(wd.pos);
                };
                auto round = [&](int32_t (&idx)[kRound], uint32_t k0) {
                    // row metadata; an index outside [0, K) reads row K-1 with a
                    // fast bound of 0 (its step then reports the index), which
                    // only a round holding such an index has to arrange
                    RowMeta m[kRound];
                    uint32_t imax = (uint32_t)idx[0];
#pragma unroll
                    for (int u = 1; u < kRound; ++u)
                        imax = max(imax, (uint32_t)idx[u]);
                    if (__builtin_expect(__ballot(imax >= K) == 0, 1)) {
#pragma unroll
                        for (int u = 0; u < kRound; ++u)
                            m[u] = lds_meta((uint32_t)idx[u]);
                    } else {
#pragma unroll
                        for (int u = 0; u < kRound; ++u) {
                            m[u] = lds_meta(min((uint32_t)idx[u], K - 1));
                            if ((uint32_t)idx[u] >= K)
                                m[u].mvf = 0;
                        }
                    }
                    if (__all(k0 + kRound <= nj)) {
                        // a full round for every lane of the wave
#pragma unroll
                        for (int u = 0; u < kRound; ++u)
                            decode_step<TPB>(idx[u], m[u], x, wd, t, out[u], lerr);
                        __builtin_amdgcn_sched_barrier(0);
                        ring_refill();
                        store_full(k0);
                    } else {
#pragma unroll
                        for (int u = 0; u < kRound; ++u) {
                            out[u] = 0;
                            if (k0 + u < nj && !lerr)
                                decode_step<TPB>(idx[u], m[u], x, wd, t, out[u], lerr);
                        }
                        __builtin_amdgcn_sched_barrier(0);
                        ring_refill();
                        store_part(k0);
                    }
                    __builtin_amdgcn_sched_barrier(0);
                    load_next(idx, k0 + 2 * kRound);
                };
                // prologue: two phases of the same shape (stores to nothing)
#pragma unroll
                for (int p = 0; p < 2; ++p) {
#pragma unroll
                    for (int u = 0; u < kRound; ++u)
                        buf_store(rout, kNoStore, 0, 0);
                    __builtin_amdgcn_sched_barrier(0);
                    load_next(p ? ib : ia, p * kRound);
                }
                // both rounds always run (symbols past the lane end are skipped inside),
                // so every path back to the loop head passes both memory phases
                for (uint32_t k0 = 0; k0 < nj && !lerr; k0 += 2 * kRound) {
                    round(ia, k0);
                    round(ib, k0 + kRound);
                }
                if (!lerr && (x != x_end || wd.pos != W - left1))
                    lerr = RANS_E_CORRUPT;
            }
            if (lerr)
                record_error(hdr, lerr);
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

template <int TPB, int CW, bool SPLIT>
hipError_t launch_decode_t(const DecodeArgs &a, hipStream_t s)
{
    const uint32_t lds_bytes = decode_lds_bytes(TPB);
    static const hipError_t attr = hipFuncSetAttribute(
        reinterpret_cast<const void *>(&decode_kernel<TPB, CW, SPLIT>),
        hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds_bytes);
    if (attr != hipSuccess)
        return attr;
    const uint32_t blocks = (dec_waves(a.lanes << a.pieces_log2) + CW - 1) / CW;
    hipLaunchKernelGGL((decode_kernel<TPB, CW, SPLIT>), dim3(blocks), dim3(TPB), lds_bytes, s, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_decode(const DecodeArgs &a, hipStream_t s)
{
    // decoding split pieces is its own instantiation (the plain decoder
    // carries none of the piece bookkeeping)
    const bool one = coding_one_per_cu(dec_waves(a.lanes << a.pieces_log2));
    if (a.pieces_log2 > 0)
        return one ? launch_decode_t<4 * kWave, 1, true>(a, s) : launch_decode_t<8 * kWave, 8, true>(a, s);
    return one ? launch_decode_t<4 * kWave, 1, false>(a, s) : launch_decode_t<8 * kWave, 8, false>(a, s);
}

}  // namespace rans
