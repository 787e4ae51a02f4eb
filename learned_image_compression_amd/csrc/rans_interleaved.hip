// rans_interleaved.hip -- interleaved streams: one stream per wavefront, one
// rANS64 state per wavefront lane, one shared word cursor per stream.
//
// The pages' fastest GPU coder maps a stream onto a warp, one state per
// lane, with a single bitstream cursor shared by the warp and a layout the
// CPU coder shares word for word (torch_ans 0.3.0, "Usage" legend,
// Interleaved States).  Here the rans64 format of the lane coder is
// interleaved 64 ways, the wavefront width:
//   - the n symbols form S streams split as lanes are; symbol k of a stream
//     is coded by state k mod 64 (lane k mod 64); a step is 64 consecutive
//     symbols, one per lane;
//   - a decoder takes the steps in order; within a step the put slots in
//     order (slot 0: every symbol's REG put; slot 1: an escape's group
//     count; slots 2..: its groups); within a slot the states in ascending
//     order, each put followed by its renormalisation, which may read the
//     next word at the shared cursor.  The encoder applies the same puts in
//     exactly the reverse order, so its emitted words, reversed, are the
//     decoder's reading order;
//   - a stream is its 64 final states (low word, high word, in state order)
//     followed by its words; the container is [S, end_0 .. end_{S-1}] and
//     the streams, as for lanes.
// The order of emissions within a slot is the order of the lanes, so a wave
// places them with one ballot: a lane's word goes at the shared cursor plus
// the number of emitting lanes before it.  A step's symbols, indexes and
// outputs are 64 consecutive int32 (one 256-byte access per wave), and a
// step's stream words are contiguous, read from a three-register window.
//
// Encoding takes two launches after table preparation: the streams into
// workspace scratch (emission order, with each stream's word count), then one
// kernel that writes the header and copies every stream into the container
// (each of its blocks sums the word counts of the streams before its own, so
// no block waits on another).  Decoding is one launch.  A table set over the
// LDS budget is read from the workspace instead of LDS, by the same code.
#include <type_traits>

#include "rans_coding.hpp"
#include "rans_frontend.hpp"
#include "rans_lookup.hpp"

namespace rans {
namespace {

constexpr uint32_t kIlW = kWave;         // states per stream
constexpr int kIlAhead = 8;              // steps of symbols/indexes loaded ahead

__device__ inline void record_error(WsHeader *hdr, int code)
{
    atomicCAS(&hdr->err, 0, code);
}

// Set bits of `mask` below the calling lane (two mbcnt instructions).
__device__ inline uint32_t lanes_below(uint64_t mask)
{
    return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                     __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

// ---- encode: streams into scratch --------------------------------------------

// The scale table of the fused front end sits in LDS after the coding tables
// and the block's bookkeeping words.
constexpr uint32_t kIlScaleLds = kEncTableBudget + kLdsMiscBytes;

constexpr uint32_t kIlScaleLutLds = kIlScaleLds + 4 * RANS_MAX_TABLES;

__device__ inline const float *il_scale_lds()
{
    extern __shared__ __align__(16) uint8_t lds[];
    return reinterpret_cast<const float *>(lds + kIlScaleLds);
}

__device__ inline const uint16_t *il_scale_lut_lds()
{
    extern __shared__ __align__(16) uint8_t lds[];
    return reinterpret_cast<const uint16_t *>(lds + kIlScaleLutLds);
}

// One step group's inputs as loaded: symbols and indexes, or (FUSED) the
// latent, means and scales from which the front end derives them.
template <bool FUSED>
struct IlIn {
    int32_t s[kIlAhead], r[kIlAhead];
};
template <>
struct IlIn<true> {
    float y[kIlAhead], mu[kIlAhead], sc[kIlAhead];
};

// One stream coded by one wave (t < S), tables in LDS or in the workspace.
template <bool FUSED, class Tab>
__device__ __forceinline__ void il_encode_stream(const IlArgs &a, const Tab &tab, uint32_t K,
                                                 uint32_t t, const ScaleTable &st)
{
    WsHeader *hdr = reinterpret_cast<WsHeader *>(a.ws);
    const uint32_t lane = threadIdx.x & (kWave - 1);
    const uint32_t S = a.streams;
    const uint64_t b = lane_begin(a.n, S, t), e = lane_begin(a.n, S, t + 1);
    const uint32_t m = (uint32_t)(e - b);
    // symbols and indexes, or the latent, means and scales
    const Rsrc rin0 = make_rsrc(FUSED ? (const void *)(a.y + b) : (const void *)(a.symbols + b), 4 * m);
    const Rsrc rin1 = make_rsrc(FUSED ? (const void *)(a.means + b) : (const void *)(a.indexes + b), 4 * m);
    const Rsrc rin2 = make_rsrc(FUSED ? (const void *)(a.scales + b) : nullptr, FUSED ? 4 * m : 0u);
    uint32_t *scr = a.scratch + il_scratch_begin(a.n, S, t);
    const uint32_t cap = 2 * m + 2 * kIlW;   // emitted words the stream's scratch holds
    uint32_t *emit = scr + 2 * kIlW;
    uint64_t x = kStateLow;
    uint32_t E = 0;    // words emitted so far (the same in every lane)
    int lerr = 0;

    // ordered emission: lanes with `need` spill their low word, the highest
    // lane first (the reverse of the decoder's reading order)
    auto spill = [&](bool need) {
        const uint64_t mask = __ballot(need);
        if (need) {
            // (the set bits above this lane's own)
            const uint32_t at = E + (uint32_t)__popcll(mask) - 1u - lanes_below(mask);
            if (at < cap)
                emit[at] = (uint32_t)x;
            x >>= 32;
        }
        E += (uint32_t)__popcll(mask);
    };

    const uint32_t G = (m + kIlW - 1) / kIlW;
    IlIn<FUSED> in_a, in_b;
    // steps g0 - 1 .. g0 - kIlAhead (steps below 0 load nothing)
    auto load = [&](IlIn<FUSED> &in, int64_t g0) {
#pragma unroll
        for (int u = 0; u < kIlAhead; ++u) {
            const int64_t g = g0 - 1 - u;
            const uint32_t off = g >= 0 ? (uint32_t)(4 * (g * kIlW + lane)) : 0x80000000u;
            if constexpr (FUSED) {
                in.y[u] = __int_as_float(buf_load(rin0, off, 0));
                in.mu[u] = __int_as_float(buf_load(rin1, off, 0));
                in.sc[u] = __int_as_float(buf_load(rin2, off, 0));
            } else {
                in.s[u] = buf_load(rin0, off, 0);
                in.r[u] = buf_load(rin1, off, 0);
            }
        }
    };
    // the symbols and indexes of a loaded group (the front end's, fused)
    auto convert = [&](const IlIn<FUSED> &in, int32_t (&s)[kIlAhead], int32_t (&r)[kIlAhead]) {
        if constexpr (FUSED) {
#pragma unroll
            for (int u = 0; u < kIlAhead; ++u)
                s[u] = saturate_round(in.y[u] - in.mu[u]);
            st.index_n(in.sc, r);
        } else {
#pragma unroll
            for (int u = 0; u < kIlAhead; ++u) {
                s[u] = in.s[u];
                r[u] = in.r[u];
            }
        }
    };
    // `full` is std::true_type in groups whose every step lies inside the
    // stream, which then carry no per-position bound checks
    auto step = [&](auto full, int32_t s, int32_t r, int64_t g) {
        const uint32_t k = (uint32_t)g * kIlW + lane;
        const bool valid = decltype(full)::value || (g >= 0 && k < m);
        const RowMeta mr = tab.meta(min((uint32_t)r, K - 1));
        const uint32_t mv = mr.mvf & 0xFFFFu;
        const uint32_t w = (uint32_t)s - (uint32_t)mr.offset;
        const bool fast = (w < (mr.mvf >> 16)) & ((uint32_t)r < K);
        if (__builtin_expect(__all(fast | !valid), 1)) {
            const uint32_t pr = tab.template load<uint32_t>(mr.base + 4 * (valid ? w : 0u));
            const uint32_t f = pr >> 16;
            spill(valid & (x >= ((uint64_t)f << (63 - kPrecision))));
            if (valid)
                x = reg_step(x, pr & 0xFFFFu, f, reciprocal(f));
            return;
        }
        // some lane escapes (or holds a bad index): put slots last to first;
        // slot 0 = REG, slot 1 = the group count nb, slot 1 + j = group j - 1
        uint32_t np = 0, nb = 0, start = 0, f = 1;
        uint64_t raw = 0;
        if (valid) {
            if ((uint32_t)r >= K) {
                lerr = lerr ? lerr : RANS_E_INDEX;
            } else {
                const int64_t v = (int64_t)s - (int64_t)mr.offset;
                const bool esc = v < 0 || v >= (int64_t)mv;
                raw = v < 0 ? (uint64_t)(-2 * v - 1) : esc ? (uint64_t)(2 * (v - (int64_t)mv)) : 0;
                if (esc && raw >= (1ull << 31)) {
                    lerr = lerr ? lerr : RANS_E_SYMBOL_RANGE;
                } else {
                    const uint32_t bits = raw ? 64u - (uint32_t)__clzll(raw) : 0u;
                    nb = esc ? (bits + kBypassBits - 1) / kBypassBits : 0u;
                    np = esc ? 2 + nb : 1;
                    const uint32_t pr = tab.template load<uint32_t>(mr.base + 4 * (esc ? mv : (uint32_t)v));
                    start = pr & 0xFFFFu;
                    f = pr >> 16;
                }
            }
        }
        // the wave's largest slot count (at most 2 + 8 < 16), bit by bit
        // from the top with one ballot each: four compares where a
        // reduction by shuffles chains six cross-lane reads
        uint32_t top = 0;
#pragma unroll
        for (uint32_t bit = 8; bit > 0; bit >>= 1)
            top |= __ballot(np >= (top | bit)) != 0 ? bit : 0u;
        for (uint32_t sl = top; sl-- > 0;) {
            const bool has = sl < np;
            if (sl == 0) {
                spill(has & (x >= ((uint64_t)f << (63 - kPrecision))));
                if (has)
                    x = reg_step(x, start, f, reciprocal(f));
            } else {
                const uint32_t b4 = sl == 1 ? nb : (uint32_t)(raw >> (kBypassBits * (sl - 2))) & 15u;
                spill(has & (x >= (1ull << (63 - kBypassBits))));
                if (has)
                    x = (x << kBypassBits) | b4;
            }
        }
    };

    load(in_a, (int64_t)G);
    load(in_b, (int64_t)G - kIlAhead);
    // steps g0 - 1 .. g0 - 2 kIlAhead
    auto group = [&](auto full, int64_t g0) {
        int32_t sv[kIlAhead], rv[kIlAhead];
        convert(in_a, sv, rv);
#pragma unroll
        for (int u = 0; u < kIlAhead; ++u)
            step(full, sv[u], rv[u], g0 - 1 - u);
        load(in_a, g0 - 2 * kIlAhead);
        convert(in_b, sv, rv);
#pragma unroll
        for (int u = 0; u < kIlAhead; ++u)
            step(full, sv[u], rv[u], g0 - kIlAhead - 1 - u);
        load(in_b, g0 - 3 * kIlAhead);
    };
    // the first group may hold the stream's partial last step; after it, the
    // groups wholly inside the stream (steps >= 0, every one full), then the
    // rest (steps below 0)
    int64_t g0 = G;
    if (g0 > 0) {
        group(std::false_type{}, g0);
        g0 -= 2 * kIlAhead;
    }
    for (; g0 >= 2 * kIlAhead; g0 -= 2 * kIlAhead)
        group(std::true_type{}, g0);
    for (; g0 > 0; g0 -= 2 * kIlAhead)
        group(std::false_type{}, g0);
    if (E > cap)
        lerr = lerr ? lerr : RANS_E_CAPACITY;
    scr[2 * lane] = (uint32_t)x;
    scr[2 * lane + 1] = (uint32_t)(x >> 32);
    if (lerr)
        record_error(hdr, lerr);
    if (lane == 0)
        a.counts[t] = 2 * kIlW + min(E, cap);
}

// A stream coded from tables read in the workspace (a set over the LDS
// budget): out of line, so that the LDS form keeps its registers.  The
// arguments arrive in vector registers and are made scalar again here.
template <bool FUSED>
__device__ __attribute__((noinline)) void il_encode_stream_global(IlArgs a_arg, uint32_t t_arg,
                                                                  uint32_t steps_arg,
                                                                  uint32_t mode_arg)
{
    const IlArgs a = uniform_copy(a_arg);
    const uint32_t t = __builtin_amdgcn_readfirstlane(t_arg);
    const uint32_t mode = __builtin_amdgcn_readfirstlane(mode_arg);   // bit 0 sorted, bit 1 lut
    ScaleTable st;
    st.t = il_scale_lds();
    st.K = a.num_tables;
    st.steps = (int32_t)__builtin_amdgcn_readfirstlane(steps_arg);
    st.sorted = (mode & 1u) != 0;
    st.lut = (mode & 2u) ? il_scale_lut_lds() : nullptr;
    il_encode_stream<FUSED>(a, GlobalTab{a.ws + ws_enc_offset(a.num_tables, a.stride)},
                            (uint32_t)a.num_tables, t, st);
}

// FUSED: the symbols and indexes come from the front end (the latent, means
// and scales, with the scale table staged in LDS after the coding tables).
template <int TPB, bool FUSED>
__global__ __launch_bounds__(TPB) void il_encode_kernel(IlArgs a)
{
    extern __shared__ __align__(16) uint8_t lds[];
    WsHeader *hdr = reinterpret_cast<WsHeader *>(a.ws);
    const uint8_t *tab = a.ws + ws_enc_offset(a.num_tables, a.stride);
    const uint32_t tid = threadIdx.x;
    const uint32_t lane = tid & (kWave - 1);
    const uint32_t S = a.streams;

    int herr = 0;
    if (hdr->magic != kMagic || hdr->num_tables != (uint32_t)a.num_tables ||
        hdr->cdf_stride != (uint32_t)a.stride)
        herr = RANS_E_ARG;
    else if (lds_address_of(lds) != 0)
        herr = RANS_E_HIP;
    const uint32_t K = (uint32_t)a.num_tables;
    // (no __syncthreads_or: its shared word would move the dynamic LDS base)
    uint32_t *misc = reinterpret_cast<uint32_t *>(lds + kEncTableBudget);
    const bool in_lds = hdr->enc_lds != 0;
    stage_tables<TPB>(lds, tab, (!herr && in_lds) ? hdr->enc_bytes : 0u);
    if (tid == 0)
        misc[0] = misc[1] = 0u;   // block OR words (tables, scale order)
    __syncthreads();
    int bad = 0;
    if (!herr) {
        const GlobalTab gt{tab};
        for (uint32_t r = tid; r < K; r += TPB)
            bad |= ((in_lds ? lds_meta(r) : gt.meta(r)).lut & kRowInvalid) ? 1 : 0;
    }
    if (block_or(&misc[0], bad) && !herr)
        herr = RANS_E_TABLE;
    ScaleTable st{};
    if constexpr (FUSED) {
        st = stage_scale_table<TPB>(a.scale_table, a.num_tables,
                                    reinterpret_cast<float *>(lds + kIlScaleLds), &misc[1]);
        build_scale_lut<TPB>(st, reinterpret_cast<uint16_t *>(lds + kIlScaleLutLds));
    }
    const uint32_t t = __builtin_amdgcn_readfirstlane(blockIdx.x * (TPB / kWave) + tid / kWave);
    if (herr) {
        if (blockIdx.x == 0 && tid == 0)
            record_error(hdr, herr);
        // the header kernel sums every stream's word count: leave none
        // stale from an earlier call on this workspace
        if (lane == 0 && t < S)
            a.counts[t] = 0;
        return;
    }
    if (t >= S)
        return;
    if (in_lds)
        il_encode_stream<FUSED>(a, LdsTab{}, K, t, st);
    else
        il_encode_stream_global<FUSED>(a, t, (uint32_t)st.steps,
                                       (st.sorted ? 1u : 0u) | (st.lut ? 2u : 0u));
}

// ---- encode: header and container (one wave per stream) -----------------------
// Block b holds streams t0 = 4b .. 4b+3.  It first sums the word counts of
// every stream before t0 (each block on its own: no block waits on another),
// then each wave adds the counts of its block's earlier streams, writes its
// header entry and copies its stream.  The wave of the last stream also
// publishes the container length and the call's status.  Counts are the
// encoder's (at most the stream's scratch span, or zero after a refusal), so
// every copy reads inside its stream's scratch; writes stop at the capacity.

constexpr int kIlCopyThreads = 4 * kWave;

__global__ __launch_bounds__(kIlCopyThreads) void il_copy_kernel(IlArgs a)
{
    __shared__ uint64_t part[kIlCopyThreads / kWave];
    WsHeader *hdr = reinterpret_cast<WsHeader *>(a.ws);
    const uint32_t tid = threadIdx.x, lane = tid & (kWave - 1), wv = tid / kWave;
    const uint32_t S = a.streams;
    const uint32_t t0 = blockIdx.x * (kIlCopyThreads / kWave);
    // t0 is a multiple of 4 and the counts are 256-byte aligned: 16-byte loads
    uint64_t sum = 0;
    const uint4 *c4 = reinterpret_cast<const uint4 *>(a.counts);
    for (uint32_t q = tid; q < t0 / 4; q += kIlCopyThreads) {
        const uint4 v = c4[q];
        sum += (uint64_t)v.x + v.y + v.z + v.w;
    }
    for (int o = kWave / 2; o > 0; o >>= 1)
        sum += __shfl_xor(sum, o);
    if (lane == 0)
        part[wv] = sum;
    __syncthreads();
    uint64_t beg = 0;
    for (uint32_t w = 0; w < kIlCopyThreads / kWave; ++w)
        beg += part[w];
    const uint32_t t = t0 + wv;
    if (t >= S)
        return;
    for (uint32_t s = t0; s < t; ++s)
        beg += a.counts[s];
    const uint64_t cnt = a.counts[t], end = beg + cnt;
    if (lane == 0) {
        if (1ull + t < a.capacity)
            a.stream[1 + t] = (uint32_t)end;
        if (t == S - 1) {
            const uint64_t words = 1ull + S + end;
            int err = hdr->err;
            if (!err && (words > a.capacity || end > 0xFFFFFFFFull))
                err = RANS_E_CAPACITY;
            a.stream[0] = S;   // the capacity holds at least the header
            *a.stream_words = words;
            *a.status = err;
            hdr->err = 0;
        }
    }
    const uint64_t dst0 = 1ull + S + beg;
    if (dst0 + cnt > a.capacity)   // a too-small output: the status says so
        return;
    const uint32_t *scr = a.scratch + il_scratch_begin(a.n, S, t);
    const uint32_t E = (uint32_t)cnt - 2 * kIlW;
    // the states, then the emitted words in reverse; eight words a lane in
    // flight at a time (one at a time, each read waited for before its
    // write, kept the waves waiting on memory most of the kernel)
    constexpr uint32_t kU = 8;
    for (uint32_t i0 = lane; i0 < cnt; i0 += kU * kWave) {
        uint32_t v[kU];
#pragma unroll
        for (uint32_t u = 0; u < kU; ++u) {
            const uint32_t i = i0 + u * kWave;
            v[u] = i < cnt ? (i < 2 * kIlW ? scr[i] : scr[2 * kIlW + (E - 1 - (i - 2 * kIlW))]) : 0u;
        }
#pragma unroll
        for (uint32_t u = 0; u < kU; ++u) {
            const uint32_t i = i0 + u * kWave;
            if (i < cnt)
                a.stream[dst0 + i] = v[u];
        }
    }
}

// ---- decode -----------------------------------------------------------------------

// The decoder table set in LDS, its lookup windows read as aligned words.
// The window of the lookup (four u16 entries at an even address) is read
// with one 8-byte access by the lane decoder, whose few lanes a wave wait on
// each step's latency; three of every four windows are then misaligned, and
// with 64 lanes a wave reading at once the LDS serves those slower.  Here
// every lane of every wave decodes, so the LDS throughput counts: the window
// comes from the three aligned words holding it, shifted into place.
struct LdsTabIl : LdsTab {
    __device__ inline uint64_t u16x4(uint32_t addr) const
    {
        // the words at a, a + 4 and a + 8 hold bytes [addr, addr + 8)
        const uint32_t a = addr & ~3u, sh = (addr & 2u) * 8u;   // 0 or 16
        const uint32_t d0 = lds_load<uint32_t>(a), d1 = lds_load<uint32_t>(a + 4),
                       d2 = lds_load<uint32_t>(a + 8);
        return (uint64_t)__builtin_amdgcn_alignbit(d1, d0, sh) |
               ((uint64_t)__builtin_amdgcn_alignbit(d2, d1, sh) << 32);
    }
};

// One stream decoded by one wave (t < S), tables in LDS or in the workspace.
template <class Tab>
__device__ __forceinline__ void il_decode_stream(const IlArgs &a, const Tab &tab, uint32_t K,
                                                 uint32_t shift, uint32_t t)
{
    WsHeader *hdr = reinterpret_cast<WsHeader *>(a.ws);
    const uint32_t lane = threadIdx.x & (kWave - 1);
    const uint32_t S = a.streams;
    int lerr = 0;
    const uint64_t b = lane_begin(a.n, S, t), e = lane_begin(a.n, S, t + 1);
    const uint32_t m = (uint32_t)(e - b);
    // wave-uniform (t is), and kept in scalar registers so that the
    // stream's buffer descriptor is too
    // (readfirstlane returns int: back to uint32_t before widening)
    const uint64_t prev = t ? (uint32_t)__builtin_amdgcn_readfirstlane(a.cstream[t]) : 0u;
    const uint64_t endt = (uint32_t)__builtin_amdgcn_readfirstlane(a.cstream[1 + t]);
    if ((uint32_t)__builtin_amdgcn_readfirstlane(a.cstream[0]) != S || endt < prev + 2 * kIlW ||
        1ull + S + endt > a.capacity) {
        lerr = RANS_E_CORRUPT;
    } else {
        const uint32_t W = (uint32_t)(endt - prev);
        const uint32_t *words = a.cstream + 1 + S + prev;
        const Rsrc rw = make_rsrc(words, rsrc_bytes(4ull * W));
        const Rsrc ridx = make_rsrc(a.indexes + b, 4 * m);
        const Rsrc rout = make_rsrc(a.symbols_out + b, 4 * m);
        uint64_t x = (uint64_t)(uint32_t)buf_load(rw, 8 * lane, 0) |
                     ((uint64_t)(uint32_t)buf_load(rw, 8 * lane + 4, 0) << 32);
        // words [cw, cw + 192) in three registers, one word per lane each
        uint32_t cw = 2 * kIlW, cursor = 2 * kIlW;
        uint32_t w0 = buf_load(rw, 4 * (cw + lane), 0);
        uint32_t w1 = buf_load(rw, 4 * (cw + kWave + lane), 0);
        uint32_t w2 = buf_load(rw, 4 * (cw + 2 * kWave + lane), 0);
        // Ordered refill: lanes with `need` read the next words, lowest lane
        // first.  The 64 words from the cursor on are one register's worth:
        // lane i holds word cw + i of w0 where i >= off = cursor - cw (< 64)
        // and word cw + 64 + i of w1 below, so word cursor + r sits in lane
        // (off + r) mod 64 and one cross-lane read serves every lane (the
        // select depends on the cursor only, not on this step's state).
        // (refill_ranked: the lanes with `need` take words cursor + rank,
        // `total` words in all, at most 64)
        auto refill_ranked = [&](bool need, uint32_t rank, uint32_t total) {
            const uint32_t off = cursor - cw;
            const uint32_t win = lane >= off ? w0 : w1;
            const uint32_t d = off + rank;   // < 128
            // (the permute reads lane (byte address / 4) mod 64: no mask needed)
            const uint32_t v = (uint32_t)__builtin_amdgcn_ds_bpermute((int)(d << 2), (int)win);
            if (need)
                x = (x << 32) | v;
            cursor += total;
            if (cursor - cw >= kWave) {   // slide the window by one register
                w0 = w1;
                w1 = w2;
                cw += kWave;
                w2 = buf_load(rw, 4 * (cw + 2 * kWave + lane), 0);
            }
        };
        auto refill = [&](bool need) {
            const uint64_t mask = __ballot(need);
            refill_ranked(need, lanes_below(mask), (uint32_t)__popcll(mask));
        };
        // The escape count's refill: few lanes escape a step, and a get
        // seldom takes the state below 2^31, so it is mostly skipped on one
        // wave-uniform test.
        auto refill_some = [&](bool need) {
            if (__ballot(need) != 0)
                refill(need);
        };
        const uint32_t G = (m + kIlW - 1) / kIlW;
        int32_t ia[kIlAhead], ib[kIlAhead];
        auto load = [&](int32_t (&r)[kIlAhead], uint32_t g0) {
#pragma unroll
            for (int u = 0; u < kIlAhead; ++u)
                r[u] = buf_load(ridx, 4 * ((g0 + u) * kIlW + lane), 0);
        };
        const DecTables dt{kPrecision - shift, shift, K};
        // `full` is std::true_type in groups whose every step lies inside
        // the stream, which then carry no per-position bound checks;
        // `chk` (wave-uniform) is set in groups holding an index outside
        // [0, K), whose steps then check their index
        auto step = [&](auto full, bool chk, int32_t r, const RowMeta &mr, uint32_t g) {
            const uint32_t k = g * kIlW + lane;
            const bool valid = decltype(full)::value || k < m;
            const uint32_t mv = mr.mvf & 0xFFFFu;
            if (chk) {
                if (valid && (uint32_t)r >= K)
                    lerr = lerr ? lerr : RANS_E_INDEX;
            }
            // the slot holding cum: the bucket's first slot fs, then one
            // 8-byte read of start-1 for slots fs .. fs+3 settles slots
            // fs .. fs+2 (the lane decoder's lookup).  Where the window's
            // last entry is below cum (rare), a walk over the row from the
            // lookup's slot: past the window it moves on from fs + 2; where
            // the window ran past the row's terminal into the next row (a
            // small entry there, the lookup's slot already right) it stays.
            Lookup sl = lookup_step(mr, x, dt, tab);
            if (__builtin_expect(__ballot(sl.beyond) != 0, 0)) {
                if (sl.beyond) {
                    const uint32_t cum = (uint32_t)x & (kTotal - 1);
                    uint32_t slot = sl.slot;
                    uint32_t nxt = tab.template load<uint16_t>(mr.base + 2 * (slot + 1));
                    for (uint32_t i = 0; i <= mv + 1 && cum > nxt; ++i) {
                        ++slot;
                        nxt = tab.template load<uint16_t>(mr.base + 2 * (slot + 1));
                    }
                    const uint32_t sm1 = tab.template load<uint16_t>(mr.base + 2 * slot);
                    sl.slot = slot;
                    sl.xn = (uint64_t)((nxt - sm1) & 0xFFFFu) * (x >> kPrecision) +
                            ((cum - sm1 - 1) & 0xFFFFu);
                }
            }
            const uint32_t slot = sl.slot;
            // a select, not a branch: the step stays one basic block
            x = valid ? sl.xn : x;
            refill(valid & (x < kStateLow));
            // Slots below the row's fast bound are ordinary symbols whose
            // value offset + slot fits int32 (the bound is 0 for a row
            // where it might not): a 32-bit add, no checks.  The escape
            // slot and such rows take the rare path, which records the
            // same errors in the same order as a check of every position.
            int32_t out = (int32_t)(slot + (uint32_t)mr.offset);
            const bool rare = valid & (slot >= (mr.mvf >> 16));
            if (__builtin_expect(__ballot(rare) != 0, 0)) {
                int64_t value = slot;
                const bool esc = valid & (slot == mv);
                if (__ballot(esc) != 0) {
                    uint32_t nb = 0;
                    if (esc) {
                        nb = (uint32_t)x & 15u;
                        x >>= kBypassBits;
                    }
                    refill_some(esc & (x < kStateLow));
                    if (nb > 8u) {
                        lerr = lerr ? lerr : RANS_E_CORRUPT;
                        nb = 0;
                    }
                    // The groups, taken at once.  Here x >= 2^31, so the get
                    // after which the state first falls below 2^31 is js =
                    // (bit length of x - 32) / 4.  A lane with js < nb
                    // refills there, and only there: the word puts 32 bits
                    // under at least 27, and at most 7 groups follow.  Its
                    // first js + 1 groups are the low bits of x, the rest
                    // the low bits of the state after the refill.  The
                    // refills read their words in order of that group, then
                    // of lane, as one get at a time would.
                    const uint32_t js = (64u - (uint32_t)__clzll(x) - 32u) >> 2;
                    const bool rf = js < nb;
                    const uint32_t k1 = rf ? js + 1 : nb;   // groups before the refill
                    uint64_t raw = x & ((1ull << (kBypassBits * k1)) - 1);
                    x >>= kBypassBits * k1;
                    uint32_t rank = 0, total = 0;
                    for (uint32_t g = 0; __ballot(rf & (js >= g)) != 0; ++g) {
                        const uint64_t m = __ballot(rf & (js == g));
                        if (rf & (js == g))
                            rank = total + lanes_below(m);
                        total += (uint32_t)__popcll(m);
                    }
                    if (total != 0) {
                        refill_ranked(rf, rank, total);
                        const uint32_t k2 = rf ? nb - k1 : 0u;
                        raw |= (x & ((1ull << (kBypassBits * k2)) - 1)) << (kBypassBits * k1);
                        x >>= kBypassBits * k2;
                    }
                    if (esc) {
                        if (raw >= (1ull << 31))
                            lerr = lerr ? lerr : RANS_E_CORRUPT;
                        value = (raw & 1) ? -(int64_t)(raw >> 1) - 1 : (int64_t)(raw >> 1) + mv;
                    }
                }
                if (rare) {
                    const int64_t sym = value + mr.offset;
                    if (sym < INT32_MIN || sym > INT32_MAX)
                        lerr = lerr ? lerr : RANS_E_CORRUPT;
                    out = (int32_t)sym;
                }
            }
            buf_store(rout, valid ? 4 * k : 0x80000000u, 0, out);
        };
        load(ia, 0);
        load(ib, kIlAhead);
        // A group's row metadata is read before its steps (it depends on
        // the index only), so a step's chain of dependent LDS reads
        // starts at the bucket table.
        RowMeta mt[kIlAhead];
        auto metas = [&](const int32_t (&r)[kIlAhead]) {
#pragma unroll
            for (int u = 0; u < kIlAhead; ++u)
                mt[u] = tab.meta(min((uint32_t)r[u], K - 1));
        };
        // does some step of these eight hold an index outside [0, K)?
        auto any_bad = [&](const int32_t (&r)[kIlAhead]) {
            uint32_t imax = (uint32_t)r[0];
#pragma unroll
            for (int u = 1; u < kIlAhead; ++u)
                imax = max(imax, (uint32_t)r[u]);
            return __ballot(imax >= K) != 0;
        };
        auto group = [&](auto full, uint32_t g0) {
            metas(ia);
            const bool chka = any_bad(ia);
#pragma unroll
            for (int u = 0; u < kIlAhead; ++u)
                step(full, chka, ia[u], mt[u], g0 + u);
            load(ia, g0 + 2 * kIlAhead);
            metas(ib);
            const bool chkb = any_bad(ib);
#pragma unroll
            for (int u = 0; u < kIlAhead; ++u)
                step(full, chkb, ib[u], mt[u], g0 + kIlAhead + u);
            load(ib, g0 + 3 * kIlAhead);
        };
        // the groups wholly inside the stream, then the rest (at most one
        // group past the stream's end: a stream holds G steps)
        uint32_t g0 = 0;
        for (; (g0 + 2 * kIlAhead) * kIlW <= m; g0 += 2 * kIlAhead)
            group(std::true_type{}, g0);
        for (; g0 < G; g0 += 2 * kIlAhead)
            group(std::false_type{}, g0);
        if (__ballot(x != kStateLow) != 0 || cursor != W)
            lerr = lerr ? lerr : RANS_E_CORRUPT;
    }
    if (lerr)
        record_error(hdr, lerr);
}

// A stream decoded from tables read in the workspace (out of line, as for
// the encoder).
__device__ __attribute__((noinline)) void il_decode_stream_global(IlArgs a_arg, uint32_t t_arg)
{
    const IlArgs a = uniform_copy(a_arg);
    const uint32_t t = __builtin_amdgcn_readfirstlane(t_arg);
    const WsHeader *hdr = reinterpret_cast<const WsHeader *>(a.ws);
    il_decode_stream(a, GlobalTab{a.ws + ws_dec_offset()}, (uint32_t)a.num_tables,
                     kPrecision - hdr->lut_q, t);
}

template <int TPB>
__global__ __launch_bounds__(TPB) void il_decode_kernel(IlArgs a)
{
    extern __shared__ __align__(16) uint8_t lds[];
    WsHeader *hdr = reinterpret_cast<WsHeader *>(a.ws);
    const uint8_t *tab = a.ws + ws_dec_offset();
    const uint32_t tid = threadIdx.x;
    const uint32_t S = a.streams;
    uint32_t *misc = reinterpret_cast<uint32_t *>(lds + kDecTableBudget);

    int herr = 0;
    if (hdr->magic != kMagic || hdr->num_tables != (uint32_t)a.num_tables ||
        hdr->cdf_stride != (uint32_t)a.stride)
        herr = RANS_E_ARG;
    else if (lds_address_of(lds) != 0)
        herr = RANS_E_HIP;
    const uint32_t K = (uint32_t)a.num_tables;
    const uint32_t shift = kPrecision - hdr->lut_q;
    const bool in_lds = hdr->dec_lds != 0;
    stage_tables<TPB>(lds, tab, (!herr && in_lds) ? hdr->dec_bytes : 0u);
    if (tid == 0)
        misc[0] = 0u;
    __syncthreads();
    int bad = 0;
    if (!herr) {
        const GlobalTab gt{tab};
        for (uint32_t r = tid; r < K; r += TPB)
            bad |= ((in_lds ? lds_meta(r) : gt.meta(r)).lut & kRowInvalid) ? 1 : 0;
    }
    if (block_or(&misc[0], bad) && !herr)
        herr = RANS_E_TABLE;
    if (herr && blockIdx.x == 0 && tid == 0)
        record_error(hdr, herr);

    // herr is the same in every thread; scalar, it keeps the decode loop's
    // control flow (and the shared word cursor) uniform for the compiler
    herr = __builtin_amdgcn_readfirstlane(herr);
    const uint32_t t = __builtin_amdgcn_readfirstlane(blockIdx.x * (TPB / kWave) + tid / kWave);
    if (!herr && t < S) {
        if (in_lds)
            il_decode_stream(a, LdsTabIl{}, K, shift, t);
        else
            il_decode_stream_global(a, t);
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

uint32_t il_blocks(uint32_t streams, uint32_t per) { return (streams + per - 1) / per; }

template <typename F>
hipError_t lds_attr(F *kernel, uint32_t bytes)
{
    return hipFuncSetAttribute(reinterpret_cast<const void *>(kernel),
                               hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
}

// Each block stages a table set into one CU's LDS (one block per CU fits),
// so a block's waves are that CU's coding waves.  More waves per SIMD hide
// more of a step's dependent LDS reads: sixteen waves (four per SIMD) once
// there are streams for every CU that way, else eight, else four.
uint32_t il_block_waves(uint32_t streams)
{
    return streams >= 16 * kCodingCUs ? 16u : (streams >= 8 * kCodingCUs ? 8u : 4u);
}

template <int TPB, bool FUSED>
hipError_t launch_il_encode_t(const IlArgs &a, hipStream_t s)
{
    const uint32_t lds_bytes = FUSED ? kIlScaleLutLds + 2u * kScaleLutCells : kIlScaleLds;
    static const hipError_t attr = lds_attr(&il_encode_kernel<TPB, FUSED>, lds_bytes);
    if (attr != hipSuccess)
        return attr;
    hipLaunchKernelGGL((il_encode_kernel<TPB, FUSED>), dim3(il_blocks(a.streams, TPB / kWave)),
                       dim3(TPB), lds_bytes, s, a);
    return hipGetLastError();
}

template <bool FUSED>
hipError_t launch_il_encode_f(const IlArgs &a, hipStream_t s)
{
    return il_block_waves(a.streams) == 16 ? launch_il_encode_t<16 * kWave, FUSED>(a, s)
           : il_block_waves(a.streams) == 8  ? launch_il_encode_t<8 * kWave, FUSED>(a, s)
                                             : launch_il_encode_t<4 * kWave, FUSED>(a, s);
}

template <int TPB>
hipError_t launch_il_decode_t(const IlArgs &a, hipStream_t s)
{
    const uint32_t lds_bytes = kDecTableBudget + kLdsMiscBytes;
    static const hipError_t attr = lds_attr(&il_decode_kernel<TPB>, lds_bytes);
    if (attr != hipSuccess)
        return attr;
    hipLaunchKernelGGL((il_decode_kernel<TPB>), dim3(il_blocks(a.streams, TPB / kWave)), dim3(TPB),
                       lds_bytes, s, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_il_encode(const IlArgs &a, hipStream_t s)
{
    const hipError_t e = a.scale_table ? launch_il_encode_f<true>(a, s) : launch_il_encode_f<false>(a, s);
    if (e != hipSuccess)
        return e;
    hipLaunchKernelGGL(il_copy_kernel, dim3(il_blocks(a.streams, kIlCopyThreads / kWave)),
                       dim3(kIlCopyThreads), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_il_decode(const IlArgs &a, hipStream_t s)
{
    return il_block_waves(a.streams) == 16 ? launch_il_decode_t<16 * kWave>(a, s)
           : il_block_waves(a.streams) == 8  ? launch_il_decode_t<8 * kWave>(a, s)
                                             : launch_il_decode_t<4 * kWave>(a, s);
}

}  // namespace rans
