// rans_internal.hpp -- constants, workspace layout and launch wrappers shared by
// the library's translation units (not part of the public ABI).
//
// Format constants follow the coder the pages name: 64-bit state, 32-bit
// words, 16-bit CDF precision (torch_ans 0.3.0 "Usage" table, rans64 row),
// with the state interval [2^31, 2^63) of 64-bit ryg_rans (kompressor
// README "Credits") and 4-bit bypass groups.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "rans_hip.h"

namespace rans {

constexpr uint32_t kPrecision = 16;
constexpr uint32_t kTotal = 1u << kPrecision;
constexpr uint64_t kStateLow = 1ull << 31;
constexpr uint32_t kBypassBits = 4;
constexpr int kWave = 64;

// LDS: 160 KiB per workgroup on gfx950.  Each coding kernel stages its table
// set and keeps a per-lane word ring after it: the decoder a ring of
// kDecRing renormalisation words (read ahead of use), the encoder a ring of
// kEncRing words spilled during the current round (a round of 8 positions
// spills at most 3 words per position).
constexpr uint32_t kLdsBytes = 160u * 1024u;
constexpr uint32_t kMaxBlockThreads = 512;
constexpr uint32_t kDecRing = 8;
constexpr uint32_t kEncRing = 24;
constexpr uint32_t kDecTableBudget = kLdsBytes - kDecRing * 4 * kMaxBlockThreads - 1024;
constexpr uint32_t kEncTableBudget = kLdsBytes - kEncRing * 4 * kMaxBlockThreads - 1024;
constexpr uint32_t kMaxLutQ = 12;        // at most 4096 buckets per row

constexpr uint32_t kHeaderBytes = 256;
constexpr uint32_t kMagic = 0x52414e53u;   // "RANS": tables prepared

// Workspace header.  The first block is written by the table-prep kernel;
// the bookkeeping block is zero between calls (each call's last finishing
// block clears it).
struct WsHeader {
    uint32_t num_tables;
    uint32_t cdf_stride;
    uint32_t total_len;     // sum of row lengths
    uint32_t lut_q;         // decode lookup: 2^lut_q buckets per row
    uint32_t enc_bytes;     // bytes of the encoder's table set [meta | pairs]
    uint32_t dec_bytes;     // bytes of the decoder's table set [meta | cdf16 | lut]
    uint32_t enc_lds;       // 1: the encoder set fits its LDS budget and is staged there;
                            // 0: the coding kernels read it from the workspace
    uint32_t dec_lds;       // the same for the decoder set
    uint32_t magic;
    uint32_t pad0[7];       // pad0 also serves as a harmless dummy store target
    // bookkeeping (self-cleaning)
    int32_t err;            // first error code of the running call, 0 if none
    uint32_t done;          // finished blocks of the running call
    uint32_t pad2;
    uint32_t pad1;
    uint64_t total_words;   // encode: payload words (all lanes)
};
static_assert(sizeof(WsHeader) <= kHeaderBytes, "header too large");

// Per-row metadata, 16 bytes, at the head of both table sets.
//   base    byte offset in the set of the row's cdfm1 entries (decoder) or
//           (start, f) pairs (encoder)
//   offset  symbol value of slot 0
//   mvf     bits 0..15: escape slot mv = len - 2; bits 16..31: the fast-path
//           bound -- slots below it are ordinary symbols whose value
//           offset + slot fits int32 (mv, or 0 when it might not)
//   lut     decoder: byte offset of the row's first-slot entries in the set;
//           both: bit 31 set when the row is invalid
struct alignas(16) RowMeta {
    uint32_t base;
    int32_t offset;
    uint32_t mvf;
    uint32_t lut;
};
constexpr uint32_t kRowInvalid = 0x80000000u;

// Encoder pair entry (4 bytes) per slot k: start(k) | f(k) << 16 (f <= 65535).

inline __host__ __device__ uint64_t align_up(uint64_t v, uint64_t a) { return (v + a - 1) / a * a; }

// Workspace regions:
//   [header | look-back flags | decoder set | encoder set | scratch]
// The flags have a fixed place and size (one per encoder wave of the largest
// lane count): a call finds the flags it uses zero because the previous call's
// last block cleared them, so no call may keep other words where a later call
// looks for flags.  Each table region holds its set in the packed layout the
// prep kernel writes; it is as large as the LDS budget or as the set of
// num_tables rows of cdf_stride entries can be, whichever is more, so any
// valid table set fits it.  A set within the LDS budget is staged into LDS by
// each coding block; a larger one is read from the workspace (through the
// caches) with a bucket table of 2^kGlobalLutQ entries per row.
constexpr uint32_t kMaxCodingWaves = RANS_MAX_LANES / kWave;
constexpr uint32_t kGlobalLutQ = 9;
inline __host__ __device__ uint64_t ws_flags_offset() { return kHeaderBytes; }
inline __host__ __device__ uint64_t ws_dec_offset()
{
    return align_up(kHeaderBytes + 8ull * kMaxCodingWaves, 256);
}
inline __host__ __device__ uint64_t meta_bytes_of(uint64_t K) { return align_up(16 * K, 16); }
// decoder set: meta, cdfm1 (sum of lengths + 4 spare u16, padded), buckets
inline __host__ __device__ uint64_t dec_set_bytes(uint64_t K, uint64_t total_len, uint32_t q)
{
    return meta_bytes_of(K) + align_up(2 * total_len + 8, 16) + align_up((2 * K) << q, 16);
}
inline __host__ __device__ uint64_t enc_set_bytes(uint64_t K, uint64_t total_len)
{
    return meta_bytes_of(K) + align_up(4 * total_len, 16);
}
inline __host__ __device__ uint64_t max_u64(uint64_t a, uint64_t b) { return a > b ? a : b; }
inline __host__ __device__ uint64_t dec_region_bytes(uint64_t K, uint64_t stride)
{
    return align_up(max_u64(kDecTableBudget, dec_set_bytes(K, K * stride, kGlobalLutQ)), 256);
}
inline __host__ __device__ uint64_t enc_region_bytes(uint64_t K, uint64_t stride)
{
    return align_up(max_u64(kEncTableBudget, enc_set_bytes(K, K * stride)), 256);
}
inline __host__ __device__ uint64_t ws_enc_offset(uint64_t K, uint64_t stride)
{
    return ws_dec_offset() + dec_region_bytes(K, stride);
}
inline __host__ __device__ uint64_t ws_scratch_offset(uint64_t K, uint64_t stride)
{
    return ws_enc_offset(K, stride) + enc_region_bytes(K, stride);
}

// Lanes per wavefront and waves per block.  Each lane is a serial chain of
// steps, so a coding kernel is bound by the latency of one step, not by issue
// width: a wave with few active lanes costs the same per step as a full one.
// What grows with the lanes of a wave is the chance that one of them leaves
// the common path at a step (an escape, a lookup outside the window), which
// the whole wave then waits for.  So lanes are spread thin (1, 2, 4, .. 64 per
// wave) until a wave budget is reached.  Each block stages the table set into
// one CU's LDS.  Measured on MI355X (1080p latent, 4096 lanes): one wave per
// CU and two waves per SIMD (8 per CU) both keep every CU at full speed, while
// four waves per CU (one per SIMD) run up to twice slower on some CUs of each
// shader engine; so blocks hold one wave or eight.
//   decoder: up to 2048 waves;
//   encoder: one wave per CU (256 waves) up to 4096 lanes, up to 1024 waves
//            beyond (its escape rounds then cost more than the CU shape).
constexpr uint32_t kCodingCUs = 256;
constexpr __host__ __device__ uint32_t lanes_per_wave_for(uint32_t lanes, uint32_t max_waves)
{
    uint32_t w = 1;
    while (w < (uint32_t)kWave && (lanes + w - 1) / w > max_waves)
        w *= 2;
    return w;
}
constexpr __host__ __device__ uint32_t dec_lanes_per_wave(uint32_t lanes)
{
    return lanes_per_wave_for(lanes, 2048);
}
constexpr __host__ __device__ uint32_t enc_lanes_per_wave(uint32_t lanes)
{
    return lanes_per_wave_for(lanes, lanes <= 4096 ? kCodingCUs : 1024);
}
constexpr __host__ __device__ uint32_t enc_waves(uint32_t lanes)
{
    const uint32_t w = enc_lanes_per_wave(lanes);
    return (lanes + w - 1) / w;
}
constexpr __host__ __device__ uint32_t dec_waves(uint32_t lanes)
{
    const uint32_t w = dec_lanes_per_wave(lanes);
    return (lanes + w - 1) / w;
}
inline __host__ __device__ uint64_t ws_flag_count(uint32_t lanes) { return enc_waves(lanes); }
// Lane j's encode scratch holds 2 * n_j + 4 words: a symbol spills at most
// 52 bits (16 for its slot, 4 for the group count, 32 for raw groups).
inline __host__ __device__ uint64_t ws_scratch_words(uint64_t n, uint32_t lanes)
{
    return 2 * n + 4ull * lanes;
}

// Lane partition: floor(j * n / L) without 128-bit arithmetic.
inline __host__ __device__ uint64_t lane_begin(uint64_t n, uint32_t lanes, uint32_t j)
{
    uint64_t a = n / lanes, b = n % lanes;
    return (uint64_t)j * a + ((uint64_t)j * b) / lanes;
}

static_assert(enc_waves(RANS_MAX_LANES) <= kMaxCodingWaves, "flag region too small");

// Block shapes: while the coding waves fit one per CU, a block has one coding
// wave and three more that only help stage the tables into LDS and then wait
// at the block's final barrier; beyond, a block has eight coding waves (two
// per SIMD), or four for an encode of at most 1024 waves, so that every CU
// takes a share (with 64 lanes a wave the encoder's per-lane memory requests
// bound it, and each CU's address units add capacity).
inline bool coding_one_per_cu(uint32_t waves) { return waves <= kCodingCUs; }
// Dynamic LDS of a coding block: the table set, a few words of block
// bookkeeping, then the word rings.  The kernels declare no static LDS, so
// the dynamic area starts at LDS address 0 and a table byte offset is its LDS
// address (no base to add on every access; each kernel checks the base once).
// The decoder's ring area is aligned to its own size, so the address of ring
// slot p of a lane is the lane's slot 0 OR'ed with (p mod 8) * 4 * TPB.
constexpr uint32_t kLdsMiscBytes = 16;
__host__ __device__ constexpr uint32_t decode_ring_base(uint32_t tpb)
{
    return (uint32_t)((kDecTableBudget + kLdsMiscBytes + kDecRing * 4 * tpb - 1) /
                      (kDecRing * 4 * tpb) * (kDecRing * 4 * tpb));
}
__host__ __device__ constexpr uint32_t decode_lds_bytes(uint32_t tpb)
{
    return decode_ring_base(tpb) + kDecRing * 4 * tpb;
}
static_assert(decode_lds_bytes(kMaxBlockThreads) <= kLdsBytes, "decoder LDS over budget");

// LDS access by byte address (the dynamic area starts at address 0).
template <typename T>
__device__ inline T lds_load(uint32_t addr)
{
    return *(const __attribute__((address_space(3))) T *)(uintptr_t)addr;
}
template <typename T>
__device__ inline void lds_store(uint32_t addr, T v)
{
    *(__attribute__((address_space(3))) T *)(uintptr_t)addr = v;
}
// Row metadata from LDS as one 16-byte read.
__device__ inline RowMeta lds_meta(uint32_t row)
{
    typedef __attribute__((ext_vector_type(4))) uint32_t v4;
    const v4 w = lds_load<v4>(16 * row);
    RowMeta m;
    m.base = w[0];
    m.offset = (int32_t)w[1];
    m.mvf = w[2];
    m.lut = w[3];
    return m;
}
// LDS address of a kernel's dynamic shared array (expected 0).
__device__ inline uint32_t lds_address_of(uint8_t *dyn)
{
    return (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint8_t *)dyn;
}
// Table access.  The coding kernels address a packed table set by byte offset
// from its start.  LdsTab reads a set staged at LDS address 0; GlobalTab reads
// one that stays in the workspace (sets over the LDS budget), through the
// caches.  u16x4 reads four consecutive u16 entries at any even offset: one
// 8-byte LDS read, or four 2-byte loads from global memory (no alignment
// beyond 2 bytes is assumed there).
struct LdsTab {
    template <typename T>
    __device__ inline T load(uint32_t addr) const { return lds_load<T>(addr); }
    __device__ inline RowMeta meta(uint32_t row) const { return lds_meta(row); }
    __device__ inline uint64_t u16x4(uint32_t addr) const { return lds_load<uint64_t>(addr); }
};
struct GlobalTab {
    const uint8_t *g;
    template <typename T>
    __device__ inline T load(uint32_t addr) const { return *reinterpret_cast<const T *>(g + addr); }
    __device__ inline RowMeta meta(uint32_t row) const
    {
        const uint4 w = *reinterpret_cast<const uint4 *>(g + 16ull * row);
        RowMeta m;
        m.base = w.x;
        m.offset = (int32_t)w.y;
        m.mvf = w.z;
        m.lut = w.w;
        return m;
    }
    __device__ inline uint64_t u16x4(uint32_t addr) const
    {
        const uint16_t *p = reinterpret_cast<const uint16_t *>(g + addr);
        return (uint64_t)p[0] | ((uint64_t)p[1] << 16) | ((uint64_t)p[2] << 32) | ((uint64_t)p[3] << 48);
    }
};

__host__ __device__ constexpr uint32_t encode_lds_bytes(uint32_t tpb)
{
    return kEncTableBudget + kEncRing * 4 * tpb + kLdsMiscBytes;
}

// Block-wide OR of one flag through an LDS word (`word` is zero on entry and
// is left zero for the next use).
__device__ inline bool block_or(uint32_t *word, bool v)
{
    if (v)
        *word = 1u;
    __syncthreads();
    const bool r = *word != 0u;
    __syncthreads();
    if (threadIdx.x == 0)
        *word = 0u;
    return r;
}

// Copy `nbytes` (a multiple of 16) of prepared tables from global memory into
// LDS.  gfx950 loads 16 bytes per lane straight into LDS (global_load_lds,
// the LDS address being a per-wave base plus 16 bytes per lane), so every
// wave issues all of its loads back to back and waits once.
template <int TPB>
__device__ inline void stage_tables(uint8_t *lds, const uint8_t *src, uint32_t nbytes)
{
    const uint32_t n16 = nbytes / 16;
    const uint32_t lane = threadIdx.x & (kWave - 1);
    for (uint32_t i0 = threadIdx.x - lane; i0 < n16; i0 += TPB) {
        const uint32_t base = __builtin_amdgcn_readfirstlane(i0);   // the wave's first chunk
        if (i0 + lane < n16)
            __builtin_amdgcn_global_load_lds(reinterpret_cast<const uint4 *>(src) + i0 + lane,
                                             (__attribute__((address_space(3))) void *)(lds + 16 * base),
                                             16, 0, 0);
    }
    __builtin_amdgcn_s_waitcnt(0);
}

// The kernel's argument struct read afresh from the kernel-argument segment
// (explicit arguments start at its offset 0; every kernel here takes one).
// The segment pointer passes through an empty asm first, so the compiler
// cannot hoist the reads: a loop that calls this per iteration re-reads the
// arguments instead of keeping them all live across its body.  Only a
// kernel's own body may call this: a called function has no kernel-argument
// pointer (it reads as null there).
template <class T>
__device__ inline T fresh_kernel_args()
{
    static_assert(sizeof(T) % 4 == 0, "argument struct of whole dwords");
    typedef const __attribute__((address_space(4))) uint32_t KWord;
    KWord *p = (KWord *)__builtin_amdgcn_kernarg_segment_ptr();
    asm volatile("" : "+s"(p));
    uint32_t w[sizeof(T) / 4];
#pragma unroll
    for (uint32_t i = 0; i < sizeof(T) / 4; ++i)
        w[i] = p[i];   // scalar loads: the values stay wave-uniform
    T v;
    __builtin_memcpy(&v, w, sizeof(T));
    return v;
}

// A wave-uniform struct that arrived in vector registers (arguments of a
// called function do) made scalar again, dword by dword, so that buffer
// descriptors built from it need no per-lane loop.
template <class T>
__device__ inline T uniform_copy(const T &in)
{
    static_assert(sizeof(T) % 4 == 0, "struct of whole dwords");
    uint32_t w[sizeof(T) / 4];
    __builtin_memcpy(w, &in, sizeof(T));
#pragma unroll
    for (uint32_t i = 0; i < sizeof(T) / 4; ++i)
        w[i] = __builtin_amdgcn_readfirstlane(w[i]);
    T v;
    __builtin_memcpy(&v, w, sizeof(T));
    return v;
}

// Raw buffer access (gfx9 buffer descriptor, 32-bit data format): the
// hardware drops stores and returns 0 for loads at byte offsets at or past
// `bytes`, and the constant part of an offset rides in the instruction.
// Every descriptor here belongs to a whole wavefront, so its base and size
// are taken from the first active lane: the descriptor then lives in scalar
// registers, as a buffer instruction needs it, even where the compiler
// cannot prove the values uniform (it would otherwise wrap every access in a
// loop over the distinct descriptors of the lanes).
typedef __amdgpu_buffer_rsrc_t Rsrc;
// A byte count capped at 2^31 for a buffer descriptor, in integer
// arithmetic (a mixed-type min() call resolves to the fp64 overload, and a
// count computed that way left a descriptor in vector registers, so that
// every access through it became a loop over its lanes' values).
__host__ __device__ inline uint32_t rsrc_bytes(uint64_t bytes)
{
    return bytes < (1ull << 31) ? (uint32_t)bytes : (1u << 31);
}
__device__ inline Rsrc make_rsrc(const void *base, uint32_t bytes)
{
    // (readfirstlane returns int: each half goes back to uint32_t before it
    // is widened, or a low half with bit 31 set would fill the high one)
    const uint64_t p = reinterpret_cast<uint64_t>(base);
    const uint64_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)p);
    const uint64_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(p >> 32));
    return __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void *>(lo | (hi << 32)), (short)0,
                                             (int)__builtin_amdgcn_readfirstlane(bytes),
                                             0x00020000);
}
__device__ inline int32_t buf_load(Rsrc r, uint32_t voff, int cofs)
{
    return __builtin_amdgcn_raw_buffer_load_b32(r, (int)voff, cofs, 0);
}
__device__ inline void buf_store(Rsrc r, uint32_t voff, int cofs, int32_t v)
{
    __builtin_amdgcn_raw_buffer_store_b32(v, r, (int)voff, cofs, 0);
}
// 16-byte forms; offsets need only 4-byte alignment, and the bounds check is
// made per 4-byte word (a straddling load reads 0 past the end, a straddling
// store writes only the words before it).
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
__device__ inline u32x4 buf_load4(Rsrc r, uint32_t voff)
{
    return __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, 0, 0);
}
__device__ inline void buf_store4(Rsrc r, uint32_t voff, u32x4 v)
{
    __builtin_amdgcn_raw_buffer_store_b128(v, r, (int)voff, 0, 0);
}

struct PrepArgs {
    const int32_t *cdf;
    const int32_t *lengths;
    const int32_t *offsets;
    int32_t num_tables;
    int32_t stride;
    uint8_t *ws;
};

struct EncodeArgs {
    const int32_t *symbols;
    const int32_t *indexes;
    uint64_t n;
    uint32_t lanes;
    int32_t num_tables;
    int32_t stride;
    uint32_t *stream;
    uint64_t capacity;
    uint64_t *stream_words;
    int32_t *status;
    uint8_t *ws;
    // split records: each lane cut into 2^pieces_log2 pieces, records
    // [L][pieces - 1][3] = (state low, state high, lane words left unread)
    uint32_t pieces_log2;
    uint32_t *split_meta;
};

struct DecodeArgs {
    const uint32_t *stream;
    uint64_t capacity;
    const int32_t *indexes;
    uint64_t n;
    int32_t num_tables;
    int32_t stride;
    int32_t *symbols;
    int32_t *status;
    uint8_t *ws;
    // with pieces_log2 > 0, every lane decodes as 2^pieces_log2 pieces, each
    // from its split record (same layout as the encoder writes); split_words
    // is the size of the record array
    uint32_t pieces_log2;
    const uint32_t *split_meta;
    uint64_t split_words;
};

// Piece s of a lane [b, e) cut into 2^pieces_log2 pieces starts at
// b + floor(s (e - b) / 2^pieces_log2).
inline __host__ __device__ uint64_t piece_begin(uint64_t b, uint64_t e, uint32_t pieces_log2,
                                                uint32_t s)
{
    const uint64_t len = e - b;
    const uint32_t sh = pieces_log2;
    // s < 2^sh: split the product to stay within 64 bits
    return b + (len >> sh) * s + (((len & ((1ull << sh) - 1)) * s) >> sh);
}

hipError_t launch_prep(const PrepArgs &a, hipStream_t s);
hipError_t launch_encode(const EncodeArgs &a, hipStream_t s);
hipError_t launch_decode(const DecodeArgs &a, hipStream_t s);

// Quantised CDF rows: Gaussian rows when scales != nullptr, else pmf rows.
struct TableArgs {
    const double *scales;
    double tail_z;
    const double *pmf;
    const int32_t *pmf_lengths;
    int32_t pmf_stride;
    int32_t num_tables;
    int32_t cdf_stride;
    int32_t *cdf;
    int32_t *lengths;
    int32_t *offsets;
    int32_t *status;
};

hipError_t launch_table_rows(const TableArgs &a, hipStream_t s);

// Interleaved streams (one stream per wavefront, one state per lane).
struct IlArgs {
    const int32_t *symbols;    // encode input
    const int32_t *indexes;
    uint64_t n;
    uint32_t streams;
    int32_t num_tables;
    int32_t stride;
    uint32_t *stream;          // encode output container
    const uint32_t *cstream;   // decode input container
    uint64_t capacity;
    uint64_t *stream_words;
    int32_t *symbols_out;
    int32_t *status;
    uint8_t *ws;
    uint32_t *scratch;         // per stream: 128 state words, then emitted words
    uint32_t *counts;          // [streams] words of each stream
    // the fused front end (encode only; symbols and indexes are then null):
    // the latent, its predicted means and scales, and one scale per table row
    const float *y;
    const float *means;
    const float *scales;
    const float *scale_table;
};

// Stream t's scratch starts at word 2 b_t + 256 t (b_t its first symbol):
// 2 m_t + 256 words, room for the 128 state words and the at most
// 2 m_t + 128 words its 64 states emit (2 n_j + 2 per state, as for a lane).
inline __host__ __device__ uint64_t il_scratch_begin(uint64_t n, uint32_t streams, uint32_t t)
{
    return 2 * lane_begin(n, streams, t) + 4ull * kWave * t;
}
inline __host__ __device__ uint64_t il_scratch_words(uint64_t n, uint32_t streams)
{
    return 2 * n + 4ull * kWave * streams;
}
inline __host__ __device__ uint64_t il_counts_offset(uint64_t n, uint32_t streams, uint64_t K,
                                                     uint64_t stride)
{
    return ws_scratch_offset(K, stride) + align_up(4 * il_scratch_words(n, streams), 256);
}

hipError_t launch_il_encode(const IlArgs &a, hipStream_t s);
hipError_t launch_il_decode(const IlArgs &a, hipStream_t s);

// The latent front end and dequantisation.
struct LatentArgs {
    const float *y;
    const float *means;
    const float *scales;
    uint64_t n;
    const float *table;
    int32_t K;
    int32_t *symbols;
    int32_t *indexes;
};

struct DequantArgs {
    const int32_t *symbols;
    const float *means;
    uint64_t n;
    float *y_hat;
};

hipError_t launch_latent_symbols(const LatentArgs &a, hipStream_t s);
hipError_t launch_dequantize(const DequantArgs &a, hipStream_t s);

}  // namespace rans
