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

// LDS: 160 KiB per workgroup on gfx950.  Tables get kTableBudget bytes; the
// coding kernels put a per-lane word ring of kRingWords words after them.
constexpr uint32_t kLdsBytes = 160u * 1024u;
constexpr uint32_t kTableBudget = 140u * 1024u;
constexpr uint32_t kRingWords = 8;
constexpr uint32_t kMaxBlockThreads = 512;
static_assert(kTableBudget + kRingWords * 4 * kMaxBlockThreads <= kLdsBytes, "LDS budget");
constexpr uint32_t kMaxLutQ = 10;        // at most 1024 buckets per row

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
    uint32_t enc_bytes;     // bytes of [meta | cdf16] staged by the encoder
    uint32_t dec_bytes;     // bytes of [meta | cdf16 | lut] staged by the decoder
    uint32_t enc_ok;        // 1 when the encoder tables fit the LDS budget
    uint32_t dec_ok;        // 1 when the decoder tables fit the LDS budget
    uint32_t magic;
    uint32_t pad0[7];
    // bookkeeping (self-cleaning)
    int32_t err;            // first error code of the running call, 0 if none
    uint32_t done;          // finished blocks of the running call
    uint32_t ticket;        // next wave ticket (encode)
    uint32_t pad1;
    uint64_t total_words;   // encode: payload words (all lanes)
};
static_assert(sizeof(WsHeader) <= kHeaderBytes, "header too large");

// Per-row metadata, 16 bytes, staged into LDS by every kernel.
struct RowMeta {
    uint32_t cdf_base;      // first entry of the row in the packed cdf16 array
    int32_t offset;         // symbol value of slot 0
    uint32_t mv;            // escape slot = len - 2; bit 31 set when the row is invalid
    uint32_t lut_base;      // first lookup entry of the row
};
constexpr uint32_t kRowInvalid = 0x80000000u;

// Decode lookup entry (8 bytes) for one bucket of 2^(16-q) cumulative values:
// the adjacent slot pair (a, a+1) covering most of the bucket.
//   bits  0..15  start(a)
//   bits 16..31  start(a+1)
//   bits 32..47  start(a+2) - 1
//   bits 48..63  a
// A cumulative value outside [start(a), start(a+2)) falls back to a search.

inline __host__ __device__ uint64_t align_up(uint64_t v, uint64_t a) { return (v + a - 1) / a * a; }

// Workspace regions: [header | tables (kTableBudget) | look-back flags | scratch].
inline __host__ __device__ uint64_t ws_tables_offset() { return kHeaderBytes; }
inline __host__ __device__ uint64_t ws_flags_offset() { return kHeaderBytes + kTableBudget; }
inline __host__ __device__ uint64_t ws_flag_count(uint32_t lanes) { return (lanes + kWave - 1) / kWave; }
inline __host__ __device__ uint64_t ws_scratch_offset(uint32_t lanes)
{
    return align_up(ws_flags_offset() + 8ull * ws_flag_count(lanes), 256);
}
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

// Threads per block for the coding kernels: every block stages the tables
// into LDS once, so blocks are made large; beyond 256 blocks (one per CU)
// more lanes go into each block.
inline uint32_t coding_block_threads(uint32_t lanes)
{
    return lanes > 256u * 256u ? 512u : 256u;
}
inline uint32_t coding_lds_bytes(uint32_t tpb) { return kTableBudget + kRingWords * 4 * tpb; }

// Copy `nbytes` (a multiple of 16) of prepared tables from global memory into
// LDS with every thread keeping eight 16-byte loads in flight.
template <int TPB>
__device__ inline void stage_tables(uint8_t *lds, const uint8_t *src, uint32_t nbytes)
{
    const uint4 *s = reinterpret_cast<const uint4 *>(src);
    uint4 *d = reinterpret_cast<uint4 *>(lds);
    const uint32_t n16 = nbytes / 16;
    if (n16 == 0)
        return;
    for (uint32_t i0 = threadIdx.x; i0 < n16; i0 += 8 * TPB) {
        uint4 v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u)
            v[u] = s[min(i0 + u * TPB, n16 - 1)];
#pragma unroll
        for (int u = 0; u < 8; ++u)
            if (i0 + u * TPB < n16)
                d[i0 + u * TPB] = v[u];
    }
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
    uint32_t *stream;
    uint64_t capacity;
    uint64_t *stream_words;
    int32_t *status;
    uint8_t *ws;
};

struct DecodeArgs {
    const uint32_t *stream;
    uint64_t capacity;
    const int32_t *indexes;
    uint64_t n;
    uint32_t lanes;
    int32_t num_tables;
    int32_t *symbols;
    int32_t *status;
    uint8_t *ws;
};

hipError_t launch_prep(const PrepArgs &a, hipStream_t s);
hipError_t launch_encode(const EncodeArgs &a, hipStream_t s);
hipError_t launch_decode(const DecodeArgs &a, hipStream_t s);

}  // namespace rans
