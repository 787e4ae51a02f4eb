/*
 * rans_oracle.h -- plain, single-threaded CPU reference of indexed rANS64
 * coding (encode_with_indexes / decode_with_indexes over independent lanes).
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load or call this.  It shares no code,
 * header, table or constant generator with the HIP library.
 *
 * Parity status: every function here is pinned by CPU tests (hand-derived
 * worked streams, round trips, the per-lane size bound, exhaustive brute
 * force on tiny inputs, bypass edge values and error cases).  Byte
 * compatibility with CompressAI's own coder cannot be checked here (no
 * CompressAI and no exported vectors), so that claim is "parity unpinned".
 *
 * Format (plainest reading of the pages; each choice is explained in
 * rans_oracle.c):
 *   - 64-bit state, 32-bit little-endian words, 16-bit CDF precision,
 *     state interval [2^31, 2^63) (kompressor README "Why": 64-bit
 *     ryg_rans-style rANS; torch_ans "Usage" table row rans64: state 64,
 *     stream 32, freq 16);
 *   - a value outside its row's coded range [offset, offset+len-2) is sent
 *     as the escape slot len-2 followed by 4-bit raw groups of a zig-zag
 *     value (torch_ans "Low-level API Reference", range limit of rans*_push);
 *   - the n symbols are cut into L contiguous lanes, lane j owning
 *     [floor(j*n/L), floor((j+1)*n/L)), each with its own state and word
 *     stream (kompressor README "Why": no cross-chunk dependency; torch_ans
 *     FAQ "parallel states ... store bitstream lengths");
 *   - container: [L, end_0, ..., end_{L-1}] then the lane streams back to
 *     back; end_j is the cumulative word count after lane j.
 */
#ifndef RANS_ORACLE_H
#define RANS_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
    ORACLE_OK = 0,
    ORACLE_E_ARG = -1,          /* bad sizes or pointers */
    ORACLE_E_TABLE = -2,        /* a CDF row is malformed */
    ORACLE_E_INDEX = -3,        /* an index is outside [0, K) */
    ORACLE_E_SYMBOL_RANGE = -4, /* escape distance needs 2^31 or more */
    ORACLE_E_CAPACITY = -5,     /* output buffer too small */
    ORACLE_E_CORRUPT = -6       /* the stream does not decode cleanly */
};

/* First symbol position of lane j (j may equal L, giving n). */
uint64_t oracle_lane_begin(uint64_t n, uint32_t num_lanes, uint32_t j);

/* 0 when every row r has 3 <= len[r] <= stride, cdf[r][0] = 0,
 * cdf[r][len-1] = 65536 and strictly increasing entries; else ORACLE_E_TABLE. */
int oracle_check_tables(const int32_t *cdf, const int32_t *lengths,
                        int32_t num_tables, int32_t stride);

/* Encode the symbols of positions [begin, end) as one lane stream.
 * Writes at most `cap` words to `out`; *words gets the lane's word count
 * (also when it exceeds cap, in which case ORACLE_E_CAPACITY is returned). */
int oracle_encode_lane(const int32_t *symbols, const int32_t *indexes,
                       uint64_t begin, uint64_t end,
                       const int32_t *cdf, const int32_t *lengths,
                       const int32_t *offsets, int32_t num_tables, int32_t stride,
                       uint32_t *out, uint64_t cap, uint64_t *words);

/* Decode positions [begin, end) from one lane stream of `words` words. */
int oracle_decode_lane(const uint32_t *lane, uint64_t words,
                       const int32_t *indexes, uint64_t begin, uint64_t end,
                       const int32_t *cdf, const int32_t *lengths,
                       const int32_t *offsets, int32_t num_tables, int32_t stride,
                       int32_t *symbols_out);

/* Whole container: header plus num_lanes lane streams.  *out_words gets
 * the total size (also on ORACLE_E_CAPACITY). */
int oracle_encode(const int32_t *symbols, const int32_t *indexes, uint64_t n,
                  const int32_t *cdf, const int32_t *lengths, const int32_t *offsets,
                  int32_t num_tables, int32_t stride, uint32_t num_lanes,
                  uint32_t *out, uint64_t cap, uint64_t *out_words);

int oracle_decode(const uint32_t *stream, uint64_t stream_words,
                  const int32_t *indexes, uint64_t n,
                  const int32_t *cdf, const int32_t *lengths, const int32_t *offsets,
                  int32_t num_tables, int32_t stride, uint32_t num_lanes,
                  int32_t *symbols_out);

/* Split metadata (decode parallelism beyond the lane count): every lane
 * [b, e) is cut into `pieces` consecutive pieces, piece s starting at
 * b + floor(s (e - b) / pieces).  For each lane j and cut s = 1 .. pieces-1,
 * split_meta[3 ((pieces - 1) j + s - 1) + 0, 1, 2] holds the state a decoder
 * has just before the cut position (low word, high word) and the number of
 * the lane's words still unread there.  The container is the same as
 * oracle_encode's.  The decoder codes each piece from its record and checks
 * that it ends exactly at the next record (the last piece: at the flushed
 * start state with every word read).  pieces in [1, 65]. */
int oracle_encode_split(const int32_t *symbols, const int32_t *indexes, uint64_t n,
                        const int32_t *cdf, const int32_t *lengths, const int32_t *offsets,
                        int32_t num_tables, int32_t stride, uint32_t num_lanes,
                        uint32_t pieces, uint32_t *out, uint64_t cap, uint64_t *out_words,
                        uint32_t *split_meta);

int oracle_decode_split(const uint32_t *stream, uint64_t stream_words,
                        const int32_t *indexes, uint64_t n,
                        const int32_t *cdf, const int32_t *lengths, const int32_t *offsets,
                        int32_t num_tables, int32_t stride, uint32_t num_lanes,
                        uint32_t pieces, const uint32_t *split_meta, int32_t *symbols_out);

/* Interleaved streams: num_streams streams split as lanes are; symbol k of a
 * stream is coded by state k mod width; words of a stream are read through
 * one shared cursor in step, put-slot, ascending-state order; a stream is
 * its width final states (low, high) then its words.  width = 1 gives the
 * lane container.  width in [1, 1024]. */
int oracle_encode_interleaved(const int32_t *symbols, const int32_t *indexes, uint64_t n,
                              const int32_t *cdf, const int32_t *lengths,
                              const int32_t *offsets, int32_t num_tables, int32_t stride,
                              uint32_t num_streams, uint32_t width, uint32_t *out, uint64_t cap,
                              uint64_t *out_words);

int oracle_decode_interleaved(const uint32_t *stream, uint64_t stream_words,
                              const int32_t *indexes, uint64_t n,
                              const int32_t *cdf, const int32_t *lengths,
                              const int32_t *offsets, int32_t num_tables, int32_t stride,
                              uint32_t num_streams, uint32_t width, int32_t *symbols_out);

/* Quantise one pmf row of m entries (alphabet, then the escape slot) to a
 * 16-bit CDF of m + 1 entries: cdf[0] = 0, cdf[m] = 65536.  ORACLE_E_TABLE
 * for an entry outside [0, 1] or NaN; ORACLE_E_ARG for m outside [2, 65536]. */
int oracle_quantize_pmf(const double *pmf, int32_t m, int32_t *cdf);

/* One discretised zero-mean Gaussian row of the given scale, half-width
 * ceil(scale * tail_z), written over `stride` entries (padding 65536).
 * ORACLE_E_TABLE when the scale or tail_z is not positive or the row needs
 * more than `stride` entries. */
int oracle_gaussian_row(double scale, double tail_z, int32_t stride, int32_t *cdf_row,
                        int32_t *length, int32_t *offset);

/* One row per scale: cdf [num_tables][stride], lengths and offsets [num_tables]. */
int oracle_gaussian_tables(const double *scales, int32_t num_tables, double tail_z,
                           int32_t stride, int32_t *cdf, int32_t *lengths, int32_t *offsets);

/* Latent front end: symbols[i] = round-half-even(y[i] - means[i]) in single
 * precision, saturated to int32 (NaN -> INT32_MIN); indexes[i] = the first k
 * with scales[i] <= scale_table[k], K - 1 when none. */
int oracle_latent_symbols(const float *y, const float *means, const float *scales, uint64_t n,
                          const float *scale_table, int32_t num_scales, int32_t *symbols,
                          int32_t *indexes);

/* y_hat[i] = (float)symbols[i] + means[i] in single precision. */
int oracle_dequantize(const int32_t *symbols, const float *means, uint64_t n, float *y_hat);

#ifdef __cplusplus
}
#endif

#endif /* RANS_ORACLE_H */
