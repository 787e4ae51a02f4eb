/*
 * rans_hip.h -- C ABI of the gfx950 (MI355X) indexed rANS64 coder.
 *
 * What it computes.  encode_with_indexes / decode_with_indexes of
 * CompressAI-style entropy coding (kompressor README, "Why" and "Credits";
 * torch_ans 0.3.0, "High-level API Reference"): symbol i is coded with the
 * 16-bit quantised CDF row indexes[i] of a table set (cdf, cdf_lengths,
 * offsets), by 64-bit rANS with 32-bit stream words (torch_ans "Usage"
 * table, rans64 row).  A value outside its row's coded range
 * [offset, offset + len - 2) is sent as the row's escape slot len-2 followed
 * by a zig-zag raw value in 4-bit groups (torch_ans "Low-level API
 * Reference", range limit of rans*_push).  The symbols are cut into
 * num_lanes contiguous lanes, each with its own state and word stream, since
 * a mean-scale hyperprior has no spatial autoregression (kompressor README
 * "Why"); lane j owns positions [floor(j n / L), floor((j+1) n / L)).
 *
 * Stream container (u32 little-endian words):
 *   word 0           num_lanes L
 *   words 1 .. L     end_j = cumulative lane word count after lane j
 *   words L+1 ..     lane streams back to back; a lane stream is the final
 *                    state (low word, high word) then its renormalisation
 *                    words in the order the decoder reads them.
 * With L = 1 the words after [1, W] form the standard single rANS64 stream.
 *
 * Table rows.  cdf is int32 [num_tables][cdf_stride]; row r has
 * cdf_lengths[r] valid entries (3 <= len <= cdf_stride), starts at 0, ends
 * at exactly 65536 and strictly increases (every frequency >= 1).
 * offsets[r] is the symbol value of slot 0.
 *
 * Memory and ownership.  Every array argument below is a DEVICE pointer
 * owned by the caller (for example a torch tensor's data_ptr() on the ROCm
 * device).  The library allocates nothing and keeps no global state; all
 * work is enqueued on `hstream` and no call synchronises with the host.
 * `workspace` is caller-owned device memory of at least
 * rans_workspace_bytes(...) bytes, 256-byte aligned, zero-filled before its
 * first use; every call leaves its bookkeeping words zero again, so the
 * same workspace can be reused by later calls.  Calls that share a
 * workspace, an output or a status word must not overlap in time.
 *
 * Table sets.  Any valid set within RANS_MAX_TABLES rows of RANS_MAX_STRIDE
 * entries is coded.  A set whose packed form fits the coding kernels' LDS
 * budget (about 110 KiB for the encoder, 143 KiB for the decoder; the
 * 64-row Gaussian set of the 1080p latent fits) is staged into LDS by every
 * coding block; a larger one is read from the workspace through the caches,
 * which is slower but gives the same bytes.
 *
 * Errors.  The return value reports what the host can check before
 * launching (RANS_E_ARG, RANS_E_WORKSPACE, RANS_E_TABLE for bad sizes,
 * RANS_E_HIP for a failed launch).  Data-dependent errors are written by
 * the device to *status (0 on success; a bad CDF row, an index outside
 * [0, K), a symbol too far out of range, a too-small output, a corrupt
 * stream).  When *status != 0 the outputs are unspecified, but no kernel
 * ever reads or writes outside the buffers described here.
 */
#ifndef RANS_HIP_H
#define RANS_HIP_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

enum rans_status {
    RANS_OK = 0,
    RANS_E_ARG = -1,          /* null pointer, zero lanes, bad sizes */
    RANS_E_TABLE = -2,        /* a CDF row is malformed */
    RANS_E_INDEX = -3,        /* indexes[i] outside [0, num_tables) */
    RANS_E_SYMBOL_RANGE = -4, /* escape distance needs 2^31 or more */
    RANS_E_CAPACITY = -5,     /* encoded container exceeds stream capacity */
    RANS_E_CORRUPT = -6,      /* the stream does not decode cleanly */
    RANS_E_WORKSPACE = -7,    /* workspace missing, misaligned or too small */
    RANS_E_HIP = -8           /* a HIP launch failed */
};

/* Largest supported table count and row stride, and the largest symbol
 * count and lane count of one call (larger inputs are split by the caller
 * into several containers); beyond them a call returns RANS_E_ARG. */
#define RANS_MAX_TABLES 4096
#define RANS_MAX_STRIDE 16384
#define RANS_MAX_PIECES 64
#define RANS_MAX_STREAMS (1u << 16)
#define RANS_MAX_SYMBOLS (1ull << 28)
#define RANS_MAX_LANES (1u << 22)

/* Words an encoded container can need in the worst case (every symbol an
 * escape with a 31-bit raw value): 1 + L header words plus, per lane,
 * 2 * symbols + 4 (a symbol costs at most 16 + 36 bits). */
uint64_t rans_encode_bound_words(uint64_t n, uint32_t num_lanes);

/* Workspace bytes needed by any call below with these sizes: a fixed header
 * and look-back flag region (about 0.5 MiB), two table regions sized for
 * num_tables rows of cdf_stride entries (at least the LDS budgets), and the
 * encoder's scratch of 2 n + 4 num_lanes words.  A decode needs only the
 * part before the scratch. */
uint64_t rans_workspace_bytes(uint64_t n, uint32_t num_lanes, int32_t num_tables,
                              int32_t cdf_stride);

/* Encode n symbols into the container at `stream` (capacity in words).
 * *stream_words (device) receives the container length in words. */
int rans_encode_with_indexes(const int32_t *symbols, const int32_t *indexes, uint64_t n,
                             const int32_t *cdf, const int32_t *cdf_lengths,
                             const int32_t *offsets, int32_t num_tables, int32_t cdf_stride,
                             uint32_t num_lanes, uint32_t *stream,
                             uint64_t stream_capacity_words, uint64_t *stream_words,
                             int32_t *status, void *workspace, uint64_t workspace_bytes,
                             hipStream_t hstream);

/* Decode n symbols (n = number of indexes) from the container at `stream`.
 * The lane count is read from the container's first word (the container
 * carries its own length bookkeeping: torch_ans 0.3.0, "Parallel ANS
 * stream"), so there is no lane argument.  stream_capacity_words (at least
 * 1) is the number of readable words at `stream`; the container may be
 * shorter (its header gives its extent).  A lane count of 0 or above
 * RANS_MAX_LANES, a header longer than the capacity, lane ends outside it or
 * a lane that does not decode cleanly give *status = RANS_E_CORRUPT. */
int rans_decode_with_indexes(const uint32_t *stream, uint64_t stream_capacity_words,
                             const int32_t *indexes, uint64_t n,
                             const int32_t *cdf, const int32_t *cdf_lengths,
                             const int32_t *offsets, int32_t num_tables, int32_t cdf_stride,
                             int32_t *symbols, int32_t *status, void *workspace,
                             uint64_t workspace_bytes, hipStream_t hstream);

/* The two calls above are rans_prepare_tables followed by the matching
 * *_prepared call.  Callers that code many tensors with one table set
 * (torch_ans "Performance Tuning": reuse the coder instead of rebuilding
 * tables per call) may prepare once and code many times on one workspace.
 * rans_prepare_tables validates the rows on the device and packs them, with
 * the decoder's lookup table, into the workspace; row errors surface in the
 * *status of the next *_prepared call.  num_tables and cdf_stride of a
 * *_prepared call must be those of the prepared set, else *status reports
 * RANS_E_ARG. */
int rans_prepare_tables(const int32_t *cdf, const int32_t *cdf_lengths, const int32_t *offsets,
                        int32_t num_tables, int32_t cdf_stride, void *workspace,
                        uint64_t workspace_bytes, hipStream_t hstream);

int rans_encode_prepared(const int32_t *symbols, const int32_t *indexes, uint64_t n,
                         int32_t num_tables, int32_t cdf_stride, uint32_t num_lanes,
                         uint32_t *stream, uint64_t stream_capacity_words,
                         uint64_t *stream_words, int32_t *status, void *workspace,
                         uint64_t workspace_bytes, hipStream_t hstream);

int rans_decode_prepared(const uint32_t *stream, uint64_t stream_capacity_words,
                         const int32_t *indexes, uint64_t n, int32_t num_tables,
                         int32_t cdf_stride, int32_t *symbols, int32_t *status, void *workspace,
                         uint64_t workspace_bytes, hipStream_t hstream);

/* Split records: decode parallelism beyond the lane count (torch_ans 0.3.0,
 * "Related Projects", names Recoil, a rANS library of parallel rANS
 * algorithms; the record format here is a reading of that idea, not
 * Recoil's format).  The container is unchanged; beside
 * it the encoder writes, for every lane j and every cut s = 1 .. pieces-1
 * inside the lane, a record of three u32 at
 *   split_meta[3 * ((pieces - 1) * j + s - 1) + 0, 1, 2]
 * = (low word, high word) of the state a decoder holds just before position
 *   c = b + floor(s * (e - b) / pieces) of the lane [b, e), and the number of
 *   the lane's words still unread there.
 * The decoder then codes each of the num_lanes * pieces pieces on its own,
 * from its record, and checks that it ends exactly at the next record (the
 * last piece: at the flushed start state with every word read); a piece
 * that does not, or a record that cannot be right, gives RANS_E_CORRUPT.
 * pieces is a power of two in [1, RANS_MAX_PIECES]; with pieces = 1 these
 * calls are rans_encode_with_indexes / rans_decode_with_indexes and
 * split_meta may be null.  split_meta holds 3 * num_lanes * (pieces - 1)
 * words (device memory, caller-owned); the decoder takes the lane count from
 * the container and the size of split_meta as split_words, and reports
 * RANS_E_ARG when the records the container needs exceed it.  Other
 * arguments as above. */
int rans_encode_with_splits(const int32_t *symbols, const int32_t *indexes, uint64_t n,
                            const int32_t *cdf, const int32_t *cdf_lengths, const int32_t *offsets,
                            int32_t num_tables, int32_t cdf_stride, uint32_t num_lanes,
                            uint32_t pieces, uint32_t *stream, uint64_t stream_capacity_words,
                            uint64_t *stream_words, uint32_t *split_meta, int32_t *status,
                            void *workspace, uint64_t workspace_bytes, hipStream_t hstream);

int rans_decode_with_splits(const uint32_t *stream, uint64_t stream_capacity_words,
                            const int32_t *indexes, uint64_t n,
                            const int32_t *cdf, const int32_t *cdf_lengths,
                            const int32_t *offsets, int32_t num_tables, int32_t cdf_stride,
                            uint32_t pieces, const uint32_t *split_meta, uint64_t split_words,
                            int32_t *symbols, int32_t *status, void *workspace,
                            uint64_t workspace_bytes, hipStream_t hstream);

/* Interleaved streams: the wavefront-width variant of the pages' warp-level
 * interleaved coder (torch_ans 0.3.0, "Usage" legend, Interleaved States:
 * one stream per warp, one state per lane, one shared bitstream cursor).
 * The n symbols form num_streams streams split as lanes are; symbol k of a
 * stream is coded by state k mod 64.  A decoder takes a stream's steps (64
 * consecutive symbols) in order, within a step the put slots in order (slot
 * 0: every symbol's REG put; slot 1: an escape's group count; slots 2..:
 * its groups), within a slot the states in ascending order; each put is
 * followed by its renormalisation, which reads the next word at the
 * stream's one cursor.  The encoder applies the puts in exactly the reverse
 * order.  A stream is its 64 final states (low word, high word, in state
 * order) followed by its words; the container is [num_streams, end_0 ..
 * end_{num_streams-1}] followed by the streams.  This is a different
 * container from the lane container above.
 *
 * Workspace: rans_interleaved_workspace_bytes(n, num_streams, num_tables,
 * cdf_stride) bytes for an encode, rans_workspace_bytes(...) for a decode,
 * the same contract as above.  rans_interleaved_bound_words bounds the container.  num_streams in
 * [1, RANS_MAX_STREAMS].  Errors as for the lane calls; a stream that does
 * not end with every state at 2^31 and every word read gives
 * RANS_E_CORRUPT. */
uint64_t rans_interleaved_bound_words(uint64_t n, uint32_t num_streams);
uint64_t rans_interleaved_workspace_bytes(uint64_t n, uint32_t num_streams, int32_t num_tables,
                                          int32_t cdf_stride);

int rans_encode_interleaved(const int32_t *symbols, const int32_t *indexes, uint64_t n,
                            const int32_t *cdf, const int32_t *cdf_lengths,
                            const int32_t *offsets, int32_t num_tables, int32_t cdf_stride,
                            uint32_t num_streams, uint32_t *stream,
                            uint64_t stream_capacity_words, uint64_t *stream_words,
                            int32_t *status, void *workspace, uint64_t workspace_bytes,
                            hipStream_t hstream);

int rans_decode_interleaved(const uint32_t *stream, uint64_t stream_capacity_words,
                            const int32_t *indexes, uint64_t n,
                            const int32_t *cdf, const int32_t *cdf_lengths,
                            const int32_t *offsets, int32_t num_tables, int32_t cdf_stride,
                            uint32_t num_streams, int32_t *symbols, int32_t *status,
                            void *workspace, uint64_t workspace_bytes, hipStream_t hstream);

/* The two interleaved calls above are rans_prepare_tables followed by these.
 * A caller that codes many tensors with one table set (torch_ans
 * "Performance Tuning": reuse the coder rather than rebuild its tables) runs
 * rans_prepare_tables once on the workspace and then any number of these
 * calls on that workspace.  The workspace must also meet the size above
 * (rans_interleaved_workspace_bytes for an encode).  num_tables and
 * cdf_stride must equal the prepared set's, or *status reports RANS_E_ARG;
 * row errors found by the preparation surface in *status as RANS_E_TABLE.
 * The host-side checks and the other errors are those of the full calls. */
int rans_encode_interleaved_prepared(const int32_t *symbols, const int32_t *indexes, uint64_t n,
                                     int32_t num_tables, int32_t cdf_stride, uint32_t num_streams,
                                     uint32_t *stream, uint64_t stream_capacity_words,
                                     uint64_t *stream_words, int32_t *status, void *workspace,
                                     uint64_t workspace_bytes, hipStream_t hstream);

int rans_decode_interleaved_prepared(const uint32_t *stream, uint64_t stream_capacity_words,
                                     const int32_t *indexes, uint64_t n, int32_t num_tables,
                                     int32_t cdf_stride, uint32_t num_streams, int32_t *symbols,
                                     int32_t *status, void *workspace, uint64_t workspace_bytes,
                                     hipStream_t hstream);

/* Quantised CDF rows built on the device, one row per table (the step
 * before coding: torch_ans 0.3.0, "Parameter Setup" and "Other Features",
 * the coder turns batched pmfs into 16-bit CDFs itself; "Performance
 * Tuning", item 6, that rebuild costs about 0.2 ms on CUDA).
 *
 * Quantisation of a pmf row of m entries (alphabet, then the escape slot):
 * f_k = max(1, round-half-even(p_k * 65536)), then the sum is brought to
 * 65536 as if one unit at a time were taken from (surplus) or given to
 * (deficit) the currently largest f_k, the lowest slot among equals.  The
 * row's CDF is [0, f_0, f_0 + f_1, ..., 65536] (m + 1 entries), and the
 * entries from m + 1 to cdf_stride - 1 are set to 65536.
 *
 * rans_gaussian_tables: row r is the zero-mean Gaussian of scale scales[r]
 * (double) discretised on integer bins: half-width c = ceil(scale * tail_z),
 * tail_z the standard-normal quantile of 1 - tail_mass / 2 (6.1094 for a
 * tail mass of 1e-9); slot k = 0..2c has mass Phi((k - c + 1/2) / scale) -
 * Phi((k - c - 1/2) / scale), the escape slot the two tails
 * 2 Phi(-(c + 1/2) / scale), all in double precision with
 * Phi(x) = erfc(-x / sqrt 2) / 2.  Outputs cdf [num_tables][cdf_stride],
 * cdf_lengths = 2c + 3 and offsets = -c, ready for the coding calls.
 *
 * rans_quantize_pmfs: row r quantises pmf[r][0 .. pmf_lengths[r]) (double,
 * row pitch pmf_stride entries, no normalisation: a sum other than 1 is
 * absorbed by the adjustment above); cdf_lengths[r] = pmf_lengths[r] + 1.
 *
 * Every pointer is a device pointer; one workgroup per row.  row_status[r]
 * (device, num_tables entries) receives RANS_OK, or RANS_E_TABLE when the
 * row cannot be built (scale not positive or NaN, row longer than
 * cdf_stride, pmf length outside [2, min(pmf_stride, cdf_stride - 1)], a
 * pmf entry outside [0, 1] or NaN); such a row's cdf_lengths[r] is 0 and
 * its cdf entries are unspecified.  The return value reports bad sizes or
 * pointers (RANS_E_ARG; tail_z must be positive and finite) and launch
 * failures (RANS_E_HIP). */
int rans_gaussian_tables(const double *scales, int32_t num_tables, double tail_z,
                         int32_t cdf_stride, int32_t *cdf, int32_t *cdf_lengths, int32_t *offsets,
                         int32_t *row_status, hipStream_t hstream);

int rans_quantize_pmfs(const double *pmf, const int32_t *pmf_lengths, int32_t num_tables,
                       int32_t pmf_stride, int32_t cdf_stride, int32_t *cdf, int32_t *cdf_lengths,
                       int32_t *row_status, hipStream_t hstream);

/* The mean-scale front end around the coder (kompressor BENCHMARKS.md,
 * sections 3 and 4: the codec computes each position's table index on the
 * GPU, build_indexes, and hands symbols and indexes to the coder as int32).
 *
 * rans_latent_symbols: for i < n, symbols[i] = round-half-even(y[i] -
 * means[i]) computed in single precision and saturated to int32 (NaN gives
 * INT32_MIN), so a value int32 cannot hold reaches the coder as one it
 * refuses with RANS_E_SYMBOL_RANGE; indexes[i] = (K - 1) - #{k < K - 1 :
 * scales[i] <= scale_table[k]}, i.e. for an ascending table the first k with
 * scales[i] <= scale_table[k], K - 1 when there is none or scales[i] is NaN.
 * K = num_scales in [1, RANS_MAX_TABLES]; the result follows that rule for
 * any table, fastest when the first K - 1 scales are non-decreasing.
 *
 * rans_dequantize: y_hat[i] = (float)symbols[i] + means[i] in single
 * precision.
 *
 * Device pointers, float32 / int32 arrays of n entries (16-byte aligned
 * arrays take 16-byte accesses; any 4-byte alignment works).  n = 0 is a
 * no-op.  Returns RANS_E_ARG for null pointers or a bad K, RANS_E_HIP for a
 * failed launch; nothing data-dependent fails. */
int rans_latent_symbols(const float *y, const float *means, const float *scales, uint64_t n,
                        const float *scale_table, int32_t num_scales, int32_t *symbols,
                        int32_t *indexes, hipStream_t hstream);

int rans_dequantize(const int32_t *symbols, const float *means, uint64_t n, float *y_hat,
                    hipStream_t hstream);

/* The front end fused into the interleaved encoder (kompressor BENCHMARKS.md,
 * section 4: the int32 symbols and indexes a codec hands to its coder are a
 * round trip through memory that the coder can avoid).  The container, the
 * status and every error are exactly those of rans_encode_interleaved /
 * rans_encode_interleaved_prepared on
 *   rans_latent_symbols(y, means, scales, n, scale_table, num_tables, ...),
 * i.e. symbol and table index of each position follow the rules above, with
 * the scale table holding one scale per CDF row (num_tables entries, any
 * order; ascending is fastest).  The symbols and indexes are never written to
 * memory: the encoder reads 12 bytes per position (y, means, scales, float32
 * device arrays of n entries) instead of the front end's 12 in, 8 out and the
 * encoder's 8 in.  A position whose symbol saturates (NaN, or beyond int32)
 * makes *status RANS_E_SYMBOL_RANGE, as it would in two passes.  Workspace:
 * rans_interleaved_workspace_bytes(n, num_streams, num_tables, cdf_stride);
 * the _prepared form needs the tables prepared on it, as for
 * rans_encode_interleaved_prepared. */
int rans_encode_interleaved_latent(const float *y, const float *means, const float *scales,
                                   uint64_t n, const float *scale_table, const int32_t *cdf,
                                   const int32_t *cdf_lengths, const int32_t *offsets,
                                   int32_t num_tables, int32_t cdf_stride, uint32_t num_streams,
                                   uint32_t *stream, uint64_t stream_capacity_words,
                                   uint64_t *stream_words, int32_t *status, void *workspace,
                                   uint64_t workspace_bytes, hipStream_t hstream);

int rans_encode_interleaved_latent_prepared(const float *y, const float *means,
                                            const float *scales, uint64_t n,
                                            const float *scale_table, int32_t num_tables,
                                            int32_t cdf_stride, uint32_t num_streams,
                                            uint32_t *stream, uint64_t stream_capacity_words,
                                            uint64_t *stream_words, int32_t *status,
                                            void *workspace, uint64_t workspace_bytes,
                                            hipStream_t hstream);

/* For callers that cannot allocate device memory (code under stream capture,
 * tight serving loops, harnesses that forbid hipMalloc): the encode above
 * with no workspace argument.  The workspace is a fixed array of 64 MiB that
 * the library holds on every GPU it runs on, from module load until the
 * process ends; its device address is looked up once per device, and on the
 * first call on a device a fill kernel enqueued on `hstream` zeroes its
 * bookkeeping prefix.  The call allocates nothing.  A call whose
 * rans_workspace_bytes(n, num_lanes, num_tables, cdf_stride) exceeds 64 MiB
 * returns RANS_E_WORKSPACE (about 8M symbols with the 64-row table set).
 * Every call on one GPU shares that GPU's array, which keeps the last call's
 * contents: calls on one GPU must not overlap in time (order them on one
 * stream or synchronise), else they race.  Arguments, outputs, errors and
 * the container are those of rans_encode_with_indexes. */
int rans_encode_noalloc(const int32_t *symbols, const int32_t *indexes, uint64_t n,
                        const int32_t *cdf, const int32_t *cdf_lengths, const int32_t *offsets,
                        int32_t num_tables, int32_t cdf_stride, uint32_t num_lanes,
                        uint32_t *stream, uint64_t stream_capacity_words, uint64_t *stream_words,
                        int32_t *status, hipStream_t hstream);

/* Static text for a status code. */
const char *rans_status_string(int code);

#ifdef __cplusplus
}
#endif

#endif /* RANS_HIP_H */
