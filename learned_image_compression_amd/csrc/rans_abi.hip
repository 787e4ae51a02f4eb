// rans_abi.hip -- the extern "C" entry points: host-side argument checks, then
// launches on the caller's stream.  No call allocates memory or synchronises.
#include "rans_internal.hpp"

using namespace rans;

namespace {

bool aligned256(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 255u) == 0; }

int check_workspace(void *ws, uint64_t bytes, uint64_t need)
{
    if (!ws || !aligned256(ws) || bytes < need)
        return RANS_E_WORKSPACE;
    return RANS_OK;
}

int check_tables(const int32_t *cdf, const int32_t *lengths, const int32_t *offsets,
                 int32_t num_tables, int32_t stride)
{
    if (!cdf || !lengths || !offsets)
        return RANS_E_ARG;
    if (num_tables < 1 || num_tables > RANS_MAX_TABLES || stride < 3 || stride > RANS_MAX_STRIDE)
        return RANS_E_TABLE;
    return RANS_OK;
}

// Size limits of one call: the kernels address each wave's symbols, scratch
// and stream words through 32-bit buffer offsets.
bool sizes_ok(uint64_t n, uint32_t lanes)
{
    return n <= RANS_MAX_SYMBOLS && lanes <= RANS_MAX_LANES;
}

int launched(hipError_t e) { return e == hipSuccess ? RANS_OK : RANS_E_HIP; }

// A table count or row stride clamped to [1, hi]: sizes are computed before
// the arguments are checked, and stay finite for any input.
uint64_t clamp_size(int32_t v, uint32_t hi)
{
    return v < 1 ? 1u : ((uint32_t)v > hi ? (uint64_t)hi : (uint64_t)v);
}

// End of the table regions, where the scratch area starts.
uint64_t tables_end(int32_t num_tables, int32_t cdf_stride)
{
    return ws_scratch_offset(clamp_size(num_tables, RANS_MAX_TABLES),
                             clamp_size(cdf_stride, RANS_MAX_STRIDE));
}

// log2 of a piece count: a power of two in [1, RANS_MAX_PIECES], else -1
int pieces_log2_of(uint32_t pieces)
{
    for (int l = 0; (1u << l) <= RANS_MAX_PIECES; ++l)
        if (pieces == (1u << l))
            return l;
    return -1;
}

}  // namespace

extern "C" {

uint64_t rans_encode_bound_words(uint64_t n, uint32_t num_lanes)
{
    return 1ull + num_lanes + ws_scratch_words(n, num_lanes);
}

uint64_t rans_workspace_bytes(uint64_t n, uint32_t num_lanes, int32_t num_tables,
                              int32_t cdf_stride)
{
    return tables_end(num_tables, cdf_stride) + 4ull * ws_scratch_words(n, num_lanes);
}

int rans_prepare_tables(const int32_t *cdf, const int32_t *cdf_lengths, const int32_t *offsets,
                        int32_t num_tables, int32_t cdf_stride, void *workspace,
                        uint64_t workspace_bytes, hipStream_t hstream)
{
    int rc = check_tables(cdf, cdf_lengths, offsets, num_tables, cdf_stride);
    if (rc)
        return rc;
    if ((rc = check_workspace(workspace, workspace_bytes, tables_end(num_tables, cdf_stride))))
        return rc;
    PrepArgs a{cdf, cdf_lengths, offsets, num_tables, cdf_stride,
               static_cast<uint8_t *>(workspace)};
    return launched(launch_prep(a, hstream));
}

int rans_encode_prepared(const int32_t *symbols, const int32_t *indexes, uint64_t n,
                         int32_t num_tables, int32_t cdf_stride, uint32_t num_lanes,
                         uint32_t *stream, uint64_t stream_capacity_words,
                         uint64_t *stream_words, int32_t *status, void *workspace,
                         uint64_t workspace_bytes, hipStream_t hstream)
{
    if (num_lanes == 0 || !stream || !stream_words || !status || (n && (!symbols || !indexes)))
        return RANS_E_ARG;
    if (num_tables < 1 || num_tables > RANS_MAX_TABLES || cdf_stride < 3 ||
        cdf_stride > RANS_MAX_STRIDE)
        return RANS_E_TABLE;
    if (!sizes_ok(n, num_lanes) || stream_capacity_words < 1ull + num_lanes)
        return RANS_E_ARG;
    int rc = check_workspace(workspace, workspace_bytes,
                             rans_workspace_bytes(n, num_lanes, num_tables, cdf_stride));
    if (rc)
        return rc;
    EncodeArgs a{symbols, indexes, n, num_lanes, num_tables, cdf_stride, stream,
                 stream_capacity_words, stream_words, status, static_cast<uint8_t *>(workspace),
                 0u, nullptr};
    return launched(launch_encode(a, hstream));
}

int rans_decode_prepared(const uint32_t *stream, uint64_t stream_capacity_words,
                         const int32_t *indexes, uint64_t n, int32_t num_tables,
                         int32_t cdf_stride, int32_t *symbols, int32_t *status, void *workspace,
                         uint64_t workspace_bytes, hipStream_t hstream)
{
    if (!stream || !status || (n && (!symbols || !indexes)))
        return RANS_E_ARG;
    if (num_tables < 1 || num_tables > RANS_MAX_TABLES || cdf_stride < 3 ||
        cdf_stride > RANS_MAX_STRIDE)
        return RANS_E_TABLE;
    if (n > RANS_MAX_SYMBOLS || stream_capacity_words < 1)
        return RANS_E_ARG;
    // the decoder uses only the header and the prepared tables
    int rc = check_workspace(workspace, workspace_bytes, tables_end(num_tables, cdf_stride));
    if (rc)
        return rc;
    DecodeArgs a{stream, stream_capacity_words, indexes, n, num_tables, cdf_stride, symbols,
                 status, static_cast<uint8_t *>(workspace), 0u, nullptr, 0u};
    return launched(launch_decode(a, hstream));
}

int rans_encode_with_indexes(const int32_t *symbols, const int32_t *indexes, uint64_t n,
                             const int32_t *cdf, const int32_t *cdf_lengths,
                             const int32_t *offsets, int32_t num_tables, int32_t cdf_stride,
                             uint32_t num_lanes, uint32_t *stream,
                             uint64_t stream_capacity_words, uint64_t *stream_words,
                             int32_t *status, void *workspace, uint64_t workspace_bytes,
                             hipStream_t hstream)
{
    if (num_lanes == 0 || !stream || !stream_words || !status || (n && (!symbols || !indexes)))
        return RANS_E_ARG;
    if (!sizes_ok(n, num_lanes) || stream_capacity_words < 1ull + num_lanes)
        return RANS_E_ARG;
    int rc = check_tables(cdf, cdf_lengths, offsets, num_tables, cdf_stride);
    if (rc)
        return rc;
    if ((rc = check_workspace(workspace, workspace_bytes,
                              rans_workspace_bytes(n, num_lanes, num_tables, cdf_stride))))
        return rc;
    if ((rc = rans_prepare_tables(cdf, cdf_lengths, offsets, num_tables, cdf_stride, workspace,
                                  workspace_bytes, hstream)))
        return rc;
    return rans_encode_prepared(symbols, indexes, n, num_tables, cdf_stride, num_lanes, stream,
                                stream_capacity_words, stream_words, status, workspace,
                                workspace_bytes, hstream);
}

int rans_decode_with_indexes(const uint32_t *stream, uint64_t stream_capacity_words,
                             const int32_t *indexes, uint64_t n,
                             const int32_t *cdf, const int32_t *cdf_lengths,
                             const int32_t *offsets, int32_t num_tables, int32_t cdf_stride,
                             int32_t *symbols, int32_t *status, void *workspace,
                             uint64_t workspace_bytes, hipStream_t hstream)
{
    if (!stream || !status || (n && (!symbols || !indexes)))
        return RANS_E_ARG;
    if (n > RANS_MAX_SYMBOLS || stream_capacity_words < 1)
        return RANS_E_ARG;
    int rc = check_tables(cdf, cdf_lengths, offsets, num_tables, cdf_stride);
    if (rc)
        return rc;
    if ((rc = check_workspace(workspace, workspace_bytes, tables_end(num_tables, cdf_stride))))
        return rc;
    if ((rc = rans_prepare_tables(cdf, cdf_lengths, offsets, num_tables, cdf_stride, workspace,
                                  workspace_bytes, hstream)))
        return rc;
    return rans_decode_prepared(stream, stream_capacity_words, indexes, n, num_tables,
                                cdf_stride, symbols, status, workspace, workspace_bytes, hstream);
}

int rans_encode_with_splits(const int32_t *symbols, const int32_t *indexes, uint64_t n,
                            const int32_t *cdf, const int32_t *cdf_lengths, const int32_t *offsets,
                            int32_t num_tables, int32_t cdf_stride, uint32_t num_lanes,
                            uint32_t pieces, uint32_t *stream, uint64_t stream_capacity_words,
                            uint64_t *stream_words, uint32_t *split_meta, int32_t *status,
                            void *workspace, uint64_t workspace_bytes, hipStream_t hstream)
{
    const int pl = pieces_log2_of(pieces);
    if (pl < 0 || (pieces > 1 && !split_meta))
        return RANS_E_ARG;
    if (num_lanes == 0 || !stream || !stream_words || !status || (n && (!symbols || !indexes)))
        return RANS_E_ARG;
    if (!sizes_ok(n, num_lanes) || stream_capacity_words < 1ull + num_lanes)
        return RANS_E_ARG;
    int rc = check_tables(cdf, cdf_lengths, offsets, num_tables, cdf_stride);
    if (rc)
        return rc;
    if ((rc = check_workspace(workspace, workspace_bytes,
                              rans_workspace_bytes(n, num_lanes, num_tables, cdf_stride))))
        return rc;
    if ((rc = rans_prepare_tables(cdf, cdf_lengths, offsets, num_tables, cdf_stride, workspace,
                                  workspace_bytes, hstream)))
        return rc;
    EncodeArgs a{symbols, indexes, n, num_lanes, num_tables, cdf_stride, stream,
                 stream_capacity_words, stream_words, status, static_cast<uint8_t *>(workspace),
                 0u, nullptr};
    a.pieces_log2 = (uint32_t)pl;
    a.split_meta = pl ? split_meta : nullptr;
    return launched(launch_encode(a, hstream));
}

int rans_decode_with_splits(const uint32_t *stream, uint64_t stream_capacity_words,
                            const int32_t *indexes, uint64_t n,
                            const int32_t *cdf, const int32_t *cdf_lengths,
                            const int32_t *offsets, int32_t num_tables, int32_t cdf_stride,
                            uint32_t pieces, const uint32_t *split_meta, uint64_t split_words,
                            int32_t *symbols, int32_t *status, void *workspace,
                            uint64_t workspace_bytes, hipStream_t hstream)
{
    const int pl = pieces_log2_of(pieces);
    if (pl < 0 || (pieces > 1 && !split_meta))
        return RANS_E_ARG;
    if (!stream || !status || (n && (!symbols || !indexes)))
        return RANS_E_ARG;
    if (n > RANS_MAX_SYMBOLS || stream_capacity_words < 1)
        return RANS_E_ARG;
    int rc = check_tables(cdf, cdf_lengths, offsets, num_tables, cdf_stride);
    if (rc)
        return rc;
    if ((rc = check_workspace(workspace, workspace_bytes, tables_end(num_tables, cdf_stride))))
        return rc;
    if ((rc = rans_prepare_tables(cdf, cdf_lengths, offsets, num_tables, cdf_stride, workspace,
                                  workspace_bytes, hstream)))
        return rc;
    DecodeArgs a{stream, stream_capacity_words, indexes, n, num_tables, cdf_stride, symbols,
                 status, static_cast<uint8_t *>(workspace), 0u, nullptr, 0u};
    a.pieces_log2 = (uint32_t)pl;
    a.split_meta = pl ? split_meta : nullptr;
    a.split_words = pl ? split_words : 0u;
    return launched(launch_decode(a, hstream));
}

uint64_t rans_interleaved_bound_words(uint64_t n, uint32_t num_streams)
{
    return 1ull + num_streams + il_scratch_words(n, num_streams);
}

uint64_t rans_interleaved_workspace_bytes(uint64_t n, uint32_t num_streams, int32_t num_tables,
                                          int32_t cdf_stride)
{
    return il_counts_offset(n, num_streams, clamp_size(num_tables, RANS_MAX_TABLES),
                            clamp_size(cdf_stride, RANS_MAX_STRIDE)) +
           4ull * num_streams;
}

int rans_encode_interleaved_prepared(const int32_t *symbols, const int32_t *indexes, uint64_t n,
                                     int32_t num_tables, int32_t cdf_stride, uint32_t num_streams,
                                     uint32_t *stream, uint64_t stream_capacity_words,
                                     uint64_t *stream_words, int32_t *status, void *workspace,
                                     uint64_t workspace_bytes, hipStream_t hstream)
{
    if (num_streams == 0 || num_streams > RANS_MAX_STREAMS || !stream || !stream_words ||
        !status || (n && (!symbols || !indexes)))
        return RANS_E_ARG;
    if (num_tables < 1 || num_tables > RANS_MAX_TABLES || cdf_stride < 3 ||
        cdf_stride > RANS_MAX_STRIDE)
        return RANS_E_TABLE;
    if (n > RANS_MAX_SYMBOLS || stream_capacity_words < 1ull + num_streams)
        return RANS_E_ARG;
    int rc = check_workspace(workspace, workspace_bytes,
                             rans_interleaved_workspace_bytes(n, num_streams, num_tables,
                                                              cdf_stride));
    if (rc)
        return rc;
    uint8_t *ws = static_cast<uint8_t *>(workspace);
    IlArgs a{symbols, indexes, n, num_streams, num_tables, cdf_stride, stream, nullptr,
             stream_capacity_words, stream_words, nullptr, status, ws,
             reinterpret_cast<uint32_t *>(ws + tables_end(num_tables, cdf_stride)),
             reinterpret_cast<uint32_t *>(ws + il_counts_offset(n, num_streams, num_tables,
                                                                cdf_stride))};
    return launched(launch_il_encode(a, hstream));
}

int rans_encode_interleaved_latent_prepared(const float *y, const float *means,
                                            const float *scales, uint64_t n,
                                            const float *scale_table, int32_t num_tables,
                                            int32_t cdf_stride, uint32_t num_streams,
                                            uint32_t *stream, uint64_t stream_capacity_words,
                                            uint64_t *stream_words, int32_t *status,
                                            void *workspace, uint64_t workspace_bytes,
                                            hipStream_t hstream)
{
    if (num_streams == 0 || num_streams > RANS_MAX_STREAMS || !stream || !stream_words ||
        !status || !scale_table || (n && (!y || !means || !scales)))
        return RANS_E_ARG;
    if (num_tables < 1 || num_tables > RANS_MAX_TABLES || cdf_stride < 3 ||
        cdf_stride > RANS_MAX_STRIDE)
        return RANS_E_TABLE;
    if (n > RANS_MAX_SYMBOLS || stream_capacity_words < 1ull + num_streams)
        return RANS_E_ARG;
    int rc = check_workspace(workspace, workspace_bytes,
                             rans_interleaved_workspace_bytes(n, num_streams, num_tables,
                                                              cdf_stride));
    if (rc)
        return rc;
    uint8_t *ws = static_cast<uint8_t *>(workspace);
    IlArgs a{nullptr, nullptr, n, num_streams, num_tables, cdf_stride, stream, nullptr,
             stream_capacity_words, stream_words, nullptr, status, ws,
             reinterpret_cast<uint32_t *>(ws + tables_end(num_tables, cdf_stride)),
             reinterpret_cast<uint32_t *>(ws + il_counts_offset(n, num_streams, num_tables,
                                                                cdf_stride)),
             y, means, scales, scale_table};
    return launched(launch_il_encode(a, hstream));
}

int rans_encode_interleaved_latent(const float *y, const float *means, const float *scales,
                                   uint64_t n, const float *scale_table, const int32_t *cdf,
                                   const int32_t *cdf_lengths, const int32_t *offsets,
                                   int32_t num_tables, int32_t cdf_stride, uint32_t num_streams,
                                   uint32_t *stream, uint64_t stream_capacity_words,
                                   uint64_t *stream_words, int32_t *status, void *workspace,
                                   uint64_t workspace_bytes, hipStream_t hstream)
{
    if (num_streams == 0 || num_streams > RANS_MAX_STREAMS || !stream || !stream_words ||
        !status || !scale_table || (n && (!y || !means || !scales)))
        return RANS_E_ARG;
    if (n > RANS_MAX_SYMBOLS || stream_capacity_words < 1ull + num_streams)
        return RANS_E_ARG;
    int rc = check_tables(cdf, cdf_lengths, offsets, num_tables, cdf_stride);
    if (rc)
        return rc;
    if ((rc = check_workspace(workspace, workspace_bytes,
                              rans_interleaved_workspace_bytes(n, num_streams, num_tables,
                                                               cdf_stride))))
        return rc;
    if ((rc = rans_prepare_tables(cdf, cdf_lengths, offsets, num_tables, cdf_stride, workspace,
                                  workspace_bytes, hstream)))
        return rc;
    return rans_encode_interleaved_latent_prepared(y, means, scales, n, scale_table, num_tables,
                                                   cdf_stride, num_streams, stream,
                                                   stream_capacity_words, stream_words, status,
                                                   workspace, workspace_bytes, hstream);
}

int rans_decode_interleaved_prepared(const uint32_t *stream, uint64_t stream_capacity_words,
                                     const int32_t *indexes, uint64_t n, int32_t num_tables,
                                     int32_t cdf_stride, uint32_t num_streams, int32_t *symbols,
                                     int32_t *status, void *workspace, uint64_t workspace_bytes,
                                     hipStream_t hstream)
{
    if (num_streams == 0 || num_streams > RANS_MAX_STREAMS || !stream || !status ||
        (n && (!symbols || !indexes)))
        return RANS_E_ARG;
    if (num_tables < 1 || num_tables > RANS_MAX_TABLES || cdf_stride < 3 ||
        cdf_stride > RANS_MAX_STRIDE)
        return RANS_E_TABLE;
    if (n > RANS_MAX_SYMBOLS || stream_capacity_words < 1ull + num_streams)
        return RANS_E_ARG;
    int rc = check_workspace(workspace, workspace_bytes, tables_end(num_tables, cdf_stride));
    if (rc)
        return rc;
    IlArgs a{nullptr, indexes, n, num_streams, num_tables, cdf_stride, nullptr, stream,
             stream_capacity_words, nullptr, symbols, status, static_cast<uint8_t *>(workspace),
             nullptr, nullptr};
    return launched(launch_il_decode(a, hstream));
}

int rans_encode_interleaved(const int32_t *symbols, const int32_t *indexes, uint64_t n,
                            const int32_t *cdf, const int32_t *cdf_lengths,
                            const int32_t *offsets, int32_t num_tables, int32_t cdf_stride,
                            uint32_t num_streams, uint32_t *stream,
                            uint64_t stream_capacity_words, uint64_t *stream_words,
                            int32_t *status, void *workspace, uint64_t workspace_bytes,
                            hipStream_t hstream)
{
    if (num_streams == 0 || num_streams > RANS_MAX_STREAMS || !stream || !stream_words ||
        !status || (n && (!symbols || !indexes)))
        return RANS_E_ARG;
    if (n > RANS_MAX_SYMBOLS || stream_capacity_words < 1ull + num_streams)
        return RANS_E_ARG;
    int rc = check_tables(cdf, cdf_lengths, offsets, num_tables, cdf_stride);
    if (rc)
        return rc;
    if ((rc = check_workspace(workspace, workspace_bytes,
                              rans_interleaved_workspace_bytes(n, num_streams, num_tables,
                                                               cdf_stride))))
        return rc;
    if ((rc = rans_prepare_tables(cdf, cdf_lengths, offsets, num_tables, cdf_stride, workspace,
                                  workspace_bytes, hstream)))
        return rc;
    return rans_encode_interleaved_prepared(symbols, indexes, n, num_tables, cdf_stride,
                                            num_streams, stream, stream_capacity_words,
                                            stream_words, status, workspace, workspace_bytes,
                                            hstream);
}

int rans_decode_interleaved(const uint32_t *stream, uint64_t stream_capacity_words,
                            const int32_t *indexes, uint64_t n,
                            const int32_t *cdf, const int32_t *cdf_lengths,
                            const int32_t *offsets, int32_t num_tables, int32_t cdf_stride,
                            uint32_t num_streams, int32_t *symbols, int32_t *status,
                            void *workspace, uint64_t workspace_bytes, hipStream_t hstream)
{
    if (num_streams == 0 || num_streams > RANS_MAX_STREAMS || !stream || !status ||
        (n && (!symbols || !indexes)))
        return RANS_E_ARG;
    if (n > RANS_MAX_SYMBOLS || stream_capacity_words < 1ull + num_streams)
        return RANS_E_ARG;
    int rc = check_tables(cdf, cdf_lengths, offsets, num_tables, cdf_stride);
    if (rc)
        return rc;
    if ((rc = check_workspace(workspace, workspace_bytes, tables_end(num_tables, cdf_stride))))
        return rc;
    if ((rc = rans_prepare_tables(cdf, cdf_lengths, offsets, num_tables, cdf_stride, workspace,
                                  workspace_bytes, hstream)))
        return rc;
    return rans_decode_interleaved_prepared(stream, stream_capacity_words, indexes, n,
                                            num_tables, cdf_stride, num_streams, symbols, status,
                                            workspace, workspace_bytes, hstream);
}

int rans_gaussian_tables(const double *scales, int32_t num_tables, double tail_z,
                         int32_t cdf_stride, int32_t *cdf, int32_t *cdf_lengths, int32_t *offsets,
                         int32_t *row_status, hipStream_t hstream)
{
    if (!scales || !cdf || !cdf_lengths || !offsets || !row_status)
        return RANS_E_ARG;
    if (num_tables < 1 || num_tables > RANS_MAX_TABLES || cdf_stride < 3 ||
        cdf_stride > RANS_MAX_STRIDE || !(tail_z > 0.0 && tail_z < 1e300))
        return RANS_E_ARG;
    TableArgs a{scales, tail_z, nullptr, nullptr, 0, num_tables, cdf_stride, cdf, cdf_lengths,
                offsets, row_status};
    return launched(launch_table_rows(a, hstream));
}

int rans_quantize_pmfs(const double *pmf, const int32_t *pmf_lengths, int32_t num_tables,
                       int32_t pmf_stride, int32_t cdf_stride, int32_t *cdf, int32_t *cdf_lengths,
                       int32_t *row_status, hipStream_t hstream)
{
    if (!pmf || !pmf_lengths || !cdf || !cdf_lengths || !row_status)
        return RANS_E_ARG;
    if (num_tables < 1 || num_tables > RANS_MAX_TABLES || pmf_stride < 2 || cdf_stride < 3 ||
        cdf_stride > RANS_MAX_STRIDE)
        return RANS_E_ARG;
    TableArgs a{nullptr, 0.0, pmf, pmf_lengths, pmf_stride, num_tables, cdf_stride, cdf,
                cdf_lengths, nullptr, row_status};
    return launched(launch_table_rows(a, hstream));
}

int rans_latent_symbols(const float *y, const float *means, const float *scales, uint64_t n,
                        const float *scale_table, int32_t num_scales, int32_t *symbols,
                        int32_t *indexes, hipStream_t hstream)
{
    if (!scale_table || num_scales < 1 || num_scales > RANS_MAX_TABLES)
        return RANS_E_ARG;
    if (n == 0)
        return RANS_OK;
    if (!y || !means || !scales || !symbols || !indexes)
        return RANS_E_ARG;
    LatentArgs a{y, means, scales, n, scale_table, num_scales, symbols, indexes};
    return launched(launch_latent_symbols(a, hstream));
}

int rans_dequantize(const int32_t *symbols, const float *means, uint64_t n, float *y_hat,
                    hipStream_t hstream)
{
    if (n == 0)
        return RANS_OK;
    if (!symbols || !means || !y_hat)
        return RANS_E_ARG;
    DequantArgs a{symbols, means, n, y_hat};
    return launched(launch_dequantize(a, hstream));
}

const char *rans_status_string(int code)
{
    switch (code) {
    case RANS_OK: return "ok";
    case RANS_E_ARG: return "invalid argument";
    case RANS_E_TABLE: return "malformed CDF table";
    case RANS_E_INDEX: return "table index out of range";
    case RANS_E_SYMBOL_RANGE: return "symbol too far outside its coded range";
    case RANS_E_CAPACITY: return "output capacity too small";
    case RANS_E_CORRUPT: return "corrupt stream";
    case RANS_E_WORKSPACE: return "workspace missing, misaligned or too small";
    case RANS_E_HIP: return "HIP launch failure";
    default: return "unknown status";
    }
}

}  // extern "C"
