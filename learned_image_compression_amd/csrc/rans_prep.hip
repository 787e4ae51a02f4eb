// rans_prep.hip -- table preparation: validate CDF rows, pack them as u16 into
// the workspace, and build the decoder's per-row bucket lookup.
//
// The pages rebuild or re-marshal the tables on every call (kompressor
// BENCHMARKS.md section 4: cdf/len/offset lists rebuilt each call; torch_ans
// "Performance Tuning": init_params rebuilds the quantised CDFs and the
// lookup table, about 0.2 ms).  Here one launch does it: every block scans
// the row lengths redundantly (K <= 4096), so no block waits for another.
//
// Two packed table sets in the workspace, each copied verbatim into LDS by
// one coding kernel:
//   decoder  [RowMeta x K][u16 cdfm1 x sum(len) + 4, padded to 16 B]
//            [u16 first x K * 2^q]
//   encoder  [RowMeta x K][u32 (start | f << 16) x sum(len)]
// cdfm1 holds start(k) - 1 mod 2^16, so that "cum >= start(k)" is
// "cum > cdfm1[k]" for every entry, the terminal 65536 included (stored as
// 65535), and f = cdfm1[k+1] - cdfm1[k] mod 2^16 (every f is in [1, 65535]).
//
// Decoder lookup (inverse-CDF table in the sense of torch_ans "Usage",
// "Inverse CDF decoding": a table keyed by the low state bits).  Each row gets
// 2^q buckets of width 2^(16-q) cumulative values, q the largest value <= 12
// for which the whole set fits the LDS budget (a set that fits for no q stays
// in the workspace, with q = 9); first[b] is the slot holding the bucket's
// lowest value.  The decoder reads cdfm1[first[b] .. +3] in one
// 8-byte access and resolves every cum that falls in those three slots.
#include "rans_internal.hpp"

namespace rans {

// One block per row (up to 256 blocks, a grid-stride loop beyond): 1024
// threads, so that the longest rows (3133 entries for the 64-row Gaussian
// set) take a few entries and buckets per thread.
constexpr int kPrepThreads = 1024;
constexpr int kPrepWaves = kPrepThreads / kWave;

__global__ __launch_bounds__(kPrepThreads) void prep_kernel(PrepArgs a)
{
    __shared__ uint32_t s_base[RANS_MAX_TABLES];
    __shared__ uint32_t s_wave[kPrepWaves];
    __shared__ int32_t s_val[RANS_MAX_STRIDE];

    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1), wv = tid / kWave;
    const int K = a.num_tables;
    const uint32_t stride = (uint32_t)a.stride;
    WsHeader *hdr = reinterpret_cast<WsHeader *>(a.ws);
    uint8_t *tab = a.ws + ws_dec_offset();
    // this block's first row's offset, and its first row's entries (up to
    // the stride, eight loads a thread: the row's length is not known yet),
    // requested before anything waits
    const int32_t off_first = (int)blockIdx.x < K ? a.offsets[blockIdx.x] : 0;
    int32_t first_row[8];
    {
        const int32_t *row = a.cdf + (int64_t)blockIdx.x * stride;
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const uint32_t k = tid + u * kPrepThreads;
            first_row[u] = ((int)blockIdx.x < K && k < stride) ? row[k] : 0;
        }
    }

    // --- 1. effective lengths and their exclusive scan (every block) ----------
    // thread t sums rows [t*chunk, (t+1)*chunk); a wave scan by shuffles, then
    // one pass over the wave totals
    const int chunk = (K + kPrepThreads - 1) / kPrepThreads;
    const int r0 = tid * chunk;
    const int r1 = min(K, r0 + chunk);
    uint32_t sum = 0;
    for (int r = r0; r < r1; ++r) {
        int32_t len = a.lengths[r];
        uint32_t eff = (len >= 3 && (uint32_t)len <= stride) ? (uint32_t)len : 3u;
        s_base[r] = eff;
        sum += eff;
    }
    uint32_t incl = sum;
    for (int o = 1; o < kWave; o <<= 1) {
        const uint32_t v = __shfl_up(incl, o, kWave);
        incl += lane >= o ? v : 0u;
    }
    if (lane == kWave - 1)
        s_wave[wv] = incl;
    __syncthreads();
    uint32_t before = 0, total = 0;
    for (int w = 0; w < kPrepWaves; ++w) {
        const uint32_t v = s_wave[w];
        before += w < wv ? v : 0u;
        total += v;
    }
    uint32_t run = before + incl - sum;
    for (int r = r0; r < r1; ++r) {
        uint32_t eff = s_base[r];
        s_base[r] = run;
        run += eff;
    }
    __syncthreads();

    // decoder set [meta | cdfm1 | first], encoder set [meta | pairs]; each is
    // staged into LDS by the coding kernels when it fits their budget, else
    // read from its workspace region, with 2^kGlobalLutQ buckets per row
    const uint32_t meta_bytes = (uint32_t)meta_bytes_of(K);
    // (8 spare bytes: the decoder reads four entries from any row position)
    const uint64_t cdf_bytes = align_up(2ull * total + 8, 16);
    const uint64_t enc_bytes = enc_set_bytes(K, total);
    const bool enc_lds = enc_bytes <= kEncTableBudget;
    int q = -1;
    for (int t = (int)kMaxLutQ; t >= 0; --t) {
        if (dec_set_bytes(K, total, t) <= kDecTableBudget) {
            q = t;
            break;
        }
    }
    const bool dec_lds = q >= 0;
    if (q < 0)
        q = (int)kGlobalLutQ;
    const uint64_t dec_bytes = dec_set_bytes(K, total, q);

    if (blockIdx.x == 0 && tid == 0) {
        hdr->num_tables = (uint32_t)K;
        hdr->cdf_stride = stride;
        hdr->total_len = total;
        hdr->lut_q = (uint32_t)q;
        hdr->enc_bytes = (uint32_t)enc_bytes;
        hdr->dec_bytes = (uint32_t)dec_bytes;
        hdr->enc_lds = enc_lds ? 1u : 0u;
        hdr->dec_lds = dec_lds ? 1u : 0u;
        hdr->err = 0;
        hdr->done = 0;
        hdr->total_words = 0;
        __threadfence();
        hdr->magic = kMagic;
    }

    RowMeta *dmeta = reinterpret_cast<RowMeta *>(tab);
    uint16_t *cdfm1 = reinterpret_cast<uint16_t *>(tab + meta_bytes);
    uint16_t *first = reinterpret_cast<uint16_t *>(tab + meta_bytes + cdf_bytes);
    uint8_t *etab = a.ws + ws_enc_offset((uint32_t)K, stride);
    RowMeta *emeta = reinterpret_cast<RowMeta *>(etab);
    uint32_t *pairs = reinterpret_cast<uint32_t *>(etab + meta_bytes);
    const uint32_t width = kTotal >> q;
    // the four spare entries after the last row read as the terminal value
    // (65535), like the first entry of every following row, so a window read
    // that runs past a row's terminal never compares below the cumulative value
    if (blockIdx.x == 0 && tid < 4)
        cdfm1[total + tid] = 0xFFFFu;

    // --- 2. rows of this block ------------------------------------------------
    for (int r = blockIdx.x; r < K; r += gridDim.x) {
        const int32_t len_in = a.lengths[r];
        const bool len_ok = len_in >= 3 && (uint32_t)len_in <= stride;
        const uint32_t len = len_ok ? (uint32_t)len_in : 3u;
        const uint32_t base = s_base[r];
        const int32_t *row = a.cdf + (int64_t)r * stride;
        int bad = len_ok ? 0 : 1;
        // stage the row as int32 (eight loads in flight per thread; the
        // block's first row was loaded at the start), then check it
        for (uint32_t k0 = tid; k0 < len; k0 += 8 * kPrepThreads) {
            int32_t v[8];
            const bool pre = r == (int)blockIdx.x && k0 == (uint32_t)tid;
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const uint32_t k = k0 + u * kPrepThreads;
                v[u] = k < len ? (len_ok ? (pre ? first_row[u] : row[k])
                                         : (k == 0 ? 0 : (k == 1 ? 1 : (int32_t)kTotal)))
                               : 0;
            }
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const uint32_t k = k0 + u * kPrepThreads;
                if (k < len)
                    s_val[k] = v[u];
            }
        }
        __syncthreads();
        for (uint32_t k = tid; k < len; k += kPrepThreads) {
            const int32_t v = s_val[k];
            if (k == 0 && v != 0)
                bad = 1;
            if (k + 1 == len && v != (int32_t)kTotal)
                bad = 1;
            if (k > 0 && v <= s_val[k - 1])
                bad = 1;
            cdfm1[base + k] = (uint16_t)((uint32_t)v - 1u);
            {
                // slot k: start | f << 16 (the terminal entry gets 0)
                const uint32_t f = k + 1 < len ? (uint32_t)(s_val[k + 1] - v) & 0xFFFFu : 0u;
                pairs[base + k] = (k + 1 < len) ? ((uint32_t)v & 0xFFFFu) | (f << 16) : 0u;
            }
        }
        bad = __syncthreads_or(bad);
        if (tid == 0) {
            const int32_t off = r == (int)blockIdx.x ? off_first : a.offsets[r];
            const uint32_t mv = len - 2;
            // slots below mv take the fast paths if offset + slot fits int32
            const bool fits = (int64_t)off + (int64_t)mv - 1 <= (int64_t)INT32_MAX;
            RowMeta m;
            m.offset = off;
            m.mvf = mv | ((fits ? mv : 0u) << 16);
            m.base = (uint32_t)(meta_bytes + 2ull * base);
            m.lut = (uint32_t)(meta_bytes + cdf_bytes + ((uint64_t)r << (q + 1))) |
                    (bad ? kRowInvalid : 0u);
            dmeta[r] = m;
            m.base = meta_bytes + 4 * base;
            m.lut = bad ? kRowInvalid : 0u;
            emeta[r] = m;
        }
        if (!bad) {
            // first[b]: the slot holding the bucket's lowest cumulative value
            // b * width, i.e. the last k with start(k) <= b * width (slot k
            // covers [start(k), start(k+1))); one thread per bucket, binary
            // search over the staged row
            for (uint32_t b = tid; b < (1u << q); b += kPrepThreads) {
                const int32_t c = (int32_t)(b * width);
                uint32_t lo = 0, hi = len - 1;   // start(lo) <= c < start(hi)
                while (hi - lo > 1) {
                    const uint32_t mid = (lo + hi) >> 1;
                    if (s_val[mid] <= c)
                        lo = mid;
                    else
                        hi = mid;
                }
                first[((uint64_t)r << q) + b] = (uint16_t)lo;
            }
        }
        __syncthreads();   // s_val is reused by the next row
    }
}

hipError_t launch_prep(const PrepArgs &a, hipStream_t s)
{
    int blocks = a.num_tables < 256 ? a.num_tables : 256;
    hipLaunchKernelGGL(prep_kernel, dim3(blocks), dim3(kPrepThreads), 0, s, a);
    return hipGetLastError();
}

}  // namespace rans
