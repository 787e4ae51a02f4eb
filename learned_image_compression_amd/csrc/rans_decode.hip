// rans_decode.hip -- lane decoder: one rANS64 state per wavefront lane,
// symbols read first to last, the symbol of each step found through the
// LDS bucket lookup (one 8-byte read in the common case) with a bounded
// binary search over the LDS row as fallback.
//
// Decoding rules (the inverse of the puts in rans_encode.hip; decode reads
// the lane's words in order):
//   cum = x mod 2^16; slot s with cdf[s] <= cum < cdf[s+1];
//   x = f * (x >> 16) + cum - cdf[s]; if x < 2^31: x = (x << 32) | next word
//   escape slot -> 4-bit gets: count nb (15 = continue), then nb raw groups,
//   least significant first; odd raw -> -(raw>>1)-1, even -> (raw>>1)+mv
// (kompressor BENCHMARKS.md section 4 names the lookup as the decoder's cost:
// CompressAI scans the row linearly, kompressor binary-searches it; torch_ans
// "Usage" describes the inverse-CDF table keyed by the low state bits.)
// A lane must end at x = 2^31 with all of its words consumed, otherwise the
// call reports RANS_E_CORRUPT; reads never leave the lane's header extent.
#include "rans_internal.hpp"

namespace rans {

namespace {

__device__ inline void record_error(WsHeader *hdr, int code)
{
    atomicCAS(&hdr->err, 0, code);
}

struct WordReader {
    const uint32_t *w;
    uint32_t pos, count;
    uint32_t next;      // w[pos] prefetched (0 past the end)

    __device__ inline bool refill(uint64_t &x)
    {
        if (x < kStateLow) {
            if (pos >= count)
                return false;
            x = (x << 32) | next;
            ++pos;
            next = pos < count ? w[pos] : 0u;
        }
        return true;
    }
};

template <int TPB>
__global__ __launch_bounds__(TPB) void decode_kernel(DecodeArgs a)
{
    extern __shared__ __align__(16) uint8_t lds[];
    __shared__ int s_last;

    WsHeader *hdr = reinterpret_cast<WsHeader *>(a.ws);
    const uint8_t *tab = a.ws + ws_tables_offset();
    const uint32_t tid = threadIdx.x;
    const uint32_t L = a.lanes;

    int herr = 0;
    if (hdr->magic != kMagic || hdr->num_tables != (uint32_t)a.num_tables)
        herr = RANS_E_ARG;
    else if (!hdr->dec_ok)
        herr = RANS_E_TABLE_SIZE;
    const uint32_t K = (uint32_t)a.num_tables;
    const uint32_t nbytes = herr ? 0u : hdr->dec_bytes;
    const uint32_t q = hdr->lut_q;
    {
        const uint4 *src = reinterpret_cast<const uint4 *>(tab);
        uint4 *dst = reinterpret_cast<uint4 *>(lds);
        for (uint32_t i = tid; i < nbytes / 16; i += TPB)
            dst[i] = src[i];
    }
    __syncthreads();
    const RowMeta *meta = reinterpret_cast<const RowMeta *>(lds);
    const uint32_t meta_bytes = (uint32_t)align_up(16ull * K, 16);
    const uint16_t *cdf16 = reinterpret_cast<const uint16_t *>(lds + meta_bytes);
    const uint64_t *lut = reinterpret_cast<const uint64_t *>(
        lds + meta_bytes + align_up(2ull * hdr->total_len, 16));
    int bad = 0;
    if (!herr)
        for (uint32_t r = tid; r < K; r += TPB)
            bad |= (meta[r].mv & kRowInvalid) ? 1 : 0;
    bad = __syncthreads_or(bad);
    if (!herr && bad)
        herr = RANS_E_TABLE;
    if (herr && blockIdx.x == 0 && tid == 0)
        record_error(hdr, herr);

    const uint32_t j = blockIdx.x * TPB + tid;
    if (!herr && j < L) {
        int lerr = 0;
        const uint64_t beg_w = j ? a.stream[j] : 0u;
        const uint64_t end_w = a.stream[1 + j];
        if (a.stream[0] != L || end_w < beg_w + 2 || 1ull + L + end_w > a.capacity) {
            lerr = RANS_E_CORRUPT;
        } else {
            WordReader rd;
            rd.w = a.stream + 1 + L + beg_w;
            rd.count = (uint32_t)(end_w - beg_w);
            uint64_t x = (uint64_t)rd.w[0] | ((uint64_t)rd.w[1] << 32);
            rd.pos = 2;
            rd.next = rd.count > 2 ? rd.w[2] : 0u;
            const uint64_t b = lane_begin(a.n, L, j);
            const uint64_t e = lane_begin(a.n, L, j + 1);
            const uint32_t shift = kPrecision - q;
            for (uint64_t i = b; i < e; ++i) {
                const int32_t r = a.indexes[i];
                if ((uint32_t)r >= K) {
                    lerr = RANS_E_INDEX;
                    break;
                }
                const RowMeta m = meta[r];
                const uint32_t cum = (uint32_t)x & (kTotal - 1);
                const uint64_t ent = lut[m.lut_base + (cum >> shift)];
                const uint32_t s0 = (uint32_t)ent & 0xFFFFu;
                const uint32_t s1 = (uint32_t)(ent >> 16) & 0xFFFFu;
                const uint32_t e1 = (uint32_t)(ent >> 32) & 0xFFFFu;
                uint32_t slot, start, f;
                if (cum >= s0 && cum <= e1) {
                    const bool second = cum >= s1;
                    slot = (uint32_t)(ent >> 48) + (second ? 1u : 0u);
                    start = second ? s1 : s0;
                    f = second ? e1 + 1 - s1 : s1 - s0;
                } else {
                    // value(k) <= cum < value(hi) with value(mv + 1) = 65536
                    const uint16_t *row = cdf16 + m.cdf_base;
                    uint32_t lo = 0, hi = m.mv + 1;
                    while (hi - lo > 1) {
                        const uint32_t mid = (lo + hi) >> 1;
                        if ((uint32_t)row[mid] <= cum)
                            lo = mid;
                        else
                            hi = mid;
                    }
                    slot = lo;
                    start = row[lo];
                    const uint32_t nxt = (lo == m.mv) ? kTotal : (uint32_t)row[lo + 1];
                    f = nxt - start;
                }
                x = (uint64_t)f * (x >> kPrecision) + (cum - start);
                if (!rd.refill(x)) {
                    lerr = RANS_E_CORRUPT;
                    break;
                }
                int64_t value = slot;
                if (slot == m.mv) {
                    uint32_t t = (uint32_t)x & 15u;
                    x >>= kBypassBits;
                    bool ok = rd.refill(x);
                    uint32_t nb = t;
                    while (ok && t == 15u && nb <= 8u) {
                        t = (uint32_t)x & 15u;
                        x >>= kBypassBits;
                        ok = rd.refill(x);
                        nb += t;
                    }
                    uint64_t raw = 0;
                    if (ok && nb <= 8u) {
                        for (uint32_t g = 0; g < nb && ok; ++g) {
                            raw |= (uint64_t)((uint32_t)x & 15u) << (kBypassBits * g);
                            x >>= kBypassBits;
                            ok = rd.refill(x);
                        }
                    }
                    if (!ok || nb > 8u || raw >= (1ull << 31)) {
                        lerr = RANS_E_CORRUPT;
                        break;
                    }
                    value = (raw & 1) ? -(int64_t)(raw >> 1) - 1 : (int64_t)(raw >> 1) + m.mv;
                }
                const int64_t sym = value + m.offset;
                if (sym < INT32_MIN || sym > INT32_MAX) {
                    lerr = RANS_E_CORRUPT;
                    break;
                }
                a.symbols[i] = (int32_t)sym;
            }
            if (!lerr && (x != kStateLow || rd.pos != rd.count))
                lerr = RANS_E_CORRUPT;
        }
        if (lerr)
            record_error(hdr, lerr);
    }

    // ---- completion: the last block publishes status and cleans up -------------
    __syncthreads();
    if (tid == 0) {
        __threadfence();
        const uint32_t old = atomicAdd(&hdr->done, 1u);
        s_last = (old == gridDim.x - 1) ? 1 : 0;
    }
    __syncthreads();
    if (s_last && tid == 0) {
        __threadfence();
        *a.status = hdr->err;
        hdr->err = 0;
        hdr->done = 0;
        __threadfence();
    }
}

template <int TPB>
hipError_t launch_decode_t(const DecodeArgs &a, hipStream_t s)
{
    static const hipError_t attr = hipFuncSetAttribute(
        reinterpret_cast<const void *>(&decode_kernel<TPB>),
        hipFuncAttributeMaxDynamicSharedMemorySize, (int)kTableBudget);
    if (attr != hipSuccess)
        return attr;
    const uint32_t blocks = (uint32_t)((a.lanes + TPB - 1) / TPB);
    hipLaunchKernelGGL(decode_kernel<TPB>, dim3(blocks), dim3(TPB), kTableBudget, s, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_decode(const DecodeArgs &a, hipStream_t s)
{
    const uint32_t t = coding_block_threads(a.lanes);
    if (t <= 256)
        return launch_decode_t<256>(a, s);
    if (t <= 512)
        return launch_decode_t<512>(a, s);
    return launch_decode_t<1024>(a, s);
}

}  // namespace rans
