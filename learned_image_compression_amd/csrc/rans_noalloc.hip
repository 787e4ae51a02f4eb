// rans_noalloc.hip -- the encode entry point for callers that cannot allocate
// device memory (code under stream capture, tight serving loops, harnesses
// that forbid hipMalloc).  It is rans_encode_with_indexes with the workspace
// taken from a fixed device array of this library instead of the caller.
//
// The array is a file-scope __device__ object: every GPU the library runs on
// holds its own copy at its own address from module load until the process
// ends.  In host code its name is only a host-side stand-in, so the device
// address is looked up once per device with hipGetSymbolAddress (with that
// device current) and that pointer is what the kernels receive.  The array
// starts with the workspace header and the look-back flags, which the coding
// kernels expect zero before a call and leave zero after it; a fill kernel
// clears that prefix once per device, on the first call's stream, before any
// coding kernel touches it.  Every call on one GPU uses
// the same array, so calls that overlap in time on one GPU race; calls must
// be ordered (one stream, or synchronised streams).
#include <mutex>

#include "rans_internal.hpp"

namespace {

constexpr uint64_t kNoAllocBytes = 64ull << 20;
constexpr int kMaxDevices = 64;

static __device__ __align__(256) uint8_t scratch[kNoAllocBytes];

struct DeviceScratch {
    std::once_flag once;
    void *ptr = nullptr;
    hipError_t err = hipSuccess;
    bool cleared = false;
};
DeviceScratch g_scratch[kMaxDevices];
std::mutex g_clear_mutex;

__global__ void zero_words_kernel(uint4 *p, uint64_t n16)
{
    const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
    for (uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += stride)
        p[i] = make_uint4(0u, 0u, 0u, 0u);
}

// The device address of `scratch` on the current device, looked up once.
int scratch_for_current_device(void **out, hipStream_t s)
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
        return RANS_E_HIP;
    DeviceScratch &d = g_scratch[dev];
    std::call_once(d.once, [&d]() {
        void *p = nullptr;
        d.err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        d.ptr = d.err == hipSuccess ? p : nullptr;
    });
    if (d.err != hipSuccess || !d.ptr)
        return RANS_E_HIP;
    {
        // the zeroed prefix: the header and the look-back flags
        std::lock_guard<std::mutex> lock(g_clear_mutex);
        if (!d.cleared) {
            const uint64_t n16 = rans::ws_dec_offset() / 16;
            hipLaunchKernelGGL(zero_words_kernel, dim3(256), dim3(256), 0, s,
                               static_cast<uint4 *>(d.ptr), n16);
            if (hipGetLastError() != hipSuccess)
                return RANS_E_HIP;
            d.cleared = true;
        }
    }
    *out = d.ptr;
    return RANS_OK;
}

}  // namespace

extern "C" int rans_encode_noalloc(const int32_t *symbols, const int32_t *indexes, uint64_t n,
                                   const int32_t *cdf, const int32_t *cdf_lengths,
                                   const int32_t *offsets, int32_t num_tables, int32_t cdf_stride,
                                   uint32_t num_lanes, uint32_t *stream,
                                   uint64_t stream_capacity_words, uint64_t *stream_words,
                                   int32_t *status, hipStream_t hstream)
{
    if (num_lanes == 0 || num_lanes > RANS_MAX_LANES || n > RANS_MAX_SYMBOLS)
        return RANS_E_ARG;
    if (rans_workspace_bytes(n, num_lanes, num_tables, cdf_stride) > kNoAllocBytes)
        return RANS_E_WORKSPACE;
    void *ws = nullptr;
    const int rc = scratch_for_current_device(&ws, hstream);
    if (rc)
        return rc;
    return rans_encode_with_indexes(symbols, indexes, n, cdf, cdf_lengths, offsets, num_tables,
                                    cdf_stride, num_lanes, stream, stream_capacity_words,
                                    stream_words, status, ws, kNoAllocBytes, hstream);
}
