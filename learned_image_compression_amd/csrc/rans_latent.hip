// rans_latent.hip -- the mean-scale front end around the coder: latent ->
// (symbols, table indexes) before encoding, symbols -> latent after decoding.
//
// The codec computes the table index of every y position on the GPU
// (build_indexes) and hands symbols and indexes to the coder as int32 tensors
// (kompressor BENCHMARKS.md, sections 3 and 4).  The symbol and index rules
// are in rans_frontend.hpp; dequantisation is y_hat = (float)symbol + mean in
// single precision.
//
// Both kernels stream HBM: 12 bytes in and 8 out per position for the front
// end, 8 in and 4 out for dequantisation.  When every array is 16-byte
// aligned, a thread takes a group of four positions (front end: its four
// index searches already keep it busy) or eight (dequantisation: two 16-byte
// loads per array in flight), all loads issued before any use.  The scale table is
// staged in LDS.
#include "rans_frontend.hpp"

#pragma clang fp contract(off)

namespace rans {
namespace {

constexpr int kLatThreads = 256;
// one group of positions per thread: a grid-stride loop over a capped grid
// kept fewer bytes in flight and ran about 10% slower at 50M positions
constexpr uint32_t kLatMaxBlocks = 1u << 30;

template <int VEC>
__global__ __launch_bounds__(kLatThreads) void latent_symbols_kernel(LatentArgs a)
{
    __shared__ float table[RANS_MAX_TABLES];
    __shared__ uint32_t flag;
    if (threadIdx.x == 0)
        flag = 0u;
    const ScaleTable st = stage_scale_table<kLatThreads>(a.table, a.K, table, &flag);
    const uint64_t groups = (a.n + VEC - 1) / VEC;
    const uint64_t stride = (uint64_t)gridDim.x * kLatThreads;
    for (uint64_t g = (uint64_t)blockIdx.x * kLatThreads + threadIdx.x; g < groups; g += stride) {
        const uint64_t i0 = g * VEC;
        if (VEC >= 4 && i0 + VEC <= a.n) {
            constexpr int U = VEC >= 4 ? VEC / 4 : 1;
            float4 y[U], m[U], s[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                y[u] = *reinterpret_cast<const float4 *>(a.y + i0 + 4 * u);
                m[u] = *reinterpret_cast<const float4 *>(a.means + i0 + 4 * u);
                s[u] = *reinterpret_cast<const float4 *>(a.scales + i0 + 4 * u);
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                int4 q, ix;
                q.x = saturate_round(y[u].x - m[u].x);
                q.y = saturate_round(y[u].y - m[u].y);
                q.z = saturate_round(y[u].z - m[u].z);
                q.w = saturate_round(y[u].w - m[u].w);
                ix.x = st.index(s[u].x);
                ix.y = st.index(s[u].y);
                ix.z = st.index(s[u].z);
                ix.w = st.index(s[u].w);
                *reinterpret_cast<int4 *>(a.symbols + i0 + 4 * u) = q;
                *reinterpret_cast<int4 *>(a.indexes + i0 + 4 * u) = ix;
            }
        } else {
            for (uint64_t i = i0; i < min(i0 + VEC, a.n); ++i) {
                a.symbols[i] = saturate_round(a.y[i] - a.means[i]);
                a.indexes[i] = st.index(a.scales[i]);
            }
        }
    }
}

template <int VEC>
__global__ __launch_bounds__(kLatThreads) void dequantize_kernel(DequantArgs a)
{
    const uint64_t groups = (a.n + VEC - 1) / VEC;
    const uint64_t stride = (uint64_t)gridDim.x * kLatThreads;
    for (uint64_t g = (uint64_t)blockIdx.x * kLatThreads + threadIdx.x; g < groups; g += stride) {
        const uint64_t i0 = g * VEC;
        if (VEC >= 4 && i0 + VEC <= a.n) {
            constexpr int U = VEC >= 4 ? VEC / 4 : 1;
            int4 q[U];
            float4 m[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                q[u] = *reinterpret_cast<const int4 *>(a.symbols + i0 + 4 * u);
                m[u] = *reinterpret_cast<const float4 *>(a.means + i0 + 4 * u);
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                float4 o;
                o.x = (float)q[u].x + m[u].x;
                o.y = (float)q[u].y + m[u].y;
                o.z = (float)q[u].z + m[u].z;
                o.w = (float)q[u].w + m[u].w;
                *reinterpret_cast<float4 *>(a.y_hat + i0 + 4 * u) = o;
            }
        } else {
            for (uint64_t i = i0; i < min(i0 + VEC, a.n); ++i)
                a.y_hat[i] = (float)a.symbols[i] + a.means[i];
        }
    }
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

uint32_t grid_for(uint64_t groups)
{
    const uint64_t b = (groups + kLatThreads - 1) / kLatThreads;
    return (uint32_t)(b < 1 ? 1 : (b > kLatMaxBlocks ? kLatMaxBlocks : b));
}

}  // namespace

hipError_t launch_latent_symbols(const LatentArgs &a, hipStream_t s)
{
    if (aligned16(a.y) && aligned16(a.means) && aligned16(a.scales) && aligned16(a.symbols) &&
        aligned16(a.indexes))
        hipLaunchKernelGGL(latent_symbols_kernel<4>, dim3(grid_for((a.n + 3) / 4)),
                           dim3(kLatThreads), 0, s, a);
    else
        hipLaunchKernelGGL(latent_symbols_kernel<1>, dim3(grid_for(a.n)), dim3(kLatThreads), 0,
                           s, a);
    return hipGetLastError();
}

hipError_t launch_dequantize(const DequantArgs &a, hipStream_t s)
{
    if (aligned16(a.symbols) && aligned16(a.means) && aligned16(a.y_hat))
        hipLaunchKernelGGL(dequantize_kernel<8>, dim3(grid_for((a.n + 7) / 8)),
                           dim3(kLatThreads), 0, s, a);
    else
        hipLaunchKernelGGL(dequantize_kernel<1>, dim3(grid_for(a.n)), dim3(kLatThreads), 0, s,
                           a);
    return hipGetLastError();
}

}  // namespace rans
