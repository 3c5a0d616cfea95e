// probe.hip -- measurement hooks: what this GPU delivers on a plain streaming
// read of HBM and on back-to-back MFMAs with register operands.  They price
// the product kernels against a measured ceiling beside the datasheet one
// (the benchmark protocol on the Tilus verdict page asks for results against
// a clear reference point; these are that point on this machine).  Neither
// hook computes any part of the product.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "launch.hpp"
#include "qmm_device.hpp"

namespace qmm {

// Streaming read: every 16-byte piece of [p, p + n16 * 16) is loaded once
// (non-temporal), U loads in flight per lane, grid-stride over the buffer so
// consecutive lanes read consecutive 16-byte pieces.  The XOR of everything
// read is written only if it equals a constant the data never gives, which
// keeps the loads alive without a store stream.
template <int U>
__global__ __launch_bounds__(256) void probe_read_kernel(const int4_t *__restrict__ p, uint64_t n16,
                                                         uint32_t *__restrict__ sink, uint32_t magic)
{
    const uint64_t stride = (uint64_t)gridDim.x * 256u;
    uint64_t i = (uint64_t)blockIdx.x * 256u + threadIdx.x;
    uint32_t acc = 0;
    for (; i + (U - 1) * stride < n16; i += U * stride) {
        int4_t v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) v[u] = __builtin_nontemporal_load(p + i + u * stride);
#pragma unroll
        for (int u = 0; u < U; ++u) acc ^= (uint32_t)(v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3]);
    }
    for (; i < n16; i += stride) {
        const int4_t v = __builtin_nontemporal_load(p + i);
        acc ^= (uint32_t)(v[0] ^ v[1] ^ v[2] ^ v[3]);
    }
    if (acc == magic) sink[blockIdx.x * 256u + threadIdx.x] = acc;
}

// Back-to-back f16 MFMAs on register operands: NA independent accumulators
// per wave, 8 waves per workgroup (two per SIMD).  SHAPE 0 is
// v_mfma_f32_16x16x32_f16 (16384 flops), SHAPE 1 v_mfma_f32_32x32x16_f16
// (32768 flops).  The accumulators are summed and written only if the sum
// equals a constant it never reaches.
template <int SHAPE>
__global__ __launch_bounds__(512) void probe_mfma_kernel(float *__restrict__ sink, int iters, float magic)
{
    constexpr int NA = SHAPE == 0 ? 8 : 4;
    typedef float float16_t __attribute__((ext_vector_type(16)));
    half8_t a, b;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        a[e] = (_Float16)(float)((threadIdx.x + e) & 7) * (_Float16)0.125f;
        b[e] = (_Float16)(float)((threadIdx.x * 3 + e) & 7) * (_Float16)0.0625f;
    }
    float tot = 0.f;
    if constexpr (SHAPE == 0) {
        float4_t acc[NA];
#pragma unroll
        for (int j = 0; j < NA; ++j) acc[j] = float4_t{0.f, 0.f, 0.f, 0.f};
        for (int it = 0; it < iters; ++it) {
#pragma unroll
            for (int j = 0; j < NA; ++j) acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, acc[j], 0, 0, 0);
        }
#pragma unroll
        for (int j = 0; j < NA; ++j) tot += acc[j][0] + acc[j][1] + acc[j][2] + acc[j][3];
    } else {
        float16_t acc[NA];
#pragma unroll
        for (int j = 0; j < NA; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[j][e] = 0.f;
        for (int it = 0; it < iters; ++it) {
#pragma unroll
            for (int j = 0; j < NA; ++j) acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, acc[j], 0, 0, 0);
        }
#pragma unroll
        for (int j = 0; j < NA; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) tot += acc[j][e];
    }
    if (tot == magic) sink[blockIdx.x * 512u + threadIdx.x] = tot;
}

hipError_t launch_probe_read(const void *buf, uint64_t bytes, uint32_t *sink, int grid, hipStream_t st)
{
    const uint64_t n16 = bytes / 16u;
    hipLaunchKernelGGL(probe_read_kernel<8>, dim3(grid), dim3(256), 0, st, reinterpret_cast<const int4_t *>(buf), n16,
                       sink, 0x9e3779b9u);
    return hipGetLastError();
}

hipError_t launch_probe_mfma(float *sink, int iters, int grid, int shape, hipStream_t st)
{
    if (shape == 0)
        hipLaunchKernelGGL(probe_mfma_kernel<0>, dim3(grid), dim3(512), 0, st, sink, iters, -1.2345e30f);
    else
        hipLaunchKernelGGL(probe_mfma_kernel<1>, dim3(grid), dim3(512), 0, st, sink, iters, -1.2345e30f);
    return hipGetLastError();
}

}  // namespace qmm
