// pack.hip -- codes [K][N] <-> packed stream Wq [N][K*k/32] on the GPU.
//
// One thread owns one (column n, run r) pair: 32 codes = k dwords.  Threads of
// a wave take consecutive columns, so the strided code reads codes[(32r+i)*N+n]
// are coalesced across the wave.  Signed (two's complement) codes are stored
// offset-binary, q + 2^(k-1): the low k bits with the top one flipped (flip).
#include "launch.hpp"
#include "qmm_device.hpp"

namespace qmm {

template <int BITS>
__global__ __launch_bounds__(256) void pack_kernel(const uint8_t *__restrict__ codes, uint32_t *__restrict__ wq,
                                                   int K, int N, uint32_t flip)
{
    const int R = K >> 5;
    const long long t = (long long)blockIdx.x * blockDim.x + threadIdx.x;
    const int n = (int)(t % N);
    const int r = (int)(t / N);
    if (r >= R) return;
    uint32_t d[BITS];
#pragma unroll
    for (int j = 0; j < BITS; ++j) d[j] = 0;
    const uint8_t *src = codes + (size_t)(32 * r) * N + n;
#pragma unroll
    for (int i = 0; i < 32; ++i) {
        const uint32_t q = (src[(size_t)i * N] ^ flip) & ((1u << BITS) - 1u);
        const int b = i * BITS, j = b >> 5, sh = b & 31;
        d[j] |= q << sh;
        if (sh + BITS > 32) d[j + 1] |= q >> (32 - sh);
    }
    uint32_t *dst = wq + ((size_t)n * R + r) * BITS;
#pragma unroll
    for (int j = 0; j < BITS; ++j) dst[j] = d[j];
}

// Inverse of pack through the same register unpack the product kernels use:
// run -> 16 fp16 pair words -> code = mantissa >> p for every half-slot.
template <int BITS>
__global__ __launch_bounds__(256) void unpack_kernel(const uint32_t *__restrict__ wq, uint8_t *__restrict__ codes,
                                                     int K, int N)
{
    const int R = K >> 5;
    const long long t = (long long)blockIdx.x * blockDim.x + threadIdx.x;
    const int n = (int)(t % N);
    const int r = (int)(t / N);
    if (r >= R) return;
    uint32_t d[BITS];
    const uint32_t *src = wq + ((size_t)n * R + r) * BITS;
#pragma unroll
    for (int j = 0; j < BITS; ++j) d[j] = src[j];
    uint32_t h[16];
    run_to_half2<BITS>(d, h);
    uint8_t *dst = codes + (size_t)(32 * r) * N + n;
#pragma unroll
    for (int sl = 0; sl < 32; ++sl) {
        const uint32_t half_bits = (h[sl >> 1] >> (16 * (sl & 1))) & 0xffffu;
        const uint32_t q = (half_bits & 0x3ffu) >> RunPlan<BITS>::pos[sl];
        dst[(size_t)RunPlan<BITS>::code[sl] * N] = (uint8_t)q;
    }
}

hipError_t launch_pack(const uint8_t *codes, uint32_t *wq, int K, int N, int bits, bool is_signed, hipStream_t st)
{
    const long long total = (long long)(K / 32) * N;
    const dim3 block(256), grid((unsigned)((total + 255) / 256));
    const uint32_t flip = is_signed ? 1u << (bits - 1) : 0u;
    switch (bits) {
#define QMM_CASE(B) case B: hipLaunchKernelGGL(pack_kernel<B>, grid, block, 0, st, codes, wq, K, N, flip); break;
        QMM_CASE(1) QMM_CASE(2) QMM_CASE(3) QMM_CASE(4) QMM_CASE(5) QMM_CASE(6) QMM_CASE(7) QMM_CASE(8)
#undef QMM_CASE
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_unpack(const uint32_t *wq, uint8_t *codes, int K, int N, int bits, hipStream_t st)
{
    const long long total = (long long)(K / 32) * N;
    const dim3 block(256), grid((unsigned)((total + 255) / 256));
    switch (bits) {
#define QMM_CASE(B) case B: hipLaunchKernelGGL(unpack_kernel<B>, grid, block, 0, st, wq, codes, K, N); break;
        QMM_CASE(1) QMM_CASE(2) QMM_CASE(3) QMM_CASE(4) QMM_CASE(5) QMM_CASE(6) QMM_CASE(7) QMM_CASE(8)
#undef QMM_CASE
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace qmm
