// launch.hpp -- internal launchers behind the C ABI (arguments already validated).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qmm {

struct GemvArgs {
    const uint16_t *X;     // fp16 [M][K]
    const uint32_t *wq;    // [N][K*bits/32]
    const uint16_t *s;     // fp16 [N][K/G]
    const uint16_t *z;     // fp16 [N][K/G] or nullptr
    uint16_t *Y;           // fp16 [M][N]
    int M, K, N, bits, G;
};

struct W4A8Args {
    const int8_t *Xq;      // [M][K]
    const uint16_t *sx;    // fp16 [M]
    const uint32_t *wq;    // [N][K*bits/32]
    const uint16_t *s;     // fp16 [N][K/G]
    const uint16_t *z;     // fp16 [N][K/G] or nullptr
    uint16_t *Y;           // fp16 [M][N]
    int32_t *acc;          // int32 [M][K/G][N] or nullptr
    int M, K, N, bits, G;
};

// Grouped M = 1 products (qmm_gemv_grouped): one launch, every problem with
// the same K and G, its own X, weights, scales, zero-points, output, N and
// code width.
constexpr int QMM_GROUP_MAX = 16;
struct GroupProblem {
    const uint16_t *X;     // fp16 [1][K]
    const uint32_t *wq;    // [N][K*bits/32]
    const uint16_t *s;     // fp16 [N][K/G]
    const uint16_t *z;     // fp16 [N][K/G] or nullptr
    uint16_t *Y;           // fp16 [1][N]
    int N, bits;
};
struct GroupArgs {
    GroupProblem p[QMM_GROUP_MAX];
    int wg0[QMM_GROUP_MAX + 1];   // workgroups of problem p: wg0[p] .. wg0[p + 1] - 1 (set by the launcher)
    int count, K, G;
};

hipError_t launch_pack(const uint8_t *codes, uint32_t *wq, int K, int N, int bits, bool is_signed, hipStream_t st);
hipError_t launch_unpack(const uint32_t *wq, uint8_t *codes, int K, int N, int bits, hipStream_t st);
hipError_t launch_gemv(const GemvArgs &a, hipStream_t st);
hipError_t launch_gemm(const GemvArgs &a, hipStream_t st);
hipError_t launch_gemm_fp(const GemvArgs &a, int fmt, hipStream_t st);
hipError_t launch_gemv_grouped(const GroupArgs &a, hipStream_t st);
hipError_t launch_gemv_lut(const GemvArgs &a, hipStream_t st);   // M = 1, 1-bit codes; NotSupported otherwise
hipError_t launch_gemv_fp(const GemvArgs &a, int fmt, hipStream_t st);   // M <= 16; NotSupported otherwise
hipError_t launch_w4a8(const W4A8Args &a, hipStream_t st);
hipError_t launch_probe_read(const void *buf, uint64_t bytes, uint32_t *sink, int grid, hipStream_t st);
hipError_t launch_probe_mfma(float *sink, int iters, int grid, int shape, hipStream_t st);
hipError_t launch_quantize(const uint16_t *W, uint8_t *codes, uint16_t *s, uint16_t *z, int K, int N, int bits, int G,
                           hipStream_t st);

}  // namespace qmm
