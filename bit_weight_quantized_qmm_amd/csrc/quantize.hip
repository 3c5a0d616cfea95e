// quantize.hip -- fp16 weights W [K][N] -> k-bit codes [K][N], s and z [N][K/G].
//
// BitLLM Sec. 2.2, eq. (1): q = clip(round(w / s) + z, qmin, qmax) with a
// floating-point scale s > 0 and an integer zero-point z.  Per (column, group)
// the scale and zero-point come from the group's range with zero kept
// representable (min-max affine mapping, unsigned codes, ties to even):
//   lo = min(0, min w),  hi = max(0, max w)
//   s  = fp16((hi - lo) / (2^k - 1)),  1 if that is 0,  65504 if it overflows
//   z  = clamp(round(-lo / s), 0, 2^k - 1),  q = clamp(round(w / s) + z, 0, 2^k - 1)
// The quotients are fp64, so each rounding decision is the one the exact
// quotient gives (fp16 operands never produce a false tie in fp64).  The codes
// feed qmm_pack.
//
// One thread per (column, group): the G rows of a column are read down the
// row-major matrix, consecutive threads on consecutive columns, twice (range,
// then codes; the second pass hits the cache).
#include "launch.hpp"
#include "qmm_device.hpp"

namespace qmm {

// Nearest fp16 to x >= 0, ties to even, in one rounding: x goes to fp32 with
// round-to-odd (the RNE result, stepped toward zero when it rounded up, with
// its last bit set when inexact), which keeps the information the fp16
// rounding needs; then v_cvt_f16_f32 rounds once.
__device__ __forceinline__ _Float16 fp16_of_double(double x)
{
    float f = (float)x;
    if ((double)f != x) {
        uint32_t b = __builtin_bit_cast(uint32_t, f);
        if ((double)f > x) b -= 1u;   // x > 0: the value below x
        f = __builtin_bit_cast(float, b | 1u);
    }
    return (_Float16)f;
}

template <int BITS>
__global__ __launch_bounds__(256) void quantize_kernel(const uint16_t *__restrict__ W, uint8_t *__restrict__ codes,
                                                       uint16_t *__restrict__ s, uint16_t *__restrict__ z, int K, int N,
                                                       int G)
{
    const int n = blockIdx.x * 256 + threadIdx.x;
    if (n >= N) return;   // no barrier in this kernel
    const int g = blockIdx.y, ng = K / G;
    constexpr double QMAX = (double)((1 << BITS) - 1);
    const size_t base = (size_t)g * G * N + n;

    float lo = 0.f, hi = 0.f;
    for (int r = 0; r < G; ++r) {
        const float w = (float)as_half(W[base + (size_t)r * N]);
        lo = fminf(lo, w);
        hi = fmaxf(hi, w);
    }
    _Float16 sh = fp16_of_double(((double)hi - (double)lo) / QMAX);
    if (sh == (_Float16)0.0f) sh = (_Float16)1.0f;
    if (__builtin_isinf((float)sh)) sh = (_Float16)65504.0f;
    const double sg = (double)sh;
    const double zg = fmin(fmax(__builtin_rint(-(double)lo / sg), 0.0), QMAX);
    for (int r = 0; r < G; ++r) {
        const double w = (double)as_half(W[base + (size_t)r * N]);
        codes[base + (size_t)r * N] = (uint8_t)fmin(fmax(__builtin_rint(w / sg) + zg, 0.0), QMAX);
    }
    s[(size_t)n * ng + g] = as_u16(sh);
    z[(size_t)n * ng + g] = as_u16((_Float16)zg);
}

hipError_t launch_quantize(const uint16_t *W, uint8_t *codes, uint16_t *s, uint16_t *z, int K, int N, int bits, int G,
                           hipStream_t st)
{
    const dim3 block(256), grid((unsigned)((N + 255) / 256), (unsigned)(K / G));
#define QMM_Q(B) hipLaunchKernelGGL(quantize_kernel<B>, grid, block, 0, st, W, codes, s, z, K, N, G)
    switch (bits) {
        case 1: QMM_Q(1); break;
        case 2: QMM_Q(2); break;
        case 3: QMM_Q(3); break;
        case 4: QMM_Q(4); break;
        case 5: QMM_Q(5); break;
        case 6: QMM_Q(6); break;
        case 7: QMM_Q(7); break;
        case 8: QMM_Q(8); break;
        default: return hipErrorInvalidValue;
    }
#undef QMM_Q
    return hipGetLastError();
}

}  // namespace qmm
