// quantize.hip -- fp16 weights W [K][N] -> k-bit codes [K][N], s and z [N][K/G].
//
// BitLLM Sec. 2.2, eq. (1): q = clip(round(w / s) + z, qmin, qmax) with a
// floating-point scale s > 0 and an integer zero-point z.  Per (column, group)
// the scale and zero-point come from the group's range with zero kept
// representable (min-max affine mapping, unsigned codes, ties to even):
//   lo = min(0, min w),  hi = max(0, max w)
//   s  = fp16((hi - lo) / (2^k - 1)),  1 if that is 0,  65504 if it overflows
//   z  = clamp(round(-lo / s), 0, 2^k - 1),  q = clamp(round(w / s) + z, 0, 2^k - 1)
// Every code and zero-point is the one the exact quotient gives
// (round_quotient rounds exactly wherever the result can change one).  The
// codes feed qmm_pack.
//
// Two kernels.  Groups of at most 256 rows (quantize_rows_kernel): one pass
// over W, each lane holding G / 16 rows in registers.  Larger groups
// (quantize_kernel): a wave covers 16 column slots of VEC adjacent columns
// (8-byte loads when VEC = 4: 128 contiguous bytes of a row per 16 lanes) and
// splits a group's G rows into 4 parts, one per 16-lane row of the wave; the
// part ranges are combined with two lane shuffles, and each lane reads its
// rows twice: range, then codes.
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

// round(w / s), ties to even, for fp16 values w and s > 0 (inv = fp32 1 / s,
// half = s / 2), as far as a code can tell: t = rint(w * inv) is already the
// answer except at an exact tie, wherever |w / s| <= 256.5 (off a tie,
// w / s lies at least about 2^-13 from a half-integer there, far more than
// the fp32 product's error); at a tie the residual w - t s from one fma is
// exactly +-s / 2, and the answer is the even one of t and t + sign(r),
// 2 rint(t / 2 + sign(r) / 4) (no integer test of t).  Beyond 256.5 the
// result can be off but stays past +-255 on the quotient's side, so every
// code, clamped to 0..2^k - 1 after adding z <= 255, is the same.  Checked
// for every finite fp16 w and every positive fp16 s on the host.
__device__ __forceinline__ float round_quotient(float w, float s, float inv, float half)
{
    const float t = __builtin_rintf(w * inv);
    const float r = __builtin_fmaf(-t, s, w);
    const float even = 2.0f * __builtin_rintf(__builtin_fmaf(t, 0.5f, __builtin_copysignf(0.25f, r)));
    return __builtin_fabsf(r) == half ? even : t;   // t itself off a tie (keeps a -0)
}

template <int BITS, int VEC>
__global__ __launch_bounds__(256) void quantize_kernel(const uint16_t *__restrict__ W, uint8_t *__restrict__ codes,
                                                       uint16_t *__restrict__ s, uint16_t *__restrict__ z, int K, int N,
                                                       int G)
{
    const int lane = threadIdx.x & 63, c = lane & 15, part = lane >> 4;
    const int n0 = ((blockIdx.x * 4 + (int)(threadIdx.x >> 6)) * 16 + c) * VEC;
    const bool live = n0 < N;   // every lane stays for the shuffles
    const int g = blockIdx.y, ng = K / G, rows = G >> 2;
    constexpr float QMAX = (float)((1 << BITS) - 1);
    const size_t base = ((size_t)g * G + (size_t)part * rows) * N + n0;

    auto load = [&](int r, float (&w)[VEC]) {
        const size_t at = base + (size_t)r * N;
        if constexpr (VEC == 4) {
            const uint2 v = *reinterpret_cast<const uint2 *>(W + at);
            const half2_t a = as_half2(v.x), b = as_half2(v.y);
            w[0] = (float)a[0];
            w[1] = (float)a[1];
            w[2] = (float)b[0];
            w[3] = (float)b[1];
        } else {
            w[0] = (float)as_half(W[at]);
        }
    };

    float lo[VEC], hi[VEC];
#pragma unroll
    for (int v = 0; v < VEC; ++v) lo[v] = hi[v] = 0.f;
    if (live) {
#pragma unroll 8
        for (int r = 0; r < rows; ++r) {
            float w[VEC];
            load(r, w);
#pragma unroll
            for (int v = 0; v < VEC; ++v) {
                lo[v] = fminf(lo[v], w[v]);
                hi[v] = fmaxf(hi[v], w[v]);
            }
        }
    }
    float sg[VEC], inv[VEC], half[VEC], zg[VEC];
#pragma unroll
    for (int v = 0; v < VEC; ++v) {
        // the four row parts of a column sit 16 lanes apart
        lo[v] = fminf(lo[v], __shfl_xor(lo[v], 16));
        lo[v] = fminf(lo[v], __shfl_xor(lo[v], 32));
        hi[v] = fmaxf(hi[v], __shfl_xor(hi[v], 16));
        hi[v] = fmaxf(hi[v], __shfl_xor(hi[v], 32));
        _Float16 sh = fp16_of_double(((double)hi[v] - (double)lo[v]) / (double)QMAX);
        if (sh == (_Float16)0.0f) sh = (_Float16)1.0f;
        if (__builtin_isinf((float)sh)) sh = (_Float16)65504.0f;
        sg[v] = (float)sh;
        inv[v] = 1.0f / sg[v];
        half[v] = 0.5f * sg[v];
        zg[v] = fminf(fmaxf(round_quotient(-lo[v], sg[v], inv[v], half[v]), 0.f), QMAX);
        if (part == 0 && n0 + v < N) {
            s[(size_t)(n0 + v) * ng + g] = as_u16(sh);
            z[(size_t)(n0 + v) * ng + g] = as_u16((_Float16)zg[v]);
        }
    }
    if (!live) return;
#pragma unroll 8
    for (int r = 0; r < rows; ++r) {
        float w[VEC];
        load(r, w);
        uint32_t packed = 0;
#pragma unroll
        for (int v = 0; v < VEC; ++v) {
            const float q = fminf(fmaxf(round_quotient(w[v], sg[v], inv[v], half[v]) + zg[v], 0.f), QMAX);
            packed = __builtin_amdgcn_cvt_pk_u8_f32(q, v, packed);   // byte v of the word, one op
        }
        const size_t at = base + (size_t)r * N;
        if constexpr (VEC == 4)
            *reinterpret_cast<uint32_t *>(codes + at) = packed;
        else
            codes[at] = (uint8_t)packed;
    }
}

// One pass over W for groups of at most 256 rows: a workgroup takes 16 column
// slots of VEC adjacent columns and splits the group's rows into 16 parts of
// G / 16 rows, one per 16-lane row of its waves; each lane keeps its rows in
// registers, the parts' ranges meet through lane shuffles and LDS, and the
// codes come from the registers (W is read once: the two-pass kernel above
// reads it twice).
constexpr int QR_MAXR = 16;   // rows per lane: G <= 256
// RPT > 0: G / 16 == RPT known at compile time (G = 64, 128, 256: 4, 8, 16
// rows per lane), so the row loops carry no per-row branches
template <int BITS, int VEC, int RPT = 0>
__global__ __launch_bounds__(256) void quantize_rows_kernel(const uint16_t *__restrict__ W, uint8_t *__restrict__ codes,
                                                            uint16_t *__restrict__ s, uint16_t *__restrict__ z, int K,
                                                            int N, int G)
{
    __shared__ float rlo[4][16][VEC], rhi[4][16][VEC];
    __shared__ float4_t rsc[16][VEC];   // per column slot: s, 1 / s, s / 2, z
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int c = lane & 15, part = tid >> 4;   // part 0..15
    const int n0 = (blockIdx.x * 16 + c) * VEC;
    const bool live = n0 < N;
    const int g = blockIdx.y, ng = K / G, rp = RPT > 0 ? RPT : G >> 4;
    constexpr float QMAX = (float)((1 << BITS) - 1);
    const size_t base = ((size_t)g * G + (size_t)part * rp) * N + n0;

    uint32_t raw[QR_MAXR][VEC == 4 ? 2 : 1];
    float lo[VEC], hi[VEC];
#pragma unroll
    for (int r = 0; r < QR_MAXR; ++r) {
        if (r < rp && live) {   // uniform in r; live per lane
            const size_t at = base + (size_t)r * N;
            if constexpr (VEC == 4) {
                const uint2 u = *reinterpret_cast<const uint2 *>(W + at);
                raw[r][0] = u.x;
                raw[r][1] = u.y;
            } else {
                raw[r][0] = W[at];
            }
        } else {
#pragma unroll
            for (int e = 0; e < (VEC == 4 ? 2 : 1); ++e) raw[r][e] = 0u;
        }
    }
    // the range on fp16 pairs (min and max pick one of their operands, so
    // fp16 and fp32 give the same values): one packed op per two codes, no
    // conversions; a lone column (VEC 1) uses the pair's low half
    constexpr int NP = VEC == 4 ? 2 : 1;
    half2_t lo2[NP], hi2[NP];
#pragma unroll
    for (int e = 0; e < NP; ++e) lo2[e] = hi2[e] = half2_t{(_Float16)0.0f, (_Float16)0.0f};
#pragma unroll
    for (int r = 0; r < QR_MAXR; ++r) {
        if (r < rp) {
#pragma unroll
            for (int e = 0; e < NP; ++e) {
                const half2_t w2 = as_half2(raw[r][e]);
                lo2[e] = __builtin_elementwise_min(lo2[e], w2);
                hi2[e] = __builtin_elementwise_max(hi2[e], w2);
            }
        }
    }
#pragma unroll
    for (int v = 0; v < VEC; ++v) {
        lo[v] = (float)lo2[v >> 1][v & 1];
        hi[v] = (float)hi2[v >> 1][v & 1];
    }
#pragma unroll
    for (int v = 0; v < VEC; ++v) {
        // the wave's four parts of a column sit 16 lanes apart; the four waves meet in LDS
        lo[v] = fminf(lo[v], __shfl_xor(lo[v], 16));
        lo[v] = fminf(lo[v], __shfl_xor(lo[v], 32));
        hi[v] = fmaxf(hi[v], __shfl_xor(hi[v], 16));
        hi[v] = fmaxf(hi[v], __shfl_xor(hi[v], 32));
        if (lane < 16) {
            rlo[wave][c][v] = lo[v];
            rhi[wave][c][v] = hi[v];
        }
    }
    __syncthreads();
    // s and z of column v of the slot (the same values in every part)
    float sg[VEC], inv[VEC], half[VEC], zg[VEC];
    auto col_scale = [&](int v, bool store) __attribute__((always_inline)) {
        lo[v] = fminf(fminf(rlo[0][c][v], rlo[1][c][v]), fminf(rlo[2][c][v], rlo[3][c][v]));
        hi[v] = fmaxf(fmaxf(rhi[0][c][v], rhi[1][c][v]), fmaxf(rhi[2][c][v], rhi[3][c][v]));
        _Float16 sh = fp16_of_double(((double)hi[v] - (double)lo[v]) / (double)QMAX);
        if (sh == (_Float16)0.0f) sh = (_Float16)1.0f;
        if (__builtin_isinf((float)sh)) sh = (_Float16)65504.0f;
        sg[v] = (float)sh;
        inv[v] = 1.0f / sg[v];
        half[v] = 0.5f * sg[v];
        zg[v] = fminf(fmaxf(round_quotient(-lo[v], sg[v], inv[v], half[v]), 0.f), QMAX);
        if (store && n0 + v < N) {
            s[(size_t)(n0 + v) * ng + g] = as_u16(sh);
            z[(size_t)(n0 + v) * ng + g] = as_u16((_Float16)zg[v]);
        }
    };
    if (rp <= 4) {
        // few rows per lane (G <= 64): the part-0 lanes (0..15 of wave 0)
        // work out each column once and hand it to the other parts through
        // LDS (G 64: 46.5 -> 37.6 us on the 7B weight); with more rows per
        // lane the extra barrier costs more than the 15 repeats it saves
        if (part == 0) {
#pragma unroll
            for (int v = 0; v < VEC; ++v) {
                col_scale(v, true);
                rsc[c][v] = float4_t{sg[v], inv[v], half[v], zg[v]};
            }
        }
        __syncthreads();
#pragma unroll
        for (int v = 0; v < VEC; ++v) {
            const float4_t q = rsc[c][v];
            sg[v] = q[0];
            inv[v] = q[1];
            half[v] = q[2];
            zg[v] = q[3];
        }
    } else {
#pragma unroll
        for (int v = 0; v < VEC; ++v) col_scale(v, part == 0);
    }
    if (!live) return;
#pragma unroll
    for (int r = 0; r < QR_MAXR; ++r) {
        if (r < rp) {
            uint32_t packed = 0;
#pragma unroll
            for (int v = 0; v < VEC; ++v) {
                const float w = VEC == 4 ? (float)as_half2(raw[r][v >> 1])[v & 1] : (float)as_half((uint16_t)raw[r][0]);
                const float q = fminf(fmaxf(round_quotient(w, sg[v], inv[v], half[v]) + zg[v], 0.f), QMAX);
                // q is a whole number in 0..255: convert and insert byte v in one op
                packed = __builtin_amdgcn_cvt_pk_u8_f32(q, v, packed);
            }
            const size_t at = base + (size_t)r * N;
            if constexpr (VEC == 4)
                *reinterpret_cast<uint32_t *>(codes + at) = packed;
            else
                codes[at] = (uint8_t)packed;
        }
    }
}

hipError_t launch_quantize(const uint16_t *W, uint8_t *codes, uint16_t *s, uint16_t *z, int K, int N, int bits, int G,
                           hipStream_t st)
{
    // four columns per thread when every row of W and of the codes stays 8- and
    // 4-byte aligned
    const bool vec = N % 4 == 0 && reinterpret_cast<uintptr_t>(W) % 8 == 0 && reinterpret_cast<uintptr_t>(codes) % 4 == 0;
    const bool one_pass = G <= 16 * QR_MAXR;   // G % 32 == 0: 2 .. 16 rows per lane
    const int per_block = one_pass ? (vec ? 64 : 16) : (vec ? 256 : 64);   // 16 or 4 x 16 column slots
    const dim3 block(256), grid((unsigned)((N + per_block - 1) / per_block), (unsigned)(K / G));
#define QMM_Q(B)                                                                                                \
    do {                                                                                                        \
        if (one_pass && vec && G == 128)                                                                        \
            hipLaunchKernelGGL((quantize_rows_kernel<B, 4, 8>), grid, block, 0, st, W, codes, s, z, K, N, G);   \
        else if (one_pass && vec && G == 64)                                                                    \
            hipLaunchKernelGGL((quantize_rows_kernel<B, 4, 4>), grid, block, 0, st, W, codes, s, z, K, N, G);   \
        else if (one_pass && vec && G == 256)                                                                   \
            hipLaunchKernelGGL((quantize_rows_kernel<B, 4, 16>), grid, block, 0, st, W, codes, s, z, K, N, G);  \
        else if (one_pass && vec)                                                                               \
            hipLaunchKernelGGL((quantize_rows_kernel<B, 4>), grid, block, 0, st, W, codes, s, z, K, N, G);      \
        else if (one_pass)                                                                                      \
            hipLaunchKernelGGL((quantize_rows_kernel<B, 1>), grid, block, 0, st, W, codes, s, z, K, N, G);      \
        else if (vec)                                                                                           \
            hipLaunchKernelGGL((quantize_kernel<B, 4>), grid, block, 0, st, W, codes, s, z, K, N, G);           \
        else                                                                                                    \
            hipLaunchKernelGGL((quantize_kernel<B, 1>), grid, block, 0, st, W, codes, s, z, K, N, G);           \
    } while (0)
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
