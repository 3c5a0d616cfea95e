// gemv.hip -- decode-shaped products Y[M,N] = X[M,K] . dequant(Wq), M <= 16.
//
// Dequantisation follows BitLLM (Sec. 2.2, eq. (5)): w = (q - z) * s with one
// s, z per group of G rows along K.  Codes are unpacked in registers from
// dword-aligned runs (qmm_device.hpp) into fp16 patterns 1024 + q * 2^p; the
// matching activation is pre-scaled by 2^-p, so a dot product with the pattern
// gives sum x*q plus a code-independent bias that is removed once per run.
#include "launch.hpp"
#include "qmm_device.hpp"

namespace qmm {

// ---------------------------------------------------------------------------
// The X side of one run: 32 activations (natural order, two per dword) ->
// 16 half2 in the half-slot order of RunPlan<BITS>, slot s scaled by 2^-pos[s].
// ---------------------------------------------------------------------------
template <int BITS>
__device__ __forceinline__ void x_slots(const uint32_t (&xr)[16], half2_t (&xs)[16])
{
    using P = RunPlan<BITS>;
    _Float16 x[32];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const half2_t p = as_half2(xr[i]);
        x[2 * i] = p[0];
        x[2 * i + 1] = p[1];
    }
#pragma unroll
    for (int j = 0; j < 16; ++j) {
        half2_t v;
        v[0] = x[P::code[2 * j]];
        v[1] = x[P::code[2 * j + 1]];
        if (P::pos[2 * j] | P::pos[2 * j + 1]) {
            half2_t sc;
            sc[0] = (_Float16)pow2neg(P::pos[2 * j]);
            sc[1] = (_Float16)pow2neg(P::pos[2 * j + 1]);
            v = v * sc;
        }
        xs[j] = v;
    }
}

// Per-slot constant of the fp16 code pattern: (1024 + zc * 2^pos) for a fixed
// zero-point zc (exact in fp16: an integer below 2048).
template <int BITS>
__device__ __forceinline__ half2_t slot_bias(int j, float zc)
{
    using P = RunPlan<BITS>;
    half2_t b;
    b[0] = (_Float16)(1024.0f + zc * (float)(1u << P::pos[2 * j]));
    b[1] = (_Float16)(1024.0f + zc * (float)(1u << P::pos[2 * j + 1]));
    return b;
}

template <int BITS>
__device__ __forceinline__ half2_t slot_pow2(int j)
{
    using P = RunPlan<BITS>;
    half2_t b;
    b[0] = (_Float16)(float)(1u << P::pos[2 * j]);
    b[1] = (_Float16)(float)(1u << P::pos[2 * j + 1]);
    return b;
}

constexpr uint32_t OOB = 0x80000000u;   // a buffer offset past every resource we build

// ---------------------------------------------------------------------------
// M = 1: split-K across the 64 lanes of a wave.  A wave owns CPW consecutive
// columns; lane l owns runs l, l+64, ... (RPL of them) of every column, keeps
// the matching activations in VGPRs, and issues all its weight loads before
// any arithmetic.  Per run: 16 v_dot2_f32_f16 give a = sum x'(1024 + q 2^p);
// y += s_g * (a - bias) with bias = sum x'(1024 + z 2^p) (precomputed per lane
// for a fixed z, or c1 + z * c2 for per-group z).  A wave reduction finishes
// each column.
// ---------------------------------------------------------------------------
template <int BITS, int RPL, int CPW, bool PGZ>
__global__ __launch_bounds__(256) void gemv_m1_kernel(const uint16_t *__restrict__ X, const uint32_t *__restrict__ wq,
                                                      const uint16_t *__restrict__ s, const uint16_t *__restrict__ z,
                                                      uint16_t *__restrict__ Y, int K, int N, int G)
{
    const int lane = threadIdx.x & 63;
    const int wave = (int)((blockIdx.x * blockDim.x + threadIdx.x) >> 6);
    const int n0 = wave * CPW;
    if (n0 >= N) return;
    const int R = K >> 5, ng = K / G;
    const uint32_t run_bytes = 4u * BITS;
    const uint32_t col_bytes = (uint32_t)R * run_bytes;
    const int ncols = min(CPW, N - n0);

    // 1. every weight load of this wave in flight first (OOB lanes read zeros).
    const __amdgpu_buffer_rsrc_t wr = make_rsrc(wq + (size_t)n0 * R * BITS, (uint32_t)ncols * col_bytes);
    uint32_t d[CPW][RPL][BITS];
#pragma unroll
    for (int c = 0; c < CPW; ++c)
#pragma unroll
        for (int j = 0; j < RPL; ++j) {
            const int r = lane + 64 * j;
            const uint32_t off = (r < R) ? (uint32_t)c * col_bytes + (uint32_t)r * run_bytes : OOB;
            load_dwords<LOAD_STREAM>(wr, off, d[c][j], BITS);
        }

    // 2. scale (and zero-point) of each (column, run).
    const __amdgpu_buffer_rsrc_t sr = make_rsrc(s + (size_t)n0 * ng, (uint32_t)(ncols * ng * 2));
    const __amdgpu_buffer_rsrc_t zr = make_rsrc(PGZ ? z + (size_t)n0 * ng : s, PGZ ? (uint32_t)(ncols * ng * 2) : 0u);
    uint16_t sv[CPW][RPL], zv[CPW][RPL];
#pragma unroll
    for (int j = 0; j < RPL; ++j) {
        const int r = lane + 64 * j;
        const int gi = (r * 32) / G;
#pragma unroll
        for (int c = 0; c < CPW; ++c) {
            const uint32_t off = (r < R) ? (uint32_t)(c * ng + gi) * 2u : OOB;
            sv[c][j] = __builtin_amdgcn_raw_buffer_load_b16(sr, off, 0, 0);
            zv[c][j] = PGZ ? __builtin_amdgcn_raw_buffer_load_b16(zr, off, 0, 0) : (uint16_t)0;
        }
    }

    // 3. this lane's activations, in slot order, and their bias sums.
    const __amdgpu_buffer_rsrc_t xr = make_rsrc(X, (uint32_t)K * 2u);
    half2_t xs[RPL][16];
    float c1[RPL], c2[RPL];
    const float zdef = (float)(1u << (BITS - 1));
#pragma unroll
    for (int j = 0; j < RPL; ++j) {
        const int r = lane + 64 * j;
        uint32_t raw[16];
        load_dwords<LOAD_DEFAULT>(xr, (r < R) ? (uint32_t)r * 64u : OOB, raw, 16);
        x_slots<BITS>(raw, xs[j]);
        float a1 = 0.f, a2 = 0.f;
#pragma unroll
        for (int p = 0; p < 16; ++p) {
            if (PGZ) {
                half2_t k1;
                k1[0] = (_Float16)1024.0f;
                k1[1] = (_Float16)1024.0f;
                a1 = __builtin_amdgcn_fdot2(xs[j][p], k1, a1, false);
                a2 = __builtin_amdgcn_fdot2(xs[j][p], slot_pow2<BITS>(p), a2, false);
            } else {
                a1 = __builtin_amdgcn_fdot2(xs[j][p], slot_bias<BITS>(p, zdef), a1, false);
            }
        }
        c1[j] = a1;
        c2[j] = a2;
    }

    // 4. per column: dot products, per-run scale, wave reduction.
    float yout = 0.f;
#pragma unroll
    for (int c = 0; c < CPW; ++c) {
        float y = 0.f;
#pragma unroll
        for (int j = 0; j < RPL; ++j) {
            uint32_t h[16];
            run_to_half2<BITS>(d[c][j], h);
            float a = 0.f;
#pragma unroll
            for (int p = 0; p < 16; ++p) a = __builtin_amdgcn_fdot2(xs[j][p], as_half2(h[p]), a, false);
            const float bias = PGZ ? fmaf((float)as_half(zv[c][j]), c2[j], c1[j]) : c1[j];
            y = fmaf((float)as_half(sv[c][j]), a - bias, y);
        }
        y = wave_sum(y);
        if (lane == c) yout = y;
    }
    if (lane < ncols) Y[n0 + lane] = f32_to_f16_bits(yout);
}

// ---------------------------------------------------------------------------
// 2 <= M <= 16 (and M = 1 with very long K): f16 MFMA 16x16x32, M padded to 16.
// A workgroup of 8 waves owns one 16-column tile at a time; the waves split K.
// In a K step of 128 rows, lane group g (lanes 16g..16g+15) owns run 4t+g of
// column (lane % 16): it unpacks the run to fp16 patterns, dequantises them in
// registers to w' = (q - z) 2^p s (exact subtraction, one rounding), and feeds
// four MFMAs.  The A operand holds X rows in the same slot order, pre-scaled
// by 2^-p, and stays in VGPRs across column tiles.  Partial tiles of the 8
// waves are summed through LDS in a fixed order.
// ---------------------------------------------------------------------------
template <int BITS, int T, bool PGZ>
__global__ __launch_bounds__(512) void gemv_mfma_kernel(const uint16_t *__restrict__ X, const uint32_t *__restrict__ wq,
                                                        const uint16_t *__restrict__ s,
                                                        const uint16_t *__restrict__ z, uint16_t *__restrict__ Y,
                                                        int M, int K, int N, int G, int passes)
{
    __shared__ float red[8][256];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int g = lane >> 4, c = lane & 15;
    const int R = K >> 5, ng = K / G;
    const uint32_t run_bytes = 4u * BITS;
    const uint32_t col_bytes = (uint32_t)R * run_bytes;
    const float zdef = (float)(1u << (BITS - 1));
    const __amdgpu_buffer_rsrc_t xr = make_rsrc(X, (uint32_t)((size_t)M * K * 2u));
    const int tiles = (N + 15) >> 4;

    half8_t a[T][4];
    int a_pass = -1;
    for (int tile = blockIdx.x; tile < tiles; tile += gridDim.x) {
        const int n = tile * 16 + c;
        const int nvalid = min(16, N - tile * 16);
        const __amdgpu_buffer_rsrc_t wr = make_rsrc(wq + (size_t)tile * 16 * R * BITS, (uint32_t)nvalid * col_bytes);
        const __amdgpu_buffer_rsrc_t sr = make_rsrc(s + (size_t)tile * 16 * ng, (uint32_t)(nvalid * ng * 2));
        const __amdgpu_buffer_rsrc_t zr =
            make_rsrc(PGZ ? z + (size_t)tile * 16 * ng : s, PGZ ? (uint32_t)(nvalid * ng * 2) : 0u);
        float4_t acc = {0.f, 0.f, 0.f, 0.f};
        for (int pass = 0; pass < passes; ++pass) {
            const int tt0 = pass * 8 * T + wave * T;
            uint32_t d[T][BITS];
            uint16_t sv[T], zv[T];
#pragma unroll
            for (int t = 0; t < T; ++t) {
                const int run = 4 * (tt0 + t) + g;
                const uint32_t off = (run < R) ? (uint32_t)c * col_bytes + (uint32_t)run * run_bytes : OOB;
                load_dwords<LOAD_STREAM>(wr, off, d[t], BITS);
                const uint32_t soff = (run < R) ? (uint32_t)(c * ng + (run * 32) / G) * 2u : OOB;
                sv[t] = __builtin_amdgcn_raw_buffer_load_b16(sr, soff, 0, 0);
                zv[t] = PGZ ? __builtin_amdgcn_raw_buffer_load_b16(zr, soff, 0, 0) : (uint16_t)0;
            }
            if (pass != a_pass) {
#pragma unroll
                for (int t = 0; t < T; ++t) {
                    const int run = 4 * (tt0 + t) + g;
                    uint32_t raw[16];
                    const uint32_t off = (run < R && c < M) ? ((uint32_t)c * K + (uint32_t)run * 32u) * 2u : OOB;
                    load_dwords<LOAD_DEFAULT>(xr, off, raw, 16);
                    half2_t xs[16];
                    x_slots<BITS>(raw, xs);
#pragma unroll
                    for (int u = 0; u < 4; ++u) {
                        half8_t v;
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            v[2 * e] = xs[4 * u + e][0];
                            v[2 * e + 1] = xs[4 * u + e][1];
                        }
                        a[t][u] = v;
                    }
                }
                a_pass = pass;
            }
#pragma unroll
            for (int t = 0; t < T; ++t) {
                uint32_t h[16];
                run_to_half2<BITS>(d[t], h);
                half2_t s2;
                s2[0] = as_half(sv[t]);
                s2[1] = s2[0];
                half2_t z2;
                z2[0] = as_half(zv[t]);
                z2[1] = z2[0];
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    half8_t b;
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int j = 4 * u + e;
                        half2_t bias;
                        if (PGZ) {
                            half2_t k1;
                            k1[0] = (_Float16)1024.0f;
                            k1[1] = (_Float16)1024.0f;
                            bias = z2 * slot_pow2<BITS>(j) + k1;
                        } else {
                            bias = slot_bias<BITS>(j, zdef);
                        }
                        const half2_t w = (as_half2(h[j]) - bias) * s2;
                        b[2 * e] = w[0];
                        b[2 * e + 1] = w[1];
                    }
                    acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[t][u], b, acc, 0, 0, 0);
                }
            }
        }
        // rows 4g..4g+3 of column c
#pragma unroll
        for (int i = 0; i < 4; ++i) red[wave][(4 * g + i) * 16 + c] = acc[i];
        __syncthreads();
        if (threadIdx.x < 256) {
            const int row = threadIdx.x >> 4, col = threadIdx.x & 15;
            float v = 0.f;
#pragma unroll
            for (int w = 0; w < 8; ++w) v += red[w][threadIdx.x];
            if (row < M && col < nvalid) Y[(size_t)row * N + tile * 16 + col] = f32_to_f16_bits(v);
        }
        __syncthreads();
        (void)n;
    }
}

// ---------------------------------------------------------------------------
// Launch selection.
// ---------------------------------------------------------------------------
template <int BITS, bool PGZ>
static hipError_t gemv_m1_launch(const GemvArgs &a, int rpl, hipStream_t st)
{
    constexpr int CPW = 4;
    const int waves = (a.N + CPW - 1) / CPW;
    const dim3 block(256), grid((waves + 3) / 4);
#define QMM_M1(RPL)                                                                                             \
    hipLaunchKernelGGL((gemv_m1_kernel<BITS, RPL, CPW, PGZ>), grid, block, 0, st, a.X, a.wq, a.s, a.z, a.Y, a.K, \
                       a.N, a.G)
    switch (rpl) {
        case 1: QMM_M1(1); break;
        case 2: QMM_M1(2); break;
        case 4: QMM_M1(4); break;
        case 8: QMM_M1(8); break;
        default: return hipErrorInvalidValue;
    }
#undef QMM_M1
    return hipGetLastError();
}

template <int BITS, bool PGZ>
static hipError_t gemv_mfma_launch(const GemvArgs &a, hipStream_t st)
{
    const int R = a.K / 32;
    const int TT = (R + 3) / 4;              // K steps of 128 rows
    int T = 1;
    while (T < 8 && 8 * T < TT) T <<= 1;
    const int passes = (TT + 8 * T - 1) / (8 * T);
    const int tiles = (a.N + 15) / 16;
    const dim3 block(512), grid((unsigned)min(tiles, 512));
#define QMM_MF(TV)                                                                                              \
    hipLaunchKernelGGL((gemv_mfma_kernel<BITS, TV, PGZ>), grid, block, 0, st, a.X, a.wq, a.s, a.z, a.Y, a.M, a.K, \
                       a.N, a.G, passes)
    switch (T) {
        case 1: QMM_MF(1); break;
        case 2: QMM_MF(2); break;
        case 4: QMM_MF(4); break;
        case 8: QMM_MF(8); break;
        default: return hipErrorInvalidValue;
    }
#undef QMM_MF
    return hipGetLastError();
}

template <int BITS>
static hipError_t gemv_dispatch(const GemvArgs &a, hipStream_t st)
{
    const int R = a.K / 32;
    const int rpl_need = (R + 63) / 64;
    if (a.M == 1 && rpl_need <= 8) {
        int rpl = 1;
        while (rpl < rpl_need) rpl <<= 1;
        return a.z ? gemv_m1_launch<BITS, true>(a, rpl, st) : gemv_m1_launch<BITS, false>(a, rpl, st);
    }
    return a.z ? gemv_mfma_launch<BITS, true>(a, st) : gemv_mfma_launch<BITS, false>(a, st);
}

hipError_t launch_gemv(const GemvArgs &a, hipStream_t st)
{
    switch (a.bits) {
        case 1: return gemv_dispatch<1>(a, st);
        case 2: return gemv_dispatch<2>(a, st);
        case 3: return gemv_dispatch<3>(a, st);
        case 4: return gemv_dispatch<4>(a, st);
        case 5: return gemv_dispatch<5>(a, st);
        case 6: return gemv_dispatch<6>(a, st);
        case 7: return gemv_dispatch<7>(a, st);
        case 8: return gemv_dispatch<8>(a, st);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace qmm
