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
// 1 <= M <= 4 (the decode shapes): f16 MFMA with one accumulator row per
// (activation row m, run e).  A workgroup of ks waves owns one 16-column tile;
// the waves split K, T steps of 128 rows each.  In a step, lane group g holds
// run 4t+g of column lane%16 as fp16 patterns (the B operand, straight from
// run_to_half2); the A operand row 4m+e carries x_m (slot order, scaled by
// 2^-p) only in lane group e, zeros elsewhere, so accumulator row 4m+e is the
// partial sum of run 4t+e alone.  Starting the accumulator at minus the run's
// bias sum leaves sum x*(q - z) per run; y += s * that, with the run's own
// group scale, so any G works.  X is staged once per workgroup in LDS (slot
// order + per-run bias sums); the tile's scales too.  Weight loads are issued
// right after the X and scale loads, before any arithmetic.
// ---------------------------------------------------------------------------
template <int BITS, int T, int IPT, bool G128, bool PGZ>
__global__ __launch_bounds__(1024) void gemv_rows_kernel(const uint16_t *__restrict__ X,
                                                         const uint32_t *__restrict__ wq,
                                                         const uint16_t *__restrict__ s,
                                                         const uint16_t *__restrict__ z, uint16_t *__restrict__ Y,
                                                         int M, int K, int N, int G, int ks)
{
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    using P = RunPlan<BITS>;
    const int R = K >> 5, R4 = (R + 3) & ~3, TT = R4 >> 2, ng = K / G;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, nthreads = 64 * ks;
    const int g = lane >> 4, c = lane & 15;
    const int n0 = blockIdx.x * 16;
    const int nvalid = min(16, N - n0);
    const uint32_t run_bytes = 4u * BITS, col_bytes = (uint32_t)R * run_bytes;

    // LDS: xs [M][R4] runs x 64 B | 64 B zeros | 64 B dummy | c1 [M][R4] + 4 dummy |
    //      c2 [M][R4] + 4 dummy (PGZ) | sl [16][ng] + 8 dummy | zl [16][ng] + 8 dummy (PGZ) |
    //      red [ks][4][16].  Staging threads without an item write the dummy slots, so the
    //      staging code has no branches (a branch would let the compiler sink the
    //      activation loads behind the weight loads, and loads complete in order).
    const uint32_t xs_bytes = (uint32_t)M * R4 * 64u;
    const int MR = M * R4 + 4;
    float *c1 = reinterpret_cast<float *>(smem + xs_bytes + 128);
    float *c2 = c1 + MR;
    uint16_t *sl = reinterpret_cast<uint16_t *>(c2 + (PGZ ? MR : 0));
    uint16_t *zl = sl + 16 * ng + 8;
    float *red = reinterpret_cast<float *>(smem + ((xs_bytes + 128 + 4u * MR * (PGZ ? 2 : 1) +
                                                    2u * (16 * ng + 8) * (PGZ ? 2 : 1) + 15u) & ~15u));

    // 1. activations for the staging (IPT (row, run) items per thread)
    const __amdgpu_buffer_rsrc_t xr = make_rsrc(X, (uint32_t)(M * K * 2));
    uint32_t raw[IPT][16];
#pragma unroll
    for (int i = 0; i < IPT; ++i) {
        const int it = tid + i * nthreads;
        const int m = it / R4, r = it - m * R4;
        const uint32_t off = (m < M && r < R) ? ((uint32_t)m * K + (uint32_t)r * 32u) * 2u : OOB;
        load_dwords<LOAD_DEFAULT>(xr, off, raw[i], 16);
    }
    // 2. the tile's scales (and zero-points): 16 contiguous rows of ng halves
    const uint32_t sbytes = (uint32_t)nvalid * ng * 2u;
    const __amdgpu_buffer_rsrc_t sr = make_rsrc(s + (size_t)n0 * ng, sbytes);
    const __amdgpu_buffer_rsrc_t zr = make_rsrc(PGZ ? z + (size_t)n0 * ng : s, PGZ ? sbytes : 0u);
    uint32_t sraw[4], zraw[4];
    const bool s_thread = tid < 2 * ng;   // 16 * ng halves = 2 * ng chunks of 16 B
    load_dwords<LOAD_DEFAULT>(sr, s_thread ? (uint32_t)tid * 16u : OOB, sraw, 4);
    if (PGZ) load_dwords<LOAD_DEFAULT>(zr, s_thread ? (uint32_t)tid * 16u : OOB, zraw, 4);
    __builtin_amdgcn_sched_barrier(0);
    // 3. this wave's packed weights, all in flight before any arithmetic
    const __amdgpu_buffer_rsrc_t wr = make_rsrc(wq + (size_t)n0 * R * BITS, (uint32_t)nvalid * col_bytes);
    const int tt0 = wave * T;
    uint32_t d[T][BITS];
#pragma unroll
    for (int t = 0; t < T; ++t) {
        const int run = 4 * (tt0 + t) + g;
        const uint32_t off = (run < R) ? (uint32_t)c * col_bytes + (uint32_t)run * run_bytes : OOB;
        load_dwords<LOAD_STREAM>(wr, off, d[t], BITS);
    }

    __builtin_amdgcn_sched_barrier(0);
    // 4. stage X in slot order with its per-run bias sums; scales; zero pad
    const float zdef = (float)(1u << (BITS - 1));
#pragma unroll
    for (int i = 0; i < IPT; ++i) {
        const int it0 = tid + i * nthreads;
        const int it = it0 < M * R4 ? it0 : M * R4;   // M * R4 = the dummy item
        {
            half2_t xs[16];
            x_slots<BITS>(raw[i], xs);
            float a1 = 0.f, a2 = 0.f;
#pragma unroll
            for (int p = 0; p < 16; ++p) {
                if (PGZ) {
                    half2_t k1;
                    k1[0] = (_Float16)1024.0f;
                    k1[1] = (_Float16)1024.0f;
                    a1 = __builtin_amdgcn_fdot2(xs[p], k1, a1, false);
                    a2 = __builtin_amdgcn_fdot2(xs[p], slot_pow2<BITS>(p), a2, false);
                } else {
                    a1 = __builtin_amdgcn_fdot2(xs[p], slot_bias<BITS>(p, zdef), a1, false);
                }
            }
            int4_t *dst = reinterpret_cast<int4_t *>(smem + (it0 < M * R4 ? (uint32_t)it * 64u : xs_bytes + 64u));
#pragma unroll
            for (int q = 0; q < 4; ++q)
                dst[q] = int4_t{(int)as_u32(xs[4 * q]), (int)as_u32(xs[4 * q + 1]), (int)as_u32(xs[4 * q + 2]),
                                (int)as_u32(xs[4 * q + 3])};
            c1[it] = a1;
            if (PGZ) c2[it] = a2;
        }
    }
    {
        const int si = s_thread ? 8 * tid : 16 * ng;   // 16 * ng = the dummy chunk
        *reinterpret_cast<int4_t *>(sl + si) = int4_t{(int)sraw[0], (int)sraw[1], (int)sraw[2], (int)sraw[3]};
        if (PGZ)
            *reinterpret_cast<int4_t *>(zl + si) = int4_t{(int)zraw[0], (int)zraw[1], (int)zraw[2], (int)zraw[3]};
    }
    if (tid < 4) reinterpret_cast<int4_t *>(smem + xs_bytes)[tid] = int4_t{0, 0, 0, 0};
    __syncthreads();

    // 5. K steps: 4 MFMAs per step, bias as the accumulator's start value
    const int r_row = c;                          // MFMA A row held by this lane
    const int am = r_row >> 2, ae = r_row & 3;    // (activation row, run) of that A row
    const bool a_live = (ae == g) && (am < M);
    const int om = g;                             // output rows 4g..4g+3 = (row g, runs 0..3)
    const int omc = min(om, M - 1);
    float y = 0.f;
#pragma unroll
    for (int t = 0; t < T; ++t) {
        const int tt = tt0 + t;
        if (tt >= TT) break;                       // wave-uniform
        uint32_t h[16];
        run_to_half2<BITS>(d[t], h);
        const float4_t cb = *reinterpret_cast<const float4_t *>(c1 + omc * R4 + 4 * tt);
        float4_t acc;
        if (PGZ) {
            const float4_t cz = *reinterpret_cast<const float4_t *>(c2 + omc * R4 + 4 * tt);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int gi = min(((4 * tt + e) * 32) / G, ng - 1);
                acc[e] = -fmaf((float)as_half(zl[c * ng + gi]), cz[e], cb[e]);
            }
        } else {
            acc = -cb;
        }
        const uint32_t abase = a_live ? ((uint32_t)(am * R4 + 4 * tt + g) * 64u) : xs_bytes;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const half8_t a = *reinterpret_cast<const half8_t *>(smem + abase + 16u * u);
            const half8_t b = __builtin_bit_cast(half8_t, int4_t{(int)h[4 * u], (int)h[4 * u + 1],
                                                                 (int)h[4 * u + 2], (int)h[4 * u + 3]});
            acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, acc, 0, 0, 0);
        }
        if (G128) {
            const float sc = (float)as_half(sl[c * ng + (tt * 128) / G]);
            y = fmaf(sc, (acc[0] + acc[1]) + (acc[2] + acc[3]), y);
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int gi = min(((4 * tt + e) * 32) / G, ng - 1);
                y = fmaf((float)as_half(sl[c * ng + gi]), acc[e], y);
            }
        }
    }

    // 6. fixed-order sum over the ks waves
    if (om < M) red[(wave * 4 + om) * 16 + c] = y;
    __syncthreads();
    if (tid < M * 16) {
        const int m = tid >> 4, cc = tid & 15;
        float v = 0.f;
        for (int w = 0; w < ks; ++w) v += red[(w * 4 + m) * 16 + cc];
        if (cc < nvalid) Y[(size_t)m * N + n0 + cc] = f32_to_f16_bits(v);
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

// LDS bytes of gemv_rows_kernel for (M, K, G, ks); 0 if it does not apply.
static size_t rows_lds_bytes(int M, int K, int G, int ks, bool pgz)
{
    const int R = K / 32, R4 = (R + 3) & ~3, ng = K / G;
    size_t b = (size_t)M * R4 * 64 + 128 + 4u * (size_t)(M * R4 + 4) * (pgz ? 2 : 1) +
               2u * (size_t)(16 * ng + 8) * (pgz ? 2 : 1);
    b = (b + 15) & ~(size_t)15;
    return b + (size_t)ks * 4 * 16 * 4;
}

template <int BITS, int T, int IPT, bool G128, bool PGZ>
static hipError_t gemv_rows_go(const GemvArgs &a, int ks, size_t lds, hipStream_t st)
{
    static bool attr_set = false;   // raise the dynamic-LDS limit once per instantiation
    if (!attr_set) {
        hipError_t e =
            hipFuncSetAttribute(reinterpret_cast<const void *>(&gemv_rows_kernel<BITS, T, IPT, G128, PGZ>),
                                hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
        if (e != hipSuccess) return e;
        attr_set = true;
    }
    const dim3 block(64 * ks), grid((a.N + 15) / 16);
    hipLaunchKernelGGL((gemv_rows_kernel<BITS, T, IPT, G128, PGZ>), grid, block, lds, st, a.X, a.wq, a.s, a.z, a.Y,
                       a.M, a.K, a.N, a.G, ks);
    return hipGetLastError();
}

template <int BITS, int IPT, bool G128, bool PGZ>
static hipError_t gemv_rows_pick_t(const GemvArgs &a, int T, int ks, size_t lds, hipStream_t st)
{
    switch (T) {
        case 1: return gemv_rows_go<BITS, 1, IPT, G128, PGZ>(a, ks, lds, st);
        case 2: return gemv_rows_go<BITS, 2, IPT, G128, PGZ>(a, ks, lds, st);
        case 4: return gemv_rows_go<BITS, 4, IPT, G128, PGZ>(a, ks, lds, st);
        default: return gemv_rows_go<BITS, 8, IPT, G128, PGZ>(a, ks, lds, st);
    }
}

template <int BITS, int IPT>
static hipError_t gemv_rows_pick(const GemvArgs &a, int T, int ks, size_t lds, hipStream_t st)
{
    const bool g128 = a.G % 128 == 0;
    if (a.z) return g128 ? gemv_rows_pick_t<BITS, IPT, true, true>(a, T, ks, lds, st)
                         : gemv_rows_pick_t<BITS, IPT, false, true>(a, T, ks, lds, st);
    return g128 ? gemv_rows_pick_t<BITS, IPT, true, false>(a, T, ks, lds, st)
                : gemv_rows_pick_t<BITS, IPT, false, false>(a, T, ks, lds, st);
}

template <int BITS>
static hipError_t gemv_dispatch(const GemvArgs &a, hipStream_t st)
{
    const int R = a.K / 32, TT = (R + 3) / 4;
    if (a.M <= 4) {
        int T = 1;
        while (T < 8 && T < TT) T <<= 1;
        const int ks = (TT + T - 1) / T;
        const size_t lds = rows_lds_bytes(a.M, a.K, a.G, ks, a.z != nullptr);
        const int R4 = (R + 3) & ~3;
        if (ks <= 16 && lds <= 160 * 1024 && 2 * (a.K / a.G) <= 64 * ks) {
            if (a.M * R4 <= 64 * ks) return gemv_rows_pick<BITS, 1>(a, T, ks, lds, st);
            if (a.M * R4 <= 2 * 64 * ks) return gemv_rows_pick<BITS, 2>(a, T, ks, lds, st);
        }
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
