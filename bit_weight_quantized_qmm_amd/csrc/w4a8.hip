// w4a8.hip -- int8 activations x 4-bit weights with exact int32 group sums.
//
// BitLLM Sec. 4.3 defines the integer dot product (dp4a: products of 8-bit
// values summed exactly into an int32) and Sec. 4.4 keeps the whole hot loop in
// the integer domain, applying the scale only at the tile boundary.  Here the
// integer products run on v_mfma_i32_16x16x64_i8; the tile boundary is the
// quantisation group:
//   A[m][g][n] = sum_{i in g} Xq[m][i] * q[i][n]  -  z[n][g] * sum_{i in g} Xq[m][i]
//   y[m][n]   += s[n][g] * float(A[m][g][n]),          Y = fp16(sx[m] * y)
// 4-bit codes become int8 lanes with one AND (even nibbles) and one shift+AND
// (odd nibbles) per dword; Xq is permuted once into that byte order.  The
// per-row group sums of Xq come from the same MFMA against an all-ones B.
//
// Workgroup: 8 waves split K for one 16-column x 16-row tile; a K step is 128
// rows = 4 runs, lane group g owning run 4t+g.  Requires G % 128 == 0 so that
// every K step lies inside one group.
#include "launch.hpp"
#include "qmm_device.hpp"

namespace qmm {

constexpr uint32_t W_OOB = 0x80000000u;

template <int T, bool PGZ>
__global__ __launch_bounds__(512) void w4a8_kernel(const int8_t *__restrict__ Xq, const uint16_t *__restrict__ sx,
                                                   const uint32_t *__restrict__ wq, const uint16_t *__restrict__ s,
                                                   const uint16_t *__restrict__ z, uint16_t *__restrict__ Y,
                                                   int32_t *__restrict__ acc_out, int M, int K, int N, int G,
                                                   int passes)
{
    __shared__ float red[8][256];
    const int lane = threadIdx.x & 63, wave = wave_id();
    const int g = lane >> 4, c = lane & 15;
    const int m0 = blockIdx.y * 16;
    const int R = K >> 5, ng = K / G, steps_per_group = G / 128;
    const uint32_t col_bytes = (uint32_t)R * 16u;
    const int mrows = min(16, M - m0);
    const __amdgpu_buffer_rsrc_t xr = make_rsrc(Xq + (size_t)m0 * K, (uint32_t)((size_t)mrows * K));
    const int tiles = (N + 15) >> 4;
    const int4_t ones = {0x01010101, 0x01010101, 0x01010101, 0x01010101};

    int4_t a[T][2];
    int4_t sxg[T];   // per K step: group sums of Xq rows 4g..4g+3 (from the MFMA against ones)
    int a_pass = -1;
    for (int tile = blockIdx.x; tile < tiles; tile += gridDim.x) {
        const int n = tile * 16 + c;
        const int nvalid = min(16, N - tile * 16);
        const __amdgpu_buffer_rsrc_t wr = make_rsrc(wq + (size_t)tile * 16 * R * 4, (uint32_t)nvalid * col_bytes);
        const __amdgpu_buffer_rsrc_t sr = make_rsrc(s + (size_t)tile * 16 * ng, (uint32_t)(nvalid * ng * 2));
        const __amdgpu_buffer_rsrc_t zr =
            make_rsrc(PGZ ? z + (size_t)tile * 16 * ng : s, PGZ ? (uint32_t)(nvalid * ng * 2) : 0u);
        float y[4] = {0.f, 0.f, 0.f, 0.f};
        for (int pass = 0; pass < passes; ++pass) {
            const int tt0 = pass * 8 * T + wave * T;
            uint32_t d[T][4];
            uint16_t sv[T], zv[T];
#pragma unroll
            for (int t = 0; t < T; ++t) {
                const int tt = tt0 + t;
                const int run = 4 * tt + g;
                const uint32_t off = (run < R) ? (uint32_t)c * col_bytes + (uint32_t)run * 16u : W_OOB;
                load_dwords<LOAD_STREAM>(wr, off, d[t], 4);
                const uint32_t soff = (4 * tt < R) ? (uint32_t)(c * ng + (tt * 128) / G) * 2u : W_OOB;
                sv[t] = __builtin_amdgcn_raw_buffer_load_b16(sr, soff, 0, 0);
                zv[t] = PGZ ? __builtin_amdgcn_raw_buffer_load_b16(zr, soff, 0, 0) : (uint16_t)0;
            }
            if (pass != a_pass) {
#pragma unroll
                for (int t = 0; t < T; ++t) {
                    const int run = 4 * (tt0 + t) + g;
                    uint32_t x[8];
                    const uint32_t off = (run < R) ? (uint32_t)c * K + (uint32_t)run * 32u : W_OOB;
                    load_dwords<LOAD_DEFAULT>(xr, off, x, 8);
#pragma unroll
                    for (int v = 0; v < 2; ++v) {
                        int4_t av;
                        av[0] = (int)__builtin_amdgcn_perm(x[4 * v + 1], x[4 * v], 0x06040200u);
                        av[1] = (int)__builtin_amdgcn_perm(x[4 * v + 1], x[4 * v], 0x07050301u);
                        av[2] = (int)__builtin_amdgcn_perm(x[4 * v + 3], x[4 * v + 2], 0x06040200u);
                        av[3] = (int)__builtin_amdgcn_perm(x[4 * v + 3], x[4 * v + 2], 0x07050301u);
                        a[t][v] = av;
                    }
                    int4_t zero4 = {0, 0, 0, 0};
                    int4_t sum = __builtin_amdgcn_mfma_i32_16x16x64_i8(a[t][0], ones, zero4, 0, 0, 0);
                    sxg[t] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a[t][1], ones, sum, 0, 0, 0);
                }
                a_pass = pass;
            }
            int4_t graw = {0, 0, 0, 0}, gsx = {0, 0, 0, 0};
#pragma unroll
            for (int t = 0; t < T; ++t) {
                const int tt = tt0 + t;
                int4_t raw = {0, 0, 0, 0};
#pragma unroll
                for (int v = 0; v < 2; ++v) {
                    const uint32_t da = d[t][2 * v], db = d[t][2 * v + 1];
                    int4_t bv;
                    bv[0] = (int)(da & 0x0f0f0f0fu);
                    bv[1] = (int)((da >> 4) & 0x0f0f0f0fu);
                    bv[2] = (int)(db & 0x0f0f0f0fu);
                    bv[3] = (int)((db >> 4) & 0x0f0f0f0fu);
                    raw = __builtin_amdgcn_mfma_i32_16x16x64_i8(a[t][v], bv, raw, 0, 0, 0);
                }
                graw += raw;
                gsx += sxg[t];
                if ((tt + 1) % steps_per_group == 0 || 4 * (tt + 1) >= R) {
                    const int grp = (tt * 128) / G;
                    const int zz = PGZ ? (int)(float)as_half(zv[t]) : 8;
                    const float sc = (float)as_half(sv[t]);
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int A = graw[i] - zz * gsx[i];
                        const int row = 4 * g + i;
                        if (acc_out && 4 * tt < R && row < mrows && c < nvalid)
                            acc_out[((size_t)(m0 + row) * ng + grp) * N + n] = A;
                        y[i] = fmaf(sc, (float)A, y[i]);
                    }
                    graw = int4_t{0, 0, 0, 0};
                    gsx = int4_t{0, 0, 0, 0};
                }
            }
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) red[wave][(4 * g + i) * 16 + c] = y[i];
        __syncthreads();
        if (threadIdx.x < 256) {
            const int row = threadIdx.x >> 4, col = threadIdx.x & 15;
            float v = 0.f;
#pragma unroll
            for (int w = 0; w < 8; ++w) v += red[w][threadIdx.x];
            if (row < mrows && col < nvalid) {
                const float sxm = (float)as_half(sx[m0 + row]);
                Y[(size_t)(m0 + row) * N + tile * 16 + col] = f32_to_f16_bits(sxm * v);
            }
        }
        __syncthreads();
    }
}

template <bool PGZ>
static hipError_t w4a8_go(const W4A8Args &a, int T, int passes, dim3 grid, hipStream_t st)
{
    const dim3 block(512);
#define QMM_W(TV)                                                                                            \
    hipLaunchKernelGGL((w4a8_kernel<TV, PGZ>), grid, block, 0, st, a.Xq, a.sx, a.wq, a.s, a.z, a.Y, a.acc, a.M, \
                       a.K, a.N, a.G, passes)
    switch (T) {
        case 1: QMM_W(1); break;
        case 2: QMM_W(2); break;
        case 4: QMM_W(4); break;
        case 8: QMM_W(8); break;
        default: return hipErrorInvalidValue;
    }
#undef QMM_W
    return hipGetLastError();
}

// Returns hipErrorNotSupported for shapes this kernel does not cover.
hipError_t launch_w4a8(const W4A8Args &a, hipStream_t st)
{
    if (a.G % 128 != 0 || a.G > 1024) return hipErrorNotSupported;
    const int R = a.K / 32;
    const int TT = (R + 3) / 4;
    int T = 1;
    while (T < 8 && 8 * T < TT) T <<= 1;
    while (T < 8 && T * 128 < a.G) T <<= 1;   // a wave's K range covers whole groups
    const int passes = (TT + 8 * T - 1) / (8 * T);
    const int tiles = (a.N + 15) / 16;
    const int mtiles = (a.M + 15) / 16;
    if (mtiles > 65535) return hipErrorNotSupported;
    const dim3 grid((unsigned)min(tiles, 512), (unsigned)mtiles);
    return a.z ? w4a8_go<true>(a, T, passes, grid, st) : w4a8_go<false>(a, T, passes, grid, st);
}

}  // namespace qmm
