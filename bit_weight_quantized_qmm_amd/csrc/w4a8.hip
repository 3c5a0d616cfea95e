// w4a8.hip -- int8 activations x k-bit weights (k = 1..8) with exact int32
// group sums.
//
// BitLLM Sec. 4.3 defines the integer dot product (dp4a: products of 8-bit
// values summed exactly into an int32) and Sec. 4.4 keeps the whole hot loop in
// the integer domain, applying the scale only at the tile boundary.  Here the
// integer products run on v_mfma_i32_16x16x64_i8; the tile boundary is the
// quantisation group:
//   A[m][g][n] = sum_{i in g} Xq[m][i] * q[i][n]  -  z[n][g] * sum_{i in g} Xq[m][i]
//   y[m][n]   += s[n][g] * float(A[m][g][n]),          Y = fp16(sx[m] * y)
// A lane's run of 32 codes becomes 32 int8 lanes (wka8_dword): for k = 1, 2, 4
// one shift and one AND per output dword, for k = 8 the bytes themselves with
// the sign bit flipped (q - 128, the zero point shifted to match), for the odd
// widths one bit-field extract per code.  Xq is permuted once into the same
// byte order.  The per-row group sums of Xq come from the same MFMA against an
// all-ones B.
//
// Workgroup: 8 waves split K for one 16-column x 16-row tile; a K step is 128
// rows = 4 runs, lane group g owning run 4t+g.  Requires G % 128 == 0 so that
// every K step lies inside one group.
#include <algorithm>
#include <type_traits>

#include "launch.hpp"
#include "qmm_device.hpp"

namespace qmm {

constexpr uint32_t W_OOB = 0x80000000u;

// Byte b of dword o (o = 0..7) of a run's int8 form holds code wka8_code(o, b)
// of the run.  For k = 1, 2, 4 (C = 32 / k codes per dword, P = C / 4 output
// dwords per input dword) output dword o is input dword o / P shifted right by
// k (o % P) and masked to the low k bits of every byte; k = 8 and the odd
// widths keep the codes in order.
template <int BITS>
__host__ __device__ constexpr int wka8_code(int o, int b)
{
    return (BITS == 1 || BITS == 2 || BITS == 4) ? (32 / BITS) * (o / (8 / BITS)) + (8 / BITS) * b + o % (8 / BITS)
                                                 : 4 * o + b;
}

// Output dword o of the int8 form of a run of BITS dwords (o a compile-time
// constant after unrolling).  For k = 8 the byte is q - 128: a signed byte.
template <int BITS>
__device__ __forceinline__ uint32_t wka8_dword(const uint32_t (&d)[BITS], int o)
{
    if constexpr (BITS == 8) {
        return d[o] ^ 0x80808080u;
    } else if constexpr (BITS == 1 || BITS == 2 || BITS == 4) {
        constexpr int P = 8 / BITS;
        constexpr uint32_t mask = ((1u << BITS) - 1u) * 0x01010101u;
        return (d[o / P] >> (BITS * (o % P))) & mask;
    } else {
        uint32_t r = 0;
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            const int bit = (4 * o + b) * BITS, w = bit >> 5, sh = bit & 31;
            const uint32_t v = sh + BITS <= 32 ? (d[w] >> sh) : __builtin_amdgcn_alignbit(d[w + 1], d[w], sh);
            r |= (v & ((1u << BITS) - 1u)) << (8 * b);
        }
        return r;
    }
}

// Dword o of a row's 32 activation bytes x[0..7] in the same order.
template <int BITS>
__device__ __forceinline__ uint32_t wka8_xdword(const uint32_t (&x)[8], int o)
{
    if constexpr (BITS == 4) {
        // bytes 0, 2, 4, 6 (o even) or 1, 3, 5, 7 (o odd) of x[o & ~1], x[o | 1]
        return __builtin_amdgcn_perm(x[o | 1], x[o & ~1], (o & 1) ? 0x07050301u : 0x06040200u);
    } else if constexpr (BITS == 8 || !(BITS == 1 || BITS == 2)) {
        return x[o];
    } else {
        uint32_t r = 0;
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            const int i = wka8_code<BITS>(o, b);
            r |= ((x[i >> 2] >> (8 * (i & 3))) & 0xffu) << (8 * b);
        }
        return r;
    }
}

// Zero point as the integer the int8 B operand needs: z for k < 8, z - 128
// for k = 8 (whose B bytes are q - 128); the default z is 2^(k-1).
template <int BITS, bool PGZ>
__device__ __forceinline__ int wka8_zero(uint32_t zbits)
{
    const int zq = PGZ ? (int)(float)as_half((uint16_t)zbits) : (1 << (BITS - 1));
    return BITS == 8 ? zq - 128 : zq;
}

template <int BITS, int T, bool PGZ>
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
    const float ginv = run_group_inv(G);
    const uint32_t run_bytes = 4u * BITS, col_bytes = (uint32_t)R * run_bytes;
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
        const __amdgpu_buffer_rsrc_t wr = make_rsrc(wq + (size_t)tile * 16 * R * BITS, (uint32_t)nvalid * col_bytes);
        const __amdgpu_buffer_rsrc_t sr = make_rsrc(s + (size_t)tile * 16 * ng, (uint32_t)(nvalid * ng * 2));
        const __amdgpu_buffer_rsrc_t zr =
            make_rsrc(PGZ ? z + (size_t)tile * 16 * ng : s, PGZ ? (uint32_t)(nvalid * ng * 2) : 0u);
        float y[4] = {0.f, 0.f, 0.f, 0.f};
        for (int pass = 0; pass < passes; ++pass) {
            const int tt0 = pass * 8 * T + wave * T;
            uint32_t d[T][BITS];
            uint16_t sv[T], zv[T];
#pragma unroll
            for (int t = 0; t < T; ++t) {
                const int tt = tt0 + t;
                const int run = 4 * tt + g;
                const uint32_t off = (run < R) ? (uint32_t)c * col_bytes + (uint32_t)run * run_bytes : W_OOB;
                load_dwords<LOAD_STREAM>(wr, off, d[t], BITS);
                const uint32_t soff = (4 * tt < R) ? (uint32_t)(c * ng + run_group(4 * tt, ginv)) * 2u : W_OOB;
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
                    for (int v = 0; v < 2; ++v)
#pragma unroll
                        for (int e = 0; e < 4; ++e) a[t][v][e] = (int)wka8_xdword<BITS>(x, 4 * v + e);
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
                    int4_t bv;
#pragma unroll
                    for (int e = 0; e < 4; ++e) bv[e] = (int)wka8_dword<BITS>(d[t], 4 * v + e);
                    raw = __builtin_amdgcn_mfma_i32_16x16x64_i8(a[t][v], bv, raw, 0, 0, 0);
                }
                graw += raw;
                gsx += sxg[t];
                if ((tt + 1) % steps_per_group == 0 || 4 * (tt + 1) >= R) {
                    const int grp = run_group(4 * tt, ginv);
                    const int zz = wka8_zero<BITS, PGZ>(zv[t]);
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

// ---------------------------------------------------------------------------
// Streaming form for K <= 8192 and G in {128, 256, 512, 1024} (G / 128 steps
// per group, never more than a wave's K slice): 8 waves per workgroup, wave w
// owns K steps w*S .. w*S + S - 1 (128 rows each) and keeps their int8 A
// fragments and the row sums of Xq (from the MFMA against ones) in registers.
// The s and z of the workgroup's (at most T) column tiles are staged once in
// LDS, so only the weight runs stream: units (tile, step) pass through a ring
// of D weight loads, each column tile walked front to back along K.  A group's
// int32 sum A = raw - z * sum(Xq) is exact, optionally dumped, and scaled into
// the fp32 partial y; at the end the 8 partial tiles are added in LDS.
// ---------------------------------------------------------------------------
template <int BITS, int S, int T, int D, bool PGZ>
__global__ __launch_bounds__(512) void w4a8_stream_kernel(const int8_t *__restrict__ Xq, const uint16_t *__restrict__ sx,
                                                          const uint32_t *__restrict__ wq,
                                                          const uint16_t *__restrict__ s, const uint16_t *__restrict__ z,
                                                          uint16_t *__restrict__ Y, int32_t *__restrict__ acc_out,
                                                          int M, int K, int N, int G, int tpw)
{
    static_assert(S % D == 0 || D % S == 0, "ring slots must stay compile-time indexes");
    __shared__ float red[8][T][64][4];
    // s | z << 16 of (group, column) for the workgroup's columns, group-major;
    // the odd row stride keeps the transposing writes free of bank conflicts
    constexpr int SZW = T * 16 + 1;
    __shared__ uint32_t sz[64 * SZW];   // K <= 8192, G >= 128: at most 64 groups
    const int lane = threadIdx.x & 63, wave = wave_id();
    const int g = lane >> 4, c = lane & 15;
    const int m0 = blockIdx.y * 16;
    const int mrows = min(16, M - m0);
    const int R = K >> 5, ng = K / G, TT = R >> 2, sp = G >> 7;
    const bool dump = acc_out != nullptr;
    const uint32_t run_bytes = 4u * BITS, col_bytes = (uint32_t)R * run_bytes;
    const int tiles = (N + 15) >> 4;
    const int tile0 = blockIdx.x * tpw;
    const int ntile = min(tpw, tiles - tile0);   // 1 <= ntile <= T
    const __amdgpu_buffer_rsrc_t xr = make_rsrc(Xq + (size_t)m0 * K, (uint32_t)((size_t)mrows * K));
    const __amdgpu_buffer_rsrc_t wr = make_rsrc(wq, (uint32_t)((size_t)N * col_bytes));
    const __amdgpu_buffer_rsrc_t sr = make_rsrc(s, (uint32_t)(N * ng * 2));
    const __amdgpu_buffer_rsrc_t zr = make_rsrc(PGZ ? z : s, PGZ ? (uint32_t)(N * ng * 2) : 0u);
    const int4_t ones = {0x01010101, 0x01010101, 0x01010101, 0x01010101};

    // the wave's Xq runs first: their round trip then overlaps the s | z
    // table's instead of following it (8B MLP shape at K 1024: 5.5 -> 4.9 us;
    // K 4096: 10.4 -> 10.3)
    uint32_t x[S][8];
#pragma unroll
    for (int st = 0; st < S; ++st) {
        const int run = 4 * (wave * S + st) + g;
        load_dwords<LOAD_DEFAULT>(xr, (run < R && c < mrows) ? (uint32_t)c * K + (uint32_t)run * 32u : W_OOB, x[st], 8);
    }
    // s and z of the workgroup's columns: wave w reads columns w, w + 8, ...,
    // lane l holding group l (past ng, or past the workgroup's columns: zeros)
    constexpr int SZE = T * 16 / 8;
    uint32_t sraw[SZE], zraw[SZE];
#pragma unroll
    for (int e = 0; e < SZE; ++e) {
        const int cl = wave + 8 * e;
        const uint32_t off = (lane < ng && cl < 16 * ntile) ? ((uint32_t)(16 * tile0 + cl) * (uint32_t)ng + (uint32_t)lane) * 2u : W_OOB;
        sraw[e] = __builtin_amdgcn_raw_buffer_load_b16(sr, off, 0, 0);
        zraw[e] = PGZ ? __builtin_amdgcn_raw_buffer_load_b16(zr, off, 0, 0) : 0u;
    }

    // weights of unit (tile j, step st) for lane (g, c): column 16 (tile) + c, run
    // 4 t + g of step t = wave * S + st.  A step past K reads other bits of the
    // resource (or zeros past its end) and meets zero activations; units past the
    // workgroup's tiles load nothing.
    uint32_t d[D][BITS];
    auto issue = [&](int j, int st, int slot) {
        const int t = wave * S + st;
        const uint32_t col = (uint32_t)(16 * (tile0 + j) + c);
        // non-temporal for k = 4, the default policy otherwise (8B MLP shape:
        // k = 4 11.3 against 11.8 us; k = 5 16.1 against 21.9, k = 8 15.7
        // against 17.4 with it)
        constexpr int POL = BITS == 4 ? LOAD_STREAM : LOAD_DEFAULT;
        load_dwords<POL>(wr, j < ntile ? col * col_bytes + (uint32_t)(4 * t + g) * run_bytes : W_OOB, d[slot], BITS);
    };
#pragma unroll
    for (int u = 0; u < D; ++u) issue(u / S, u % S, u);

#pragma unroll
    for (int e = 0; e < SZE; ++e) {
        const int cl = wave + 8 * e;
        if (lane < ng) sz[lane * SZW + cl] = (sraw[e] & 0xffffu) | (zraw[e] << 16);
    }

    // A fragments of step st: lane (g, c) holds row c, run 4 t + g (32 bytes), bytes
    // permuted to the nibble order of the B operand (even codes, then odd codes)
    int4_t a[S][2], sxg[S];
    {
#pragma unroll
        for (int st = 0; st < S; ++st) {
#pragma unroll
            for (int v = 0; v < 2; ++v)
#pragma unroll
                for (int e = 0; e < 4; ++e) a[st][v][e] = (int)wka8_xdword<BITS>(x[st], 4 * v + e);
            const int4_t zero4 = {0, 0, 0, 0};
            sxg[st] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a[st][1], ones,
                                                             __builtin_amdgcn_mfma_i32_16x16x64_i8(a[st][0], ones, zero4, 0, 0, 0),
                                                             0, 0, 0);
        }
    }
    __syncthreads();

    // UT tiles per loop iteration keep every ring slot a compile-time index
    constexpr int UT = D > S ? D / S : 1;
    // the tile loop, compiled for SP1 (G = 128, every step ends its group: no
    // running sums) or the general case, each with and without the dump of the
    // sums; uniform branches pick one
    const int lsp = __builtin_ctz((unsigned)sp);   // sp = G / 128 is a power of two
    auto tiles_loop = [&](auto sp1_tag, auto dump_tag) {
        constexpr bool SP1 = decltype(sp1_tag)::value, DUMP = decltype(dump_tag)::value;
#pragma unroll 1
        for (int jb = 0; jb < ntile; jb += UT) {
#pragma unroll
            for (int jj = 0; jj < UT; ++jj) {
                const int j = jb + jj;
                float4_t y = float4_t{0.f, 0.f, 0.f, 0.f};
                int4_t graw = {0, 0, 0, 0}, gsx = {0, 0, 0, 0};
                const int n = 16 * (tile0 + j) + c;
                // y += s * A of a finished group (a step past K adds nothing:
                // its sums are zero and its s is replaced by 0)
                auto end_group = [&](const int4_t &A, float sc, int t, int grp) __attribute__((always_inline)) {
                    if constexpr (DUMP) {   // the exact group sums, for callers that ask
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            const int row = 4 * g + i;
                            if (t < TT && row < mrows && j < ntile && n < N)
                                acc_out[((size_t)(m0 + row) * ng + grp) * N + n] = A[i];
                        }
                    }
                    const float scv = t < TT ? sc : 0.f;
#pragma unroll
                    for (int i = 0; i < 4; ++i) y[i] = fmaf(scv, (float)A[i], y[i]);
                };
                // SP1: a step's group end runs after the next step's MFMAs are
                // issued, so it does not wait for its own MFMAs' results
                int4_t Ap = {0, 0, 0, 0};
                float scp = 0.f;
                int tp = 0;
#pragma unroll
                for (int st = 0; st < S; ++st) {
                    const int slot = (jj * S + st) % D;
                    const int t = wave * S + st;
                    const int grp = SP1 ? t : t >> lsp;
                    const uint32_t szv = sz[min(grp, ng - 1) * SZW + 16 * j + c];
                    int4_t raw = {0, 0, 0, 0};
#pragma unroll
                    for (int v = 0; v < 2; ++v) {
                        int4_t bv;
#pragma unroll
                        for (int e = 0; e < 4; ++e) bv[e] = (int)wka8_dword<BITS>(d[slot], 4 * v + e);
                        raw = __builtin_amdgcn_mfma_i32_16x16x64_i8(a[st][v], bv, raw, 0, 0, 0);
                    }
                    const int zz = wka8_zero<BITS, PGZ>(szv >> 16);
                    const float sc = (float)as_half((uint16_t)(szv & 0xffffu));
                    // refill the slot with the unit D ahead (past the tiles: no load)
                    issue(jb + (jj * S + st + D) / S, (jj * S + st + D) % S, slot);
                    if constexpr (SP1) {
                        if (st > 0) end_group(Ap, scp, tp, tp);
                        Ap = raw - zz * sxg[st];
                        scp = sc;
                        tp = t;
                    } else {
                        // the group's int32 sums A, scaled into y when the group
                        // ends with this step
                        graw += raw;
                        gsx += sxg[st];
                        if (((t + 1) & (sp - 1)) == 0) {
                            end_group(graw - zz * gsx, sc, t, grp);
                            graw = int4_t{0, 0, 0, 0};
                            gsx = int4_t{0, 0, 0, 0};
                        }
                    }
                }
                if constexpr (SP1) end_group(Ap, scp, tp, tp);
                // lane (g, c) of a tile holds rows 4g..4g+3, column c
                *reinterpret_cast<float4_t *>(&red[wave][j][lane][0]) = y;
            }
        }
    };
    if (sp == 1) {
        if (dump) tiles_loop(std::true_type{}, std::true_type{});
        else tiles_loop(std::true_type{}, std::false_type{});
    } else {
        if (dump) tiles_loop(std::false_type{}, std::true_type{});
        else tiles_loop(std::false_type{}, std::false_type{});
    }
    __syncthreads();
    for (int o = threadIdx.x; o < ntile * 256; o += 512) {
        const int j = o >> 8, m = (o >> 4) & 15, col = o & 15;
        const int l = (m >> 2) * 16 + col, i = m & 3;
        float v = 0.f;
#pragma unroll
        for (int w = 0; w < 8; ++w) v += red[w][j][l][i];
        const int n = 16 * (tile0 + j) + col;
        if (m < mrows && n < N) {
            const float sxm = (float)as_half(sx[m0 + m]);
            Y[(size_t)(m0 + m) * N + n] = f32_to_f16_bits(sxm * v);
        }
    }
}

// Weight units in flight per wave (fastest measured on the 8B MLP shape at
// k = 4: 4 against 1, 2 and 8, though within 4 %: 10.6 / 11.0 / 10.6 us at
// 4 / 2 / 8).  k = 8 with at most 4 steps per wave (K <= 4096) takes 2: a unit
// is twice the bytes, and M 16 / 8 / 1 measured 15.7 / 14.8 / 14.3 us with 4
// against 14.7 / 14.1 / 13.9 with 2 (at K 8192, 26.7 against 27.3; k = 5..7
// were slower with 2).
constexpr int W4A8_RING = 4;

template <int BITS, int S, int T, bool PGZ>
static hipError_t w4a8_stream_go(const W4A8Args &a, dim3 grid, int tpw, hipStream_t st)
{
    // a power of two that divides, or is a multiple of, the steps per tile
    constexpr int RING = BITS == 8 && S <= 4 ? 2 : W4A8_RING;
    constexpr int D = S * T < RING ? S * T : RING;
    hipLaunchKernelGGL((w4a8_stream_kernel<BITS, S, T, D, PGZ>), grid, dim3(512), 0, st, a.Xq, a.sx, a.wq, a.s, a.z, a.Y,
                       a.acc, a.M, a.K, a.N, a.G, tpw);
    return hipGetLastError();
}

template <int BITS, int S, bool PGZ>
static hipError_t w4a8_stream_pick_t(const W4A8Args &a, dim3 grid, int tpw, hipStream_t st)
{
    if (tpw <= 1) return w4a8_stream_go<BITS, S, 1, PGZ>(a, grid, tpw, st);
    if (tpw <= 2) return w4a8_stream_go<BITS, S, 2, PGZ>(a, grid, tpw, st);
    if (tpw <= 4) return w4a8_stream_go<BITS, S, 4, PGZ>(a, grid, tpw, st);
    return w4a8_stream_go<BITS, S, 8, PGZ>(a, grid, tpw, st);
}

// Returns hipErrorNotSupported when the shape needs more than 8 steps per wave.
template <int BITS, bool PGZ>
static hipError_t w4a8_stream_launch(const W4A8Args &a, hipStream_t st)
{
    const int TT = a.K / 128, sp = a.G / 128;
    int S = 1;
    while (S < 8 && (S * 8 < TT || S < sp)) S <<= 1;
    if (S * 8 < TT || S < sp) return hipErrorNotSupported;
    const int mtiles = (a.M + 15) / 16;
    if (mtiles > 65535) return hipErrorNotSupported;
    const int tiles = (a.N + 15) / 16;
    int cus = 0, dev = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
        cus = 256;
    const int per_m = std::max(1, cus / mtiles);
    const int tpw = std::min(8, std::max(1, (tiles + per_m - 1) / per_m));   // one batch of tiles per workgroup
    const dim3 grid((unsigned)((tiles + tpw - 1) / tpw), (unsigned)mtiles);
    switch (S) {
        case 1: return w4a8_stream_pick_t<BITS, 1, PGZ>(a, grid, tpw, st);
        case 2: return w4a8_stream_pick_t<BITS, 2, PGZ>(a, grid, tpw, st);
        case 4: return w4a8_stream_pick_t<BITS, 4, PGZ>(a, grid, tpw, st);
        default: return w4a8_stream_pick_t<BITS, 8, PGZ>(a, grid, tpw, st);
    }
}

// ---------------------------------------------------------------------------
// Prefill-sized products, k <= 7: the fp16 GEMM's tiling on the int8 MFMA.
// Workgroup tile 128 (M) x 256 (N): 8 waves of 128 x 32 (8 x 2 MFMA tiles),
// so every weight run is turned into int8 lanes by exactly one lane.  K step
// 128 rows = 4 runs, lane group g owning run 4t + g; the step's X tile (in the
// runs' byte order) and the s and z of the 256 columns are double-buffered in
// LDS; X, s, z and the weight runs are loaded two steps ahead, into two
// register sets that alternate with the step's parity.
// B carries q - z itself: a run's int8 form plus 128 - z in every byte (no
// carries, as q + 128 - z lies in 1..255 for q, z <= 127), sign bit flipped,
// is q - z as a signed byte.  The MFMA sums over a group are then A of
// BitLLM Sec. 4.4 directly, and the group's end applies y += s * float(A)
// (the deferred dequantisation); Y = fp16(sx * y).
// ---------------------------------------------------------------------------
// X tile in LDS, per K step: run-major, [run g][row][two 16-byte chunks],
// rows XOR-ed with g and the chunk index with bit 2 of the row and bit 0 of
// g.  Chosen by measurement (the SQ_LDS_BANK_CONFLICT counter over a family
// of layouts): neither the A-fragment reads nor the staging writes wait on
// bank conflicts; a row-major tile with a 144-byte pitch conflicts on both.
constexpr int WG_RUNB = 128 * 32;   // bytes of one run's column of the tile
__device__ __forceinline__ int wg_xoff(int row, int run, int q)
{
    return run * WG_RUNB + 32 * (row ^ run) + 16 * (q ^ ((row >> 2) & 1) ^ (run & 1));
}

template <int BITS, int SPG, bool DUMP>
__global__ __launch_bounds__(512) void w4a8_gemm_kernel(const int8_t *__restrict__ Xq, const uint16_t *__restrict__ sx,
                                                        const uint32_t *__restrict__ wq, const uint16_t *__restrict__ s,
                                                        const uint16_t *__restrict__ z, uint16_t *__restrict__ Y,
                                                        int32_t *__restrict__ acc_out, int M, int K, int N, int G,
                                                        int mtiles, int ntiles)
{
    static_assert(BITS >= 1 && BITS <= 7, "q - z must fit a signed byte");
    constexpr int MS = 8, NS = 2;
    // k = 1, 3, 4: a group's y += s * float(A) runs inside the next group's
    // first MFMAs (below); k = 2 and k >= 5 keep it as a phase of its own (the
    // fused form spilled there and measured slower: k 2 69.1 -> 70.8 us,
    // k 7 103 -> 112 at M 2048, K = N = 4096)
    constexpr bool FUSE = BITS <= 4 && BITS != 2;
    __shared__ __attribute__((aligned(16))) uint8_t lds[2][4 * WG_RUNB];
    __shared__ uint16_t ssz[2][2][256];   // [buffer][s, z][column of the tile], fp16 bits
    int mt, nt;
    band_tile(mtiles, ntiles, mt, nt);
    const int m0 = mt * 128, n0 = nt * 256;
    const int tid = threadIdx.x, lane = tid & 63, wave = wave_id();
    const int g = lane >> 4, c = lane & 15;
    const int R = K >> 5, ng = K / G;
    const float ginv = run_group_inv(G);
    const uint32_t run_bytes = 4u * BITS, col_bytes = (uint32_t)R * run_bytes;
    const int mrows = min(128, M - m0);
    const __amdgpu_buffer_rsrc_t xr = make_rsrc(Xq + (size_t)m0 * K, (uint32_t)((size_t)mrows * K));
    const int wn0 = n0 + wave * 32;
    const int wcols = max(0, min(32, N - wn0));
    const __amdgpu_buffer_rsrc_t wr = make_rsrc(wq + (size_t)min(wn0, N) * R * BITS, (uint32_t)wcols * col_bytes);
    // staging: thread t loads the 32 bytes of X row t / 4, run t % 4 of the
    // step, and s (t < 256) or z (t >= 256) of tile column t % 256 (clamped:
    // columns past N stage a valid column's values and are never written)
    const int xrow = tid >> 2, xrun = tid & 3;
    const bool stage_z = tid >= 256, zfill = stage_z && !z;   // zfill: stage the default z, 2^(k-1)
    const uint16_t *szp = (stage_z && z ? z : s) + (size_t)min(n0 + (tid & 255), N - 1) * ng;
    const uint16_t zdef = as_u16((_Float16)(float)(1 << (BITS - 1)));

    struct XSet {
        uint32_t x[8];
        uint16_t sz;
    };
    auto load_x = [&](int tt, XSet &xs) {
        const int run = 4 * tt + xrun;
        const uint32_t off = run < R ? (uint32_t)xrow * (uint32_t)K + (uint32_t)run * 32u : W_OOB;
        load_dwords<LOAD_DEFAULT>(xr, off, xs.x, 8);
        xs.sz = szp[min(run_group(4 * tt, ginv), ng - 1)];
    };
    auto store_x = [&](int buf, const XSet &xs) {
        uint8_t *dst = &lds[buf][0];
        int4_t v0, v1;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            v0[e] = (int)wka8_xdword<BITS>(xs.x, e);
            v1[e] = (int)wka8_xdword<BITS>(xs.x, 4 + e);
        }
        *reinterpret_cast<int4_t *>(dst + wg_xoff(xrow, xrun, 0)) = v0;
        *reinterpret_cast<int4_t *>(dst + wg_xoff(xrow, xrun, 1)) = v1;
        ssz[buf][tid >> 8][tid & 255] = zfill ? zdef : xs.sz;
    };
    auto load_w = [&](int tt, uint32_t (&d)[NS][BITS]) {
        const int run = 4 * tt + g;
#pragma unroll
        for (int ns = 0; ns < NS; ++ns) {
            const uint32_t off = run < R ? (uint32_t)(ns * 16 + c) * col_bytes + (uint32_t)run * run_bytes : W_OOB;
            load_dwords<LOAD_STREAM>(wr, off, d[ns], BITS);
        }
    };

    float y[MS][NS][4];
    int4_t acc[MS][NS];   // the current group's sums
#pragma unroll
    for (int i = 0; i < MS; ++i)
#pragma unroll
        for (int j = 0; j < NS; ++j)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                y[i][j][e] = 0.f;
                acc[i][j][e] = 0;
            }
    // s of the group whose sums acc holds (FUSE: 0 before the first group,
    // whose "previous group" then adds nothing)
    float sc[NS] = {0.f, 0.f};

    XSet xa, xb;
    uint32_t wa[NS][BITS], wb[NS][BITS];
    load_x(0, xa);
    load_w(0, wa);
    store_x(0, xa);
    load_x(1, xa);
    load_w(1, wb);
    load_x(2, xb);
    __syncthreads();
    // lane (g, c) reads rows c + 16 ms of run g (16 ms leaves the XOR terms alone)
    const uint8_t *abase0[2] = {&lds[0][wg_xoff(c, g, 0)], &lds[0][wg_xoff(c, g, 1)]};

    // y += s * float(A) of a finished group, for MFMA tile (ms, ns) (and the
    // sums written out when asked for)
    auto add_group = [&](int gi, int ms, int ns) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            y[ms][ns][i] = fmaf(sc[ns], (float)acc[ms][ns][i], y[ms][ns][i]);
            if constexpr (DUMP) {
                const int row = m0 + ms * 16 + 4 * g + i, col = wn0 + ns * 16 + c;
                if (gi >= 0 && row < M && col < N) acc_out[((size_t)row * ng + gi) * N + col] = acc[ms][ns][i];
            }
        }
    };
    // step tt: xin holds X(tt + 1), w the runs of step tt; afterwards they
    // receive X(tt + 3) and the runs of step tt + 2.  sched_barriers keep the
    // two steps of an iteration apart (their registers would otherwise be live
    // together), and the empty asm statements keep everything computed from
    // loaded values at its point of use (moved into the previous step, it
    // would wait there for loads still in flight).  FUSE: the first step of
    // group gi adds group gi - 1's sums to y tile by tile just before the MFMA
    // that starts the tile's new sum, and scheduling groups interleave that
    // VALU work with the MFMAs, so it runs beside the matrix core (as a phase
    // of its own after a group's last MFMAs it is more than half of the
    // loop's VALU instructions at G = 128).  M 2048, K = N = 4096, k 4:
    // 66.2 -> 61.0 us (k 3: 77.0 -> 74.3, k 1: 69.0 -> 66.9; M 1024, k 4:
    // 60.1 -> 54.7), Y bitwise the same.
    auto step = [&](int tt, int gi, bool first, XSet &xin, uint32_t (&w)[NS][BITS]) __attribute__((always_inline)) {
        float scn[NS];
        const int cur = tt & 1;
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int ns = 0; ns < NS; ++ns)
#pragma unroll
            for (int b = 0; b < BITS; ++b) asm volatile("" : "+v"(w[ns][b]));
        int4_t bv[NS][2];
#pragma unroll
        for (int ns = 0; ns < NS; ++ns) {
            const int col = wave * 32 + ns * 16 + c;
            const int zq = (int)(float)as_half(ssz[cur][1][col]);
            const uint32_t cz = (uint32_t)(128 - zq) * 0x01010101u;
#pragma unroll
            for (int v = 0; v < 2; ++v)
#pragma unroll
                for (int e = 0; e < 4; ++e) bv[ns][v][e] = (int)((wka8_dword<BITS>(w[ns], 4 * v + e) + cz) ^ 0x80808080u);
            if (first) scn[ns] = (float)as_half(ssz[cur][0][col]);
        }
        load_w(tt + 2, w);
        const int bufoff = cur * (4 * WG_RUNB);
#pragma unroll
        for (int v = 0; v < 2; ++v) {
            int4_t a[MS];
#pragma unroll
            for (int ms = 0; ms < MS; ++ms) a[ms] = *reinterpret_cast<const int4_t *>(abase0[v] + bufoff + ms * 16 * 32);
#pragma unroll
            for (int ns = 0; ns < NS; ++ns)
#pragma unroll
                for (int ms = 0; ms < MS; ++ms) {
                    const int4_t zero4 = {0, 0, 0, 0};
                    if (FUSE && first && v == 0) add_group(gi - 1, ms, ns);
                    acc[ms][ns] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a[ms], bv[ns][v],
                                                                        (first && v == 0) ? zero4 : acc[ms][ns], 0, 0, 0);
                }
        }
        if (FUSE && first) {
            // the dequantisation's VALU first, then one MFMA per 8 VALU
            // (a tile's 4 conversions and 4 fmas), then the second half's MFMAs
            __builtin_amdgcn_sched_group_barrier(0x002, 40, 0);
#pragma unroll
            for (int i = 0; i < MS * NS; ++i) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x002, 8, 0);
            }
            __builtin_amdgcn_sched_group_barrier(0x008, MS * NS, 0);
        }
        if (first) {
#pragma unroll
            for (int ns = 0; ns < NS; ++ns) sc[ns] = scn[ns];
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int q = 0; q < 8; ++q) asm volatile("" : "+v"(xin.x[q]));
        asm volatile("" : "+v"(xin.sz));
        store_x(cur ^ 1, xin);
        load_x(tt + 3, xin);
        __syncthreads();
        __builtin_amdgcn_sched_barrier(0);
    };
    // a group of SPG steps; step tt uses register set A when tt is even
    auto group = [&](int gi, bool odd) __attribute__((always_inline)) {
#pragma unroll
        for (int j = 0; j < SPG; ++j) {
            if (((j & 1) != 0) == odd) step(gi * SPG + j, gi, j == 0, xa, wa);
            else step(gi * SPG + j, gi, j == 0, xb, wb);
        }
        if constexpr (!FUSE) {
#pragma unroll
            for (int ms = 0; ms < MS; ++ms)
#pragma unroll
                for (int ns = 0; ns < NS; ++ns) add_group(gi, ms, ns);
        }
    };
    if constexpr (SPG == 1) {
        int gi = 0;
        for (; gi + 1 < ng; gi += 2) {
            group(gi, false);
            group(gi + 1, true);
        }
        if (gi < ng) group(gi, false);
    } else {
        for (int gi = 0; gi < ng; ++gi) group(gi, false);
    }
    if constexpr (FUSE) {   // the last group's sums
#pragma unroll
        for (int ms = 0; ms < MS; ++ms)
#pragma unroll
            for (int ns = 0; ns < NS; ++ns) add_group(ng - 1, ms, ns);
    }

#pragma unroll
    for (int ms = 0; ms < MS; ++ms)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int row = m0 + ms * 16 + 4 * g + i;
            if (row >= M) continue;
            const float sxm = (float)as_half(sx[row]);
#pragma unroll
            for (int ns = 0; ns < NS; ++ns) {
                const int col = wn0 + ns * 16 + c;
                if (col < N) Y[(size_t)row * N + col] = f32_to_f16_bits(sxm * y[ms][ns][i]);
            }
        }
}

template <int BITS, int SPG>
static hipError_t w4a8_gemm_go(const W4A8Args &a, hipStream_t st)
{
    const int mtiles = (a.M + 127) / 128, ntiles = (a.N + 255) / 256;
    const dim3 grid((unsigned)(mtiles * ntiles)), block(512);
    if (a.acc)
        hipLaunchKernelGGL((w4a8_gemm_kernel<BITS, SPG, true>), grid, block, 0, st, a.Xq, a.sx, a.wq, a.s, a.z, a.Y, a.acc,
                           a.M, a.K, a.N, a.G, mtiles, ntiles);
    else
        hipLaunchKernelGGL((w4a8_gemm_kernel<BITS, SPG, false>), grid, block, 0, st, a.Xq, a.sx, a.wq, a.s, a.z, a.Y,
                           a.acc, a.M, a.K, a.N, a.G, mtiles, ntiles);
    return hipGetLastError();
}

template <int BITS>
static hipError_t w4a8_gemm_launch(const W4A8Args &a, hipStream_t st)
{
    switch (a.G) {
        case 128: return w4a8_gemm_go<BITS, 1>(a, st);
        case 256: return w4a8_gemm_go<BITS, 2>(a, st);
        case 512: return w4a8_gemm_go<BITS, 4>(a, st);
        case 1024: return w4a8_gemm_go<BITS, 8>(a, st);
        default: return hipErrorNotSupported;
    }
}

static int w4a8_cus()
{
    static int cus = 0;
    if (cus == 0) {
        int dev = 0, v = 0;
        cus = (hipGetDevice(&dev) == hipSuccess &&
               hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && v > 0) ? v : 256;
    }
    return cus;
}

// The tiled kernel when its estimated time is below the streaming kernel's.
// Both estimates are measured on this GPU (K = 4096, k = 4): a workgroup of
// the tiled kernel needs about 1.65 us per 128-row step, so a product takes
// that times the K steps times the rounds of workgroups over the CUs; the
// streaming kernel about 6.8e-9 us per multiply-add (it re-reads the weights
// for every 16 rows).
static bool w4a8_prefer_gemm(const W4A8Args &a)
{
    const long long tiles = (long long)((a.M + 127) / 128) * ((a.N + 255) / 256);
    const long long cus = w4a8_cus();
    const double rounds = (double)((tiles + cus - 1) / cus);
    const double t_gemm = rounds * (a.K / 128) * 1.65;
    const double t_stream = (double)a.M * a.N * a.K * 6.8e-9;
    return t_gemm < t_stream;
}

template <int BITS, bool PGZ>
static hipError_t w4a8_go(const W4A8Args &a, int T, int passes, dim3 grid, hipStream_t st)
{
    const dim3 block(512);
#define QMM_W(TV)                                                                                                  \
    hipLaunchKernelGGL((w4a8_kernel<BITS, TV, PGZ>), grid, block, 0, st, a.Xq, a.sx, a.wq, a.s, a.z, a.Y, a.acc, a.M, \
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

template <int BITS>
static hipError_t launch_wka8_bits(const W4A8Args &a, hipStream_t st)
{
    if constexpr (BITS <= 7) {
        if (w4a8_prefer_gemm(a)) return w4a8_gemm_launch<BITS>(a, st);
    }
    if (a.K <= 8192 && (size_t)a.N * (a.K / 32) * 4 * BITS < 0x7fffffffu) {
        const hipError_t e = a.z ? w4a8_stream_launch<BITS, true>(a, st) : w4a8_stream_launch<BITS, false>(a, st);
        if (e != hipErrorNotSupported) return e;
    }
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
    return a.z ? w4a8_go<BITS, true>(a, T, passes, grid, st) : w4a8_go<BITS, false>(a, T, passes, grid, st);
}

// Returns hipErrorNotSupported for shapes these kernels do not cover.
hipError_t launch_w4a8(const W4A8Args &a, hipStream_t st)
{
    if (a.G % 128 != 0 || a.G > 1024) return hipErrorNotSupported;
    switch (a.bits) {
        case 1: return launch_wka8_bits<1>(a, st);
        case 2: return launch_wka8_bits<2>(a, st);
        case 3: return launch_wka8_bits<3>(a, st);
        case 4: return launch_wka8_bits<4>(a, st);
        case 5: return launch_wka8_bits<5>(a, st);
        case 6: return launch_wka8_bits<6>(a, st);
        case 7: return launch_wka8_bits<7>(a, st);
        case 8: return launch_wka8_bits<8>(a, st);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace qmm
