// gemv.hip -- decode-shaped products Y[M,N] = X[M,K] . dequant(Wq), M <= 16.
//
// Dequantisation follows BitLLM (Sec. 2.2, eq. (5)): w = (q - z) * s with one
// s, z per group of G rows along K.  Codes are unpacked in registers from
// dword-aligned runs (qmm_device.hpp) into fp16 patterns 1024 + q * 2^p; the
// matching activation is pre-scaled by 2^-p, so a dot product with the pattern
// gives sum x*q plus a code-independent bias that is removed once per run.
#include <algorithm>

#include "launch.hpp"
#include "qmm_device.hpp"

namespace qmm {

// ---------------------------------------------------------------------------
// The X side of one run: 32 activations (natural order, two per dword) ->
// 16 half2 in the half-slot order of RunPlan<BITS>, slot s scaled by
// 2^(e - pos[s]).  e is the exponent that brings the activation row's largest
// magnitude into [128, 256) (row_exponent): the row is normalised before the
// 2^-pos scaling, so no activation of normal size goes subnormal in fp16
// however small the row is, the per-128-row sums of the MFMA GEMV stay below
// 2^15, and the caller undoes 2^e on the fp32 result.  The product of the
// two powers of two is formed in fp32 (exact), then each value is rounded
// once to fp16.
// ---------------------------------------------------------------------------
template <int BITS>
__device__ __forceinline__ void x_slots_e(const uint32_t (&xr)[16], half2_t (&xs)[16], int e)
{
    using P = RunPlan<BITS>;
    _Float16 x[32];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const half2_t p = as_half2(xr[i]);
        x[2 * i] = p[0];
        x[2 * i + 1] = p[1];
    }
    // 2^(e - pos) as two fp16 powers of two: 2^a with a = clamp(e - pos, -14, 15),
    // then 2^(e - pos - a), both exact (e <= 29, pos <= 10).  Each product is exact
    // unless it leaves the fp16 normal range, which only activations below 2^-22 of
    // the row maximum can do.
    auto f1 = [&](int pos) { return (_Float16)__builtin_ldexpf(1.0f, min(15, max(-14, e - pos))); };
    auto f2 = [&](int pos) { return (_Float16)__builtin_ldexpf(1.0f, e - pos - min(15, max(-14, e - pos))); };
#pragma unroll
    for (int j = 0; j < 16; ++j) {
        half2_t v, a, b;
        v[0] = x[P::code[2 * j]];
        v[1] = x[P::code[2 * j + 1]];
        a[0] = f1(P::pos[2 * j]);
        a[1] = f1(P::pos[2 * j + 1]);
        b[0] = f2(P::pos[2 * j]);
        b[1] = f2(P::pos[2 * j + 1]);
        xs[j] = (v * a) * b;
    }
}

// The X side without scaling: 32 activations permuted into the slot order,
// for kernels whose B operand is (q - z) s itself.
template <int BITS>
__device__ __forceinline__ void x_perm(const uint32_t (&xr)[16], half2_t (&xs)[16])
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
        xs[j] = v;
    }
}

// Largest |x| of the fp16 values in a run's 16 dwords, as a 15-bit magnitude
// pattern (patterns of finite non-negative fp16 values order like the values).
__device__ __forceinline__ uint32_t run_absmax_bits(const uint32_t (&xr)[16])
{
    uint32_t m = 0;
#pragma unroll
    for (int i = 0; i < 16; ++i) m = max(m, max(xr[i] & 0x7fffu, (xr[i] >> 16) & 0x7fffu));
    return m;
}

template <int CTRL, int ROWM, int BANKM, bool BC>
__device__ __forceinline__ uint32_t dpp_max(uint32_t v)
{
    return max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, ROWM, BANKM, BC));
}

// Maximum over the 64 lanes of a wave (DPP, as wave_sum_dpp), in every lane.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v)
{
    v = dpp_max<0xB1, 0xF, 0xF, true>(v);    // quad_perm [1,0,3,2]
    v = dpp_max<0x4E, 0xF, 0xF, true>(v);    // quad_perm [2,3,0,1]
    v = dpp_max<0x141, 0xF, 0xF, true>(v);   // row_half_mirror
    v = dpp_max<0x140, 0xF, 0xF, true>(v);   // row_mirror
    v = dpp_max<0x142, 0xA, 0xF, false>(v);  // row_bcast:15
    v = dpp_max<0x143, 0xC, 0xF, false>(v);  // row_bcast:31: lane 63 holds the maximum
    return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}

// e such that the row maximum |x| (given as its fp16 magnitude pattern) times
// 2^e lies in [128, 256), at most 29 (a row whose largest value is an fp16
// subnormal below 2^-21 stays below 128); 8 for an all-zero row (any value
// would do).
__device__ __forceinline__ int row_exponent(uint32_t maxbits)
{
    return min(29, 8 - __builtin_amdgcn_frexp_expf((float)as_half((uint16_t)maxbits)));
}

// (1024 * 2^-pos + zc) for both halves of slot pair j: with h = 1024 + q 2^pos,
// h * 2^-pos - that = q - zc exactly in fp16 (all terms are small integers
// or exact powers of two).
template <int BITS>
__device__ __forceinline__ half2_t slot_base(int j, float zc)
{
    using P = RunPlan<BITS>;
    half2_t b;
    b[0] = (_Float16)(1024.0f * pow2neg(P::pos[2 * j]) + zc);
    b[1] = (_Float16)(1024.0f * pow2neg(P::pos[2 * j + 1]) + zc);
    return b;
}

template <int BITS>
__device__ __forceinline__ half2_t slot_pow2neg(int j)
{
    using P = RunPlan<BITS>;
    half2_t b;
    b[0] = (_Float16)pow2neg(P::pos[2 * j]);
    b[1] = (_Float16)pow2neg(P::pos[2 * j + 1]);
    return b;
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
// M = 1: split-K across the 64 lanes of a wave, one 32-code run per lane and
// load, so a wave's load of one column is one contiguous k*256-byte stretch
// (the access pattern of a plain streaming read).  Persistent: one workgroup
// of 4 waves per CU, wave w of W takes columns w, w + W, ... and keeps D
// columns of loads in flight.  Once per workgroup X is staged in LDS in the
// unpack's slot order (scaled by 2^-p) with the per-run bias sums; the X loads
// go out before the weight loads, so the staging overlaps the weight stream.
// Lane l owns runs l, l+64, ... (RPL of them); per run 16 v_dot2_f32_f16 give
// a = sum x'(1024 + q 2^p), and y += s_g * (a - bias).  A DPP reduction
// finishes each column.  Floating-point codes (FMT != 0): X is staged in code
// order without bias sums, the run's pairs come from the packed fp4 / fp6 /
// fp8 conversions (exact values), and y += s_g * a.
// ---------------------------------------------------------------------------
template <int CTRL, int ROWM, int BANKM, bool BC>
__device__ __forceinline__ float dpp_add(float v)
{
    const int s = __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, ROWM, BANKM, BC);
    return v + __builtin_bit_cast(float, s);
}

// Sum over the 64 lanes of a wave; the total lands in lane 63.
__device__ __forceinline__ float wave_sum_dpp(float v)
{
    v = dpp_add<0xB1, 0xF, 0xF, true>(v);    // quad_perm [1,0,3,2]
    v = dpp_add<0x4E, 0xF, 0xF, true>(v);    // quad_perm [2,3,0,1]
    v = dpp_add<0x141, 0xF, 0xF, true>(v);   // row_half_mirror
    v = dpp_add<0x140, 0xF, 0xF, true>(v);   // row_mirror: every lane holds its row's sum
    v = dpp_add<0x142, 0xA, 0xF, false>(v);  // row_bcast:15 into rows 1 and 3
    v = dpp_add<0x143, 0xC, 0xF, false>(v);  // row_bcast:31 into rows 2 and 3
    return v;
}

// The workgroup is number wg of the nwg that share the product's columns
// (the whole grid for qmm_gemv; a slice of it in a grouped launch).
template <int BITS, int RPL, int D, int IPT, bool PGZ, int FMT>
__device__ __forceinline__ void m1_body(const uint16_t *__restrict__ X, const uint32_t *__restrict__ wq,
                                        const uint16_t *__restrict__ s, const uint16_t *__restrict__ z,
                                        uint16_t *__restrict__ Y, int K, int N, int G, int wg, int nwg)
{
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    const int tid = threadIdx.x, lane = tid & 63, wave = wave_id();
    const int R = K >> 5, ng = K / G;
    const uint32_t run_bytes = 4u * BITS, col_bytes = (uint32_t)R * run_bytes;
    // waves sweep the columns together: wave w takes w, w + W, w + 2W, ...
    const int W = nwg * 4;
    const int w = wg * 4 + wave;
    const int ncw = w < N ? (N - 1 - w) / W + 1 : 0;    // columns of this wave (<= 64)

    // LDS: xs [RX] runs x 64 B | 64 B zeros | 64 B dummy | c1 [RX] + 4 | c2 [RX] + 4 (PGZ) | rmax [4].
    // XL (more than 8 runs per lane): X stays in LDS and every lane reads its
    // runs from there for each column; the runs are staged up to 64 RPL (zeros
    // past K), so that each run's address is a base plus a constant.
    constexpr bool XL = RPL > 8;
    const int RX = XL ? 64 * RPL : R;
    const uint32_t xs_bytes = (uint32_t)RX * 64u;
    float *c1 = reinterpret_cast<float *>(smem + xs_bytes + 128);
    float *c2 = c1 + RX + 4;
    uint32_t *rmax = reinterpret_cast<uint32_t *>(c2 + (PGZ ? RX + 4 : 0));

    // 1. activations for the staging (IPT runs per thread)
    const __amdgpu_buffer_rsrc_t xr = make_rsrc(X, (uint32_t)K * 2u);
    uint32_t raw[IPT][16];
#pragma unroll
    for (int i = 0; i < IPT; ++i) {
        const int it = tid + 256 * i;
        load_dwords<LOAD_DEFAULT>(xr, it < R ? (uint32_t)it * 64u : OOB, raw[i], 16);
    }
    __builtin_amdgcn_sched_barrier(0);

    // 2. prefetch the first D columns (weights and per-run scales)
    const __amdgpu_buffer_rsrc_t wr = make_rsrc(wq, (uint32_t)min((size_t)N * col_bytes, (size_t)0x7fffffffu));
    const __amdgpu_buffer_rsrc_t sr = make_rsrc(s, (uint32_t)(N * ng * 2));
    const __amdgpu_buffer_rsrc_t zr = make_rsrc(PGZ ? z : s, PGZ ? (uint32_t)(N * ng * 2) : 0u);
    // Branch-free addressing: a column past N lies past the end of the resource
    // (the load returns zeros), and a run past K reads some other column's bits
    // but meets a zero activation and a zero bias, so it adds nothing.
    int gi[RPL];
    uint32_t roff[RPL];
#pragma unroll
    for (int j = 0; j < RPL; ++j) {
        const int r = lane + 64 * j;
        gi[j] = min((r * 32) / G, ng - 1);
        roff[j] = (uint32_t)r * run_bytes;
    }
    uint32_t d[D][RPL][BITS];
    uint16_t sv[D][RPL], zv[D][RPL];
    auto issue = [&](int slot, int i) {
        const uint32_t n = (uint32_t)(w + i * W);
#pragma unroll
        for (int j = 0; j < RPL; ++j) {
            // default cache policy: the non-temporal hint measured slower here
            // (7B decode k = 6: 9.1 -> 8.0 us; 70B M = 1 k = 5: 31.8 -> 27.1 us)
            load_dwords<LOAD_DEFAULT>(wr, n * col_bytes + roff[j], d[slot][j], BITS);
            const uint32_t so = (n * (uint32_t)ng + (uint32_t)gi[j]) * 2u;
            sv[slot][j] = __builtin_amdgcn_raw_buffer_load_b16(sr, so, 0, 0);
            zv[slot][j] = PGZ ? __builtin_amdgcn_raw_buffer_load_b16(zr, so, 0, 0) : (uint16_t)0;
        }
        __builtin_amdgcn_sched_barrier(0);   // keep slots in issue order (loads complete in order)
    };
    // (with 16 runs per lane the first columns go out after the staging: their
    // 16 k dwords and X's 64 would not fit in the registers together)
    if constexpr (RPL <= 8) {
#pragma unroll
        for (int q = 0; q < D; ++q) issue(q, q);
    }
    __builtin_amdgcn_sched_barrier(0);

    // 3. staging: waves that own items convert X to slot order with bias sums,
    //    the row first normalised by 2^e (x_slots_e); float codes keep X as is
    const float zdef = (float)(1u << (BITS - 1));
#pragma unroll
    for (int i = 0; i < IPT; ++i) asm volatile("" ::"v"(raw[i][0]), "v"(raw[i][15]));   // keep the loads here
    if (tid < 4) reinterpret_cast<int4_t *>(smem + xs_bytes)[tid] = int4_t{0, 0, 0, 0};
    int e = 0;
    if constexpr (FMT == 0) {
        uint32_t mx = 0;
#pragma unroll
        for (int i = 0; i < IPT; ++i) mx = max(mx, run_absmax_bits(raw[i]));   // zeros past K
        mx = wave_max_u32(mx);
        if (lane == 0) rmax[wave] = mx;
        __syncthreads();
        e = row_exponent(max(max(rmax[0], rmax[1]), max(rmax[2], rmax[3])));
    }
#pragma unroll
    for (int i = 0; i < IPT; ++i) {
        if (256 * i + 64 * wave < RX) {              // wave-uniform
            const int it0 = tid + 256 * i;
            const int it = it0 < RX ? it0 : RX;      // RX = the dummy item
            half2_t xs[16];
            float a1 = 0.f, a2 = 0.f;
            if constexpr (FMT != 0) {   // float codes: X in code order, no bias
#pragma unroll
                for (int p = 0; p < 16; ++p) xs[p] = as_half2(raw[i][p]);
            } else {
                x_slots_e<BITS>(raw[i], xs, e);
            }
#pragma unroll
            for (int p = 0; p < 16 && FMT == 0; ++p) {
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
            int4_t *dst = reinterpret_cast<int4_t *>(smem + (it0 < RX ? (uint32_t)it * 64u : xs_bytes + 64u));
            // 16-byte chunk q of item it sits at q ^ (bits 2..3 of it): 16
            // neighbouring lanes then write (and read back) 16 distinct chunk
            // slots instead of 4 (a 4-way LDS bank conflict)
            const int sw = (it0 >> 2) & 3;
#pragma unroll
            for (int q = 0; q < 4; ++q)
                dst[q ^ sw] = int4_t{(int)as_u32(xs[4 * q]), (int)as_u32(xs[4 * q + 1]), (int)as_u32(xs[4 * q + 2]),
                                     (int)as_u32(xs[4 * q + 3])};
            c1[it] = a1;
            if (PGZ) c2[it] = a2;
        }
    }
    __syncthreads();

    if constexpr (RPL > 8) {
#pragma unroll
        for (int q = 0; q < D; ++q) issue(q, q);
    }

    // 4. this lane's activations and bias sums (runs past K read the zero slot):
    //    in VGPRs up to 8 runs per lane; beyond (XL, K up to 32768) they stay
    //    in LDS and are read for every column
    constexpr int RV = XL ? 1 : RPL;
    half2_t xv[RV][16];
    float b1[RV], b2[RV];
    auto run_x = [&](int j, half2_t (&xj)[16], float &bj1, float &bj2) {
        const int r = lane + 64 * j;
        const int4_t *src = reinterpret_cast<const int4_t *>(smem + (r < R ? (uint32_t)r * 64u : xs_bytes));
        const int sw = (r >> 2) & 3;   // the staging's chunk order (the zero slot reads zeros anyway)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int4_t v = src[q ^ sw];
#pragma unroll
            for (int e = 0; e < 4; ++e) xj[4 * q + e] = as_half2((uint32_t)v[e]);
        }
        const int rc = r < R ? r : R;               // c1[R] is written only by the dummy item: mask it
        bj1 = r < R ? c1[rc] : 0.f;
        bj2 = (PGZ && r < R) ? c2[rc] : 0.f;
    };
    if constexpr (!XL) {
#pragma unroll
        for (int j = 0; j < RPL; ++j) run_x(j, xv[j], b1[j], b2[j]);
    }
    // XL: chunk q of this lane's run j at xq[q] + 4096 j (the swizzle depends
    // on bits 2..3 of the run index, the same for every j), its bias sums at
    // c1 / c2 [lane + 64 j]
    const uint8_t *xq[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) xq[q] = smem + (uint32_t)lane * 64u + 16u * (uint32_t)(q ^ ((lane >> 2) & 3));
    auto run_xl = [&](int j, half2_t (&xj)[16], float &bj1, float &bj2) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int4_t v = *reinterpret_cast<const int4_t *>(xq[q] + 4096 * j);
#pragma unroll
            for (int e = 0; e < 4; ++e) xj[4 * q + e] = as_half2((uint32_t)v[e]);
        }
        bj1 = c1[lane + 64 * j];
        bj2 = PGZ ? c2[lane + 64 * j] : 0.f;
    };

    // 5. stream the wave's columns: compute column i while columns i+1..i+D-1 load
    float yout = 0.f;
    for (int i0 = 0; i0 < ncw; i0 += D) {
#pragma unroll
        for (int q = 0; q < D; ++q) {
            const int i = i0 + q;                     // columns past ncw compute on zeros
            {
                float y = 0.f;
                // XL: run j's activations come from LDS, read one run ahead into
                // two alternating register sets; the scheduling barrier at the end
                // of each run keeps the compiler from hoisting all 16 runs' reads
                half2_t xl[2][16];
                float bl1[2] = {0.f, 0.f}, bl2[2] = {0.f, 0.f};
                if constexpr (XL) run_xl(0, xl[0], bl1[0], bl2[0]);
#pragma unroll
                for (int j = 0; j < RPL; ++j) {
                    if constexpr (XL) {
                        if (j + 1 < RPL) run_xl(j + 1, xl[(j + 1) & 1], bl1[(j + 1) & 1], bl2[(j + 1) & 1]);
                    }
                    uint32_t h[16];
                    if constexpr (FMT != 0) {
                        fp_run_to_half2<FMT>(d[q][j], h);
                    } else {
                        run_to_half2<BITS>(d[q][j], h);
                    }
                    const half2_t (&xj)[16] = XL ? xl[j & 1] : xv[XL ? 0 : j];
                    const float bj1 = XL ? bl1[j & 1] : b1[XL ? 0 : j], bj2 = XL ? bl2[j & 1] : b2[XL ? 0 : j];
                    float a = 0.f, a_odd = 0.f;
#pragma unroll
                    for (int p = 0; p < 16; p += 2) {
                        a = __builtin_amdgcn_fdot2(xj[p], as_half2(h[p]), a, false);
                        a_odd = __builtin_amdgcn_fdot2(xj[p + 1], as_half2(h[p + 1]), a_odd, false);
                    }
                    if constexpr (FMT != 0) {   // exact code values: no bias
                        y = fmaf((float)as_half(sv[q][j]), a + a_odd, y);
                    } else {
                        const float bias = PGZ ? fmaf((float)as_half(zv[q][j]), bj2, bj1) : bj1;
                        y = fmaf((float)as_half(sv[q][j]), (a + a_odd) - bias, y);
                    }
                    if constexpr (XL) __builtin_amdgcn_sched_barrier(0);
                }
                issue(q, i + D);                      // refill this slot (zeros past the wave's columns)
                y = wave_sum_dpp(y);
                const float tot = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, y), 63));
                if (lane == i) yout = tot;
            }
        }
    }
    if (lane < ncw) Y[w + lane * W] = f32_to_f16_bits(yout * __builtin_ldexpf(1.0f, -e));
}

template <int BITS, int RPL, int D, int IPT, bool PGZ, int FMT = 0>
__global__ __launch_bounds__(256) void gemv_m1_kernel(const uint16_t *__restrict__ X, const uint32_t *__restrict__ wq,
                                                      const uint16_t *__restrict__ s, const uint16_t *__restrict__ z,
                                                      uint16_t *__restrict__ Y, int K, int N, int G)
{
    m1_body<BITS, RPL, D, IPT, PGZ, FMT>(X, wq, s, z, Y, K, N, G, (int)blockIdx.x, (int)gridDim.x);
}

// Columns in flight per wave for RPL runs per lane (the fastest measured:
// 8 / 4 / 2 / 1 for RPL 1 / 2 / 4 / 8; 4 for RPL 4 at k <= 2, whose columns
// carry few bytes) and items of X staging per thread.
__host__ __device__ constexpr int m1_depth(int bits, int rpl) { return rpl <= 1 ? 8 : rpl == 2 ? 4 : rpl == 4 ? (bits <= 2 ? 4 : 2) : 1; }
__host__ __device__ constexpr int m1_ipt(int rpl) { return rpl == 16 ? 4 : rpl == 12 ? 3 : rpl == 8 ? 2 : 1; }

// Several M = 1 products in one launch (qmm_gemv_grouped): workgroups
// wg0[p] .. wg0[p + 1] - 1 serve problem p, each running the decode body above
// for that problem's code width, so all problems stream at once over their
// own share of the CUs and the launch's start-up and drain are paid once.
template <int RPL>
__global__ __launch_bounds__(256) void gemv_m1_grouped_kernel(const GroupArgs a)
{
    int p = 0;
    while (p + 1 < a.count && (int)blockIdx.x >= a.wg0[p + 1]) ++p;   // wave-uniform
    const GroupProblem g = a.p[p];
    const int wg = (int)blockIdx.x - a.wg0[p], nwg = a.wg0[p + 1] - a.wg0[p];
    constexpr int IPT = m1_ipt(RPL);
#define QMM_GB(B)                                                                                                    \
    case 2 * B:                                                                                                      \
        m1_body<B, RPL, m1_depth(B, RPL), IPT, false, 0>(g.X, g.wq, g.s, g.z, g.Y, a.K, g.N, a.G, wg, nwg);          \
        break;                                                                                                       \
    case 2 * B + 1:                                                                                                  \
        m1_body<B, RPL, m1_depth(B, RPL), IPT, true, 0>(g.X, g.wq, g.s, g.z, g.Y, a.K, g.N, a.G, wg, nwg);           \
        break;
    switch (2 * g.bits + (g.z != nullptr ? 1 : 0)) {
        QMM_GB(1) QMM_GB(2) QMM_GB(3) QMM_GB(4) QMM_GB(5) QMM_GB(6) QMM_GB(7) QMM_GB(8)
        default: break;
    }
#undef QMM_GB
}

// ---------------------------------------------------------------------------
// 2 <= M <= 16 (and M = 1 with very long K): f16 MFMA 16x16x32, M padded to 16.
// A workgroup of 8 waves owns one 16-column tile at a time; the waves split K.
// In a K step of 128 rows, lane group g (lanes 16g..16g+15) owns run 4t+g of
// column (lane % 16): it unpacks the run to fp16 patterns h = 1024 + q 2^p,
// dequantises them in registers to w = (h 2^-p - (1024 2^-p + z)) s = (q - z) s
// (exact difference, one rounding), and feeds four MFMAs.  The A operand holds
// X rows permuted into the same slot order (unscaled) and stays in VGPRs
// across column tiles.  Partial tiles of the 8 waves are summed through LDS in
// a fixed order.
// ---------------------------------------------------------------------------
template <int BITS, int T, bool PGZ>
__global__ __launch_bounds__(512) void gemv_mfma_kernel(const uint16_t *__restrict__ X, const uint32_t *__restrict__ wq,
                                                        const uint16_t *__restrict__ s,
                                                        const uint16_t *__restrict__ z, uint16_t *__restrict__ Y,
                                                        int M, int K, int N, int G, int passes)
{
    __shared__ float red[8][256];
    const int lane = threadIdx.x & 63, wave = wave_id();
    const int g = lane >> 4, c = lane & 15;
    const int R = K >> 5, ng = K / G;
    const float ginv = run_group_inv(G);
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
                const uint32_t soff = (run < R) ? (uint32_t)(c * ng + run_group(run, ginv)) * 2u : OOB;
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
                    x_perm<BITS>(raw, xs);
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
                        // h 2^-pos - (1024 2^-pos + z) = q - z exactly; one rounding multiply by s
                        const half2_t base = PGZ ? slot_base<BITS>(j, 0.f) + z2 : slot_base<BITS>(j, zdef);
                        const half2_t w = (as_half2(h[j]) * slot_pow2neg<BITS>(j) - base) * s2;
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
template <int BITS, int T, int IPT, int SPT, bool G128, bool PGZ>
__global__ __launch_bounds__(512) void gemv_rows_kernel(const uint16_t *__restrict__ X,
                                                         const uint32_t *__restrict__ wq,
                                                         const uint16_t *__restrict__ s,
                                                         const uint16_t *__restrict__ z, uint16_t *__restrict__ Y,
                                                         int M, int K, int N, int G, int ks)
{
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    using P = RunPlan<BITS>;
    const int R = K >> 5, R4 = (R + 3) & ~3, TT = R4 >> 2, ng = K / G;
    const float ginv = run_group_inv(G);
    const int tid = threadIdx.x, lane = tid & 63, wave = wave_id(), nthreads = 64 * ks;
    const int g = lane >> 4, c = lane & 15;
    const int n0 = blockIdx.x * 16;
    const int nvalid = min(16, N - n0);
    const uint32_t run_bytes = 4u * BITS, col_bytes = (uint32_t)R * run_bytes;

    // LDS: xs [M][R4] runs x 64 B | 64 B zeros | 64 B dummy | c1 [M][R4] + 4 dummy |
    //      c2 [M][R4] + 4 dummy (PGZ) | sl [16][ng] + 8 dummy | zl [16][ng] + 8 dummy (PGZ) |
    //      red [ks][4][16] | rmax [4].  Staging threads without an item write the dummy slots, so the
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
    // 2. the tile's scales (and zero-points): 16 contiguous rows of ng halves, loaded
    //    element by element (each 2-byte load is range-checked on its own, so the
    //    ragged last tile reads zeros past its columns and nothing else)
    const uint32_t sbytes = (uint32_t)nvalid * ng * 2u;
    const __amdgpu_buffer_rsrc_t sr = make_rsrc(s + (size_t)n0 * ng, sbytes);
    const __amdgpu_buffer_rsrc_t zr = make_rsrc(PGZ ? z + (size_t)n0 * ng : s, PGZ ? sbytes : 0u);
    uint16_t sraw[SPT], zraw[SPT];
#pragma unroll
    for (int i = 0; i < SPT; ++i) {
        const int si = tid + i * nthreads;
        const uint32_t off = si < 16 * ng ? (uint32_t)si * 2u : OOB;
        sraw[i] = __builtin_amdgcn_raw_buffer_load_b16(sr, off, 0, 0);
        zraw[i] = PGZ ? __builtin_amdgcn_raw_buffer_load_b16(zr, off, 0, 0) : (uint16_t)0;
    }
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
    // 4. per-row maximum |x| (every row normalised by its own 2^e, undone at the end)
    uint32_t *rmax = reinterpret_cast<uint32_t *>(red + ks * 4 * 16);
    if (tid < 4) rmax[tid] = 0u;
    __syncthreads();
#pragma unroll
    for (int i = 0; i < IPT; ++i) {
        const int it0 = tid + i * nthreads;
        atomicMax(&rmax[min(it0 / R4, 3)], it0 < M * R4 ? run_absmax_bits(raw[i]) : 0u);
    }
    __syncthreads();
    // 5. stage X in slot order with its per-run bias sums; scales; zero pad
    const float zdef = (float)(1u << (BITS - 1));
#pragma unroll
    for (int i = 0; i < IPT; ++i) {
        const int it0 = tid + i * nthreads;
        const int it = it0 < M * R4 ? it0 : M * R4;   // M * R4 = the dummy item
        {
            half2_t xs[16];
            x_slots_e<BITS>(raw[i], xs, row_exponent(rmax[min(it0 / R4, M - 1)]));
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
#pragma unroll
    for (int i = 0; i < SPT; ++i) {
        const int si0 = tid + i * nthreads;
        const int si = si0 < 16 * ng ? si0 : 16 * ng;   // 16 * ng = the dummy slot
        sl[si] = sraw[i];
        if (PGZ) zl[si] = zraw[i];
    }
    if (tid < 4) reinterpret_cast<int4_t *>(smem + xs_bytes)[tid] = int4_t{0, 0, 0, 0};
    __syncthreads();

    // 6. K steps: 4 dependent MFMAs per step, the run bias as the accumulator's
    //    start value.  Rule kept throughout: no load is issued while a chain is in
    //    flight.  The LDS operands of step t+1 are read before chain t starts (so
    //    they cannot land in registers chain t still reads), and chain t's result is
    //    consumed before anything of step t+2 is loaded.
    const int r_row = c;                          // MFMA A row held by this lane
    const int am = r_row >> 2, ae = r_row & 3;    // (activation row, run) of that A row
    const bool a_live = (ae == g) && (am < M);
    const int om = g;                             // output rows 4g..4g+3 = (row g, runs 0..3)
    const int omc = min(om, M - 1);
    const int nsteps = max(0, min(T, TT - tt0));

    struct StepOps {
        half8_t a[4];
        float4_t init;
        float sc[4];
    };
    auto load_step = [&](int t, StepOps &o) {
        const int tt = tt0 + t;
        const uint32_t abase = a_live ? ((uint32_t)(am * R4 + 4 * tt + g) * 64u) : xs_bytes;
#pragma unroll
        for (int u = 0; u < 4; ++u) o.a[u] = *reinterpret_cast<const half8_t *>(smem + abase + 16u * u);
        const float4_t cb = *reinterpret_cast<const float4_t *>(c1 + omc * R4 + 4 * tt);
        if (PGZ) {
            const float4_t cz = *reinterpret_cast<const float4_t *>(c2 + omc * R4 + 4 * tt);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int gi = min(run_group(4 * tt + e, ginv), ng - 1);
                o.init[e] = -fmaf((float)as_half(zl[c * ng + gi]), cz[e], cb[e]);
                o.sc[e] = (float)as_half(sl[c * ng + gi]);
            }
        } else {
            o.init = -cb;
            if (G128) {
                o.sc[0] = (float)as_half(sl[c * ng + run_group(4 * tt, ginv)]);
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e) o.sc[e] = (float)as_half(sl[c * ng + min(run_group(4 * tt + e, ginv), ng - 1)]);
            }
        }
        if (PGZ && G128) o.sc[1] = o.sc[2] = o.sc[3] = o.sc[0];
    };

    float y = 0.f;
    StepOps cur, nxt;
    if (nsteps > 0) load_step(0, cur);
#pragma unroll
    for (int t = 0; t < T; ++t) {
        if (t >= nsteps) break;                    // wave-uniform
        if (t + 1 < nsteps) load_step(t + 1, nxt);
        __builtin_amdgcn_sched_barrier(0);
        uint32_t h[16];
        run_to_half2<BITS>(d[t], h);
        // The unpack's v_and_or_b32 is inline asm, which the compiler does not
        // count as a VALU write when it spaces an MFMA that reads the result:
        // fence the unpack off and give the MFMAs explicit wait states.
        __builtin_amdgcn_sched_barrier(0);
        asm volatile("s_nop 7");
        float4_t acc = cur.init;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const half8_t b = __builtin_bit_cast(half8_t, int4_t{(int)h[4 * u], (int)h[4 * u + 1],
                                                                 (int)h[4 * u + 2], (int)h[4 * u + 3]});
            acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(cur.a[u], b, acc, 0, 0, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
        if (G128 && !PGZ) {
            y = fmaf(cur.sc[0], (acc[0] + acc[1]) + (acc[2] + acc[3]), y);
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) y = fmaf(cur.sc[e], acc[e], y);
        }
        __builtin_amdgcn_sched_barrier(0);
        cur = nxt;
    }

    // 7. fixed-order sum over the ks waves, the row's 2^e undone
    if (om < M) red[(wave * 4 + om) * 16 + c] = y;
    __syncthreads();
    if (tid < M * 16) {
        const int m = tid >> 4, cc = tid & 15;
        float v = 0.f;
        for (int w = 0; w < ks; ++w) v += red[(w * 4 + m) * 16 + cc];
        v *= __builtin_ldexpf(1.0f, -row_exponent(rmax[m]));
        if (cc < nvalid) Y[(size_t)m * N + n0 + cc] = f32_to_f16_bits(v);
    }
}

// ---------------------------------------------------------------------------
// Launch selection.
// ---------------------------------------------------------------------------
// ---------------------------------------------------------------------------
// M <= 16 on MFMA, G % 128 == 0, any K (passes of 8192 rows).  One v_mfma_f32_16x16x32_f16 tile
// is 16 rows (X, zero past M) by 16 columns.  The B operand is the raw fp16
// code pattern 1024 + q 2^p of each lane's run (no per-weight arithmetic past
// the unpack); the A operand is X in slot order scaled by 2^-p.  Per 128-row
// step (one group or part of one) the tile's products are
//   acc = sum_k x'_k (1024 + q_k 2^p_k) - 1024 S1 - z S2,
//   S1 = sum_k x'_k,  S2 = sum_k x_k,
// the correction entering as one more MFMA whose A fragment carries S1 and S2
// split into fp16 high and low parts and whose B fragment carries -1024 and
// -z; then y += s * acc (BitLLM Sec. 2.2, eq. (5): w = (q - z) s, factored so
// that the code-independent parts are applied once per step and group).
// Floating-point codes (FMT != 0): A is X in code order and B the codes'
// exact values from the packed fp4 / fp8 conversions; there is no correction.
//
// A workgroup of 8 waves owns tpw <= T consecutive 16-column tiles; in each
// pass of 8 S K steps, wave w owns steps w*S .. w*S + S - 1 of the pass for
// every tile and keeps the A fragments of that K slice in registers.  The s and z of the workgroup's columns are
// staged once in LDS (read along the group index, so every load is a whole
// column's run of groups), which leaves only the weight runs in the per-unit
// stream: units (tile, step) pass through a ring of D weight loads in flight,
// each tile walked front to back along K.  At the end the 8 waves' partial
// tiles are added in LDS and written out.
// ---------------------------------------------------------------------------
static int num_cus();

constexpr int MMA_WAVES = 8;   // waves per workgroup of the M <= 16 MFMA GEMV
constexpr int MMA_MAXNG = 64;  // groups per column and pass: 8192 rows, G >= 128

template <int BITS, int S, int T, int D, bool PGZ, int FMT = 0, bool MP = false>
__global__ __launch_bounds__(64 * MMA_WAVES) void gemv_mma_kernel(const uint16_t *__restrict__ X, const uint32_t *__restrict__ wq,
                                                       const uint16_t *__restrict__ s, const uint16_t *__restrict__ z,
                                                       uint16_t *__restrict__ Y, int M, int K, int N, int G, int tpw)
{
    static_assert(S % D == 0 || D % S == 0, "ring slots must stay compile-time indexes");
    __shared__ float red[MMA_WAVES][T][64][4];
    // s | z << 16 of (group, column) for the workgroup's columns, group-major;
    // the odd row stride keeps the transposing writes free of bank conflicts
    constexpr int SZW = T * 16 + 1;
    __shared__ uint32_t sz[MMA_MAXNG * SZW];
    __shared__ uint32_t rmx[MMA_WAVES][16];   // per wave, per row: max |x| over the wave's K slice
    const int lane = threadIdx.x & 63, wave = wave_id();
    const int g = lane >> 4, c = lane & 15;
    const int R = K >> 5, ng = K / G;
    const float ginv = run_group_inv(G);
    const uint32_t run_bytes = 4u * BITS, col_bytes = (uint32_t)R * run_bytes;
    const int tiles = (N + 15) >> 4;
    const int tile0 = blockIdx.x * tpw;
    const int ntile = min(tpw, tiles - tile0);   // 1 <= ntile <= T

    const __amdgpu_buffer_rsrc_t xr = make_rsrc(X, (uint32_t)(M * K * 2));
    const __amdgpu_buffer_rsrc_t wr = make_rsrc(wq, (uint32_t)((size_t)N * col_bytes));
    const __amdgpu_buffer_rsrc_t sr = make_rsrc(s, (uint32_t)(N * ng * 2));
    const __amdgpu_buffer_rsrc_t zr = make_rsrc(PGZ ? z : s, PGZ ? (uint32_t)(N * ng * 2) : 0u);
    const uint32_t zdef_bits = (uint32_t)as_u16((_Float16)(float)(1u << (BITS - 1)));

    // K in passes of MMA_WAVES * S steps (one pass up to K = 8192 at S = 8):
    // every pass stages its groups' s | z, its X fragments and row exponents,
    // and streams the workgroup's tiles over its K range; each wave adds the
    // pass's tile sums, scaled back to X's units, into its own LDS slots.
    // (MP: more than one pass; the one-pass form keeps the row scaling for the
    // epilogue and spends no registers on it inside the loop)
    const int KS = MMA_WAVES * S, P = MP ? (((R + 3) >> 2) + KS - 1) / KS : 1;
    auto pass_g0 = [&](int pass) { return min(run_group(4 * pass * KS, ginv), ng - 1); };   // first group of a pass

    // s and z of the workgroup's columns: wave w reads columns w, w + 8, ...,
    // lane l holding group g0 + l (past ng, or past the workgroup's columns: zeros)
    constexpr int SZE = T * 16 / MMA_WAVES;
    uint32_t sraw[SZE], zraw[SZE];
    auto load_sz = [&](int g0) {
#pragma unroll
        for (int e = 0; e < SZE; ++e) {
            const int cl = wave + MMA_WAVES * e;
            const uint32_t off = (g0 + lane < ng && cl < 16 * ntile)
                                     ? ((uint32_t)(16 * tile0 + cl) * (uint32_t)ng + (uint32_t)(g0 + lane)) * 2u : OOB;
            sraw[e] = __builtin_amdgcn_raw_buffer_load_b16(sr, off, 0, 0);
            zraw[e] = PGZ ? __builtin_amdgcn_raw_buffer_load_b16(zr, off, 0, 0) : zdef_bits;
        }
    };
    // X run of this lane for step t: row c, run 4 t + g (zeros past M or K)
    auto load_xrun = [&](int t, uint32_t (&raw)[16]) {
        const int run = 4 * t + g;
        load_dwords<LOAD_DEFAULT>(xr, (run < R && c < M) ? ((uint32_t)c * K + (uint32_t)run * 32u) * 2u : OOB, raw, 16);
    };
    uint32_t xa[S][16];   // the wave's X runs of a pass
    auto load_xa = [&](int tb) {
#pragma unroll
        for (int st = 0; st < S; ++st) load_xrun(tb + wave * S + st, xa[st]);
    };
    // MP: a pass's s | z and X loads go out during the previous pass's stream
    if constexpr (MP) {
        load_sz(pass_g0(0));
        load_xa(0);
    }

    for (int pass = 0; pass < P; ++pass) {
    const int tb = pass * KS;                       // first step of the pass
    const int g0 = pass_g0(pass);
    if (pass > 0) __syncthreads();                  // the previous pass's table and row maxima are read
    if constexpr (!MP) {
        // X first: its round trip then overlaps the s | z table's
        load_xa(tb);
        load_sz(g0);
    }

    // weights of unit (tile j, step st) for lane (g, c): column 16 (tile) + c,
    // run 4 t + g of step t = wave * S + st.  Consecutive units walk one column
    // tile through the wave's K slice, so every column is read front to back.
    // A run past K reads other bits of the resource (or zeros past its end)
    // and meets zero activations; units past the workgroup's tiles load nothing.
    uint32_t d[D][BITS];
    auto issue = [&](int j, int st, int slot) {
        const int t = tb + wave * S + st;
        const uint32_t col = (uint32_t)(16 * (tile0 + j) + c);
        // default cache policy: a unit's runs cut cache lines that the wave's next
        // unit reads, and with the non-temporal hint those lines were fetched
        // again (70B MLP-up M = 8, k = 5: 68 -> 42 us)
        load_dwords<LOAD_DEFAULT>(wr, j < ntile ? col * col_bytes + (uint32_t)(4 * t + g) * run_bytes : OOB, d[slot], BITS);
    };
#pragma unroll
    for (int u = 0; u < D; ++u) issue(u / S, u % S, u);

#pragma unroll
    for (int e = 0; e < SZE; ++e) {
        const int cl = wave + MMA_WAVES * e;
        if (g0 + lane < ng) sz[lane * SZW + cl] = (sraw[e] & 0xffffu) | (zraw[e] << 16);
    }

    // A fragments and correction fragments of the wave's K slice, once: they
    // do not depend on the column tile.  Row c is first normalised by 2^e (its
    // maximum |x| over all of K taken across the 8 waves), so S1 and S2 stay
    // below 2^15 and fit the fp16 high part; 2^e is undone on the output.
    half8_t A[S][4];
    uint32_t AC[S][2];   // correction fragment of lane group 0: (S1 hi, S1 lo), (S2 hi, S2 lo)
    {
        int erow = 0;
        if constexpr (FMT == 0) {
            uint32_t mx = 0;
#pragma unroll
            for (int st = 0; st < S; ++st) mx = max(mx, run_absmax_bits(xa[st]));
            mx = max(mx, (uint32_t)__shfl_xor((int)mx, 16));
            mx = max(mx, (uint32_t)__shfl_xor((int)mx, 32));
            if (g == 0) rmx[wave][c] = mx;
        }
        __syncthreads();   // also orders the s | z table writes before the loop's reads
        if constexpr (FMT == 0) {
            uint32_t mx = 0;
#pragma unroll
            for (int w = 0; w < MMA_WAVES; ++w) mx = max(mx, rmx[w][c]);
            erow = row_exponent(mx);
        }
#pragma unroll
        for (int st = 0; st < S; ++st) {
            half2_t xs[16];
            if constexpr (FMT != 0) {   // float codes: X in code order, no correction
#pragma unroll
                for (int p = 0; p < 16; ++p) xs[p] = as_half2(xa[st][p]);
            } else {
                x_slots_e<BITS>(xa[st], xs, erow);
            }
            half2_t one2;
            one2[0] = (_Float16)1.0f;
            one2[1] = (_Float16)1.0f;
            float s1 = 0.f, s2 = 0.f;
#pragma unroll
            for (int p = 0; p < 16 && FMT == 0; ++p) {
                s1 = __builtin_amdgcn_fdot2(xs[p], one2, s1, false);
                s2 = __builtin_amdgcn_fdot2(as_half2(xa[st][p]), one2, s2, false);
            }
#pragma unroll
            for (int u = 0; u < 4; ++u)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    A[st][u][2 * e] = xs[4 * u + e][0];
                    A[st][u][2 * e + 1] = xs[4 * u + e][1];
                }
            // the step's four runs sit in lane groups 0..3 of the same row
            s1 += __shfl_xor(s1, 16);
            s1 += __shfl_xor(s1, 32);
            s2 += __shfl_xor(s2, 16);
            s2 += __shfl_xor(s2, 32);
            s2 = __builtin_ldexpf(s2, erow);   // sum of x 2^e (exact scaling)
            const _Float16 s1h = (_Float16)s1, s2h = (_Float16)s2;
            const _Float16 s1l = (_Float16)(s1 - (float)s1h), s2l = (_Float16)(s2 - (float)s2h);
            half2_t p1, p2;
            p1[0] = s1h;
            p1[1] = s1l;
            p2[0] = s2h;
            p2[1] = s2l;
            AC[st][0] = g == 0 ? as_u32(p1) : 0u;
            AC[st][1] = g == 0 ? as_u32(p2) : 0u;
        }
    }
    // the next pass's s | z and X runs load under this pass's stream (xa, sraw
    // and zraw are free again: the fragments and the table are built)
    if constexpr (MP) {
        if (pass + 1 < P) {
            load_sz(pass_g0(pass + 1));
            load_xa(tb + KS);
        }
    }

    // 2^-e of this lane's output rows 4g..4g+3 in this pass (the rows' X was
    // scaled by 2^e)
    float oscale[4] = {1.f, 1.f, 1.f, 1.f};
    if constexpr (FMT == 0 && MP) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            uint32_t mx = 0;
#pragma unroll
            for (int w = 0; w < MMA_WAVES; ++w) mx = max(mx, rmx[w][4 * g + i]);
            oscale[i] = __builtin_ldexpf(1.0f, -row_exponent(mx));
        }
    }

    // UT tiles per loop iteration keep every ring slot a compile-time index
    constexpr int UT = D > S ? D / S : 1;
#pragma unroll 1
    for (int jb = 0; jb < ntile; jb += UT) {
#pragma unroll
        for (int jj = 0; jj < UT; ++jj) {
            const int j = jb + jj;
            float4_t y = float4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int st = 0; st < S; ++st) {
                const int slot = (jj * S + st) % D;
                const int t = tb + wave * S + st;
                const uint32_t szv = sz[(min(run_group(4 * t, ginv), ng - 1) - g0) * SZW + 16 * j + c];
                uint32_t h[16];
                if constexpr (FMT != 0) {
                    fp_run_to_half2<FMT>(d[slot], h);
                } else {
                    run_to_half2<BITS>(d[slot], h);
                }
                half8_t bc;
                {
                    const _Float16 zero = (_Float16)0.0f;
                    const _Float16 zz = as_half((uint16_t)(szv >> 16));
                    bc[0] = g == 0 ? (_Float16)-1024.0f : zero;
                    bc[1] = bc[0];
                    bc[2] = g == 0 ? (_Float16)(-zz) : zero;
                    bc[3] = bc[2];
                    bc[4] = zero;
                    bc[5] = zero;
                    bc[6] = zero;
                    bc[7] = zero;
                }
                const float sc = (float)as_half((uint16_t)(szv & 0xffffu));
                half8_t b[4];
#pragma unroll
                for (int u = 0; u < 4; ++u)
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const half2_t hh = as_half2(h[4 * u + e]);
                        b[u][2 * e] = hh[0];
                        b[u][2 * e + 1] = hh[1];
                    }
                // The unpack's v_and_or_b32 is inline asm, which the compiler does
                // not count as a VALU write when it spaces an MFMA that reads the
                // result; fence the unpack off and give the MFMAs explicit wait
                // states (k = 7 read stale B operands without them).
                __builtin_amdgcn_sched_barrier(0);
                asm volatile("s_nop 7");
                half8_t ac;
                {
                    const half2_t p1 = as_half2(AC[st][0]), p2 = as_half2(AC[st][1]);
                    const _Float16 zero = (_Float16)0.0f;
                    ac[0] = p1[0];
                    ac[1] = p1[1];
                    ac[2] = p2[0];
                    ac[3] = p2[1];
                    ac[4] = zero;
                    ac[5] = zero;
                    ac[6] = zero;
                    ac[7] = zero;
                }
                float4_t acc = float4_t{0.f, 0.f, 0.f, 0.f};
                if constexpr (FMT == 0) acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(ac, bc, acc, 0, 0, 0);
#pragma unroll
                for (int u = 0; u < 4; ++u) acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(A[st][u], b[u], acc, 0, 0, 0);
                // refill the slot with the unit D ahead (past the tiles: no load)
                issue(jb + (jj * S + st + D) / S, (jj * S + st + D) % S, slot);
#pragma unroll
                for (int i = 0; i < 4; ++i) y[i] = fmaf(sc, acc[i], y[i]);
            }
            // lane (g, c) of a tile holds rows 4g..4g+3, column c
            float4_t *rs = reinterpret_cast<float4_t *>(&red[wave][j][lane][0]);
            if constexpr (MP) {
#pragma unroll
                for (int i = 0; i < 4; ++i) y[i] *= oscale[i];   // exact: powers of two
                *rs = pass == 0 ? y : *rs + y;
            } else {
                *rs = y;
            }
        }
    }
    }   // passes
    // add the 8 waves' partial tiles
    __syncthreads();
    for (int o = threadIdx.x; o < ntile * 256; o += 64 * MMA_WAVES) {
        const int j = o >> 8, m = (o >> 4) & 15, col = o & 15;
        const int l = (m >> 2) * 16 + col, i = m & 3;
        float v = 0.f;
#pragma unroll
        for (int w = 0; w < MMA_WAVES; ++w) v += red[w][j][l][i];
        const int n = 16 * (tile0 + j) + col;
        if constexpr (FMT == 0 && !MP) {   // undo the row's 2^e (one pass)
            uint32_t mx = 0;
#pragma unroll
            for (int w = 0; w < MMA_WAVES; ++w) mx = max(mx, rmx[w][m]);
            v *= __builtin_ldexpf(1.0f, -row_exponent(mx));
        }
        if (m < M && n < N) Y[(size_t)m * N + n] = f32_to_f16_bits(v);
    }
}

// Weight units in flight per wave: a power of two that divides, or is a
// multiple of, the steps per tile.  The depth changes little once s and z come
// from LDS; these are the fastest measured on the 70B MLP-up shape (K 8192,
// N 28672) at M = 8 and 16 (wider codes leave fewer free registers).
__host__ __device__ constexpr int mma_ring(int bits) { return bits <= 3 || bits == 7 ? 8 : bits == 8 ? 2 : 4; }

template <int BITS, int S, int T, bool PGZ, int FMT, bool MP = false>
static hipError_t gemv_mma_go(const GemvArgs &a, int grid, int tpw, hipStream_t st)
{
    // (the pass form holds the next pass's X runs during the stream: at most
    // 4 units in flight there)
    constexpr int D0 = MP && mma_ring(BITS) > 4 ? 4 : mma_ring(BITS);
    constexpr int D = D0 < S * T ? D0 : S * T;
    hipLaunchKernelGGL((gemv_mma_kernel<BITS, S, T, D, PGZ, FMT, MP>), dim3(grid), dim3(64 * MMA_WAVES), 0, st, a.X, a.wq, a.s, a.z, a.Y,
                       a.M, a.K, a.N, a.G, tpw);
    return hipGetLastError();
}

template <int BITS, int S, bool PGZ, int FMT>
static hipError_t gemv_mma_pick_t(const GemvArgs &a, int grid, int tpw, hipStream_t st)
{
    if (tpw <= 1) return gemv_mma_go<BITS, S, 1, PGZ, FMT>(a, grid, tpw, st);
    if (tpw <= 2) return gemv_mma_go<BITS, S, 2, PGZ, FMT>(a, grid, tpw, st);
    if (tpw <= 4) return gemv_mma_go<BITS, S, 4, PGZ, FMT>(a, grid, tpw, st);
    return gemv_mma_go<BITS, S, 8, PGZ, FMT>(a, grid, tpw, st);
}

// Requires G % 128 == 0.  One pass up to K = 8192 (8 waves x 8 steps of 128
// rows); beyond, passes of 4096 rows (4 steps per wave: the pass form's
// registers at 8 steps per wave spill).  One batch of at most 8 tiles per
// workgroup; past 8 x (CU count) tiles the workgroups run in several rounds.
template <int BITS, bool PGZ, int FMT = 0>
static hipError_t gemv_mma_launch(const GemvArgs &a, hipStream_t st)
{
    const int TT = (a.K / 32 + 3) / 4;                   // 128-row steps
    const int steps = (TT + MMA_WAVES - 1) / MMA_WAVES;  // per wave
    const int tiles = (a.N + 15) / 16;
    const int tpw = std::min(8, std::max(1, (tiles + num_cus() - 1) / num_cus()));
    const int grid = (tiles + tpw - 1) / tpw;
    if (steps > 8) {   // the pass form: at most 4 tiles per workgroup (its registers)
        if (tpw <= 2) return gemv_mma_go<BITS, 4, 2, PGZ, FMT, true>(a, grid, tpw, st);
        const int tpw4 = std::min(tpw, 4);
        return gemv_mma_go<BITS, 4, 4, PGZ, FMT, true>(a, (tiles + tpw4 - 1) / tpw4, tpw4, st);
    }
    if (steps <= 1) return gemv_mma_pick_t<BITS, 1, PGZ, FMT>(a, grid, tpw, st);
    if (steps <= 2) return gemv_mma_pick_t<BITS, 2, PGZ, FMT>(a, grid, tpw, st);
    if (steps <= 4) return gemv_mma_pick_t<BITS, 4, PGZ, FMT>(a, grid, tpw, st);
    return gemv_mma_pick_t<BITS, 8, PGZ, FMT>(a, grid, tpw, st);
}

static size_t m1_lds_bytes(int K, bool pgz)
{
    const int R = K / 32;
    return (size_t)R * 64 + 128 + 4u * (size_t)(R + 4) * (pgz ? 2 : 1) + 16;
}

// Workgroups for the M = 1 stream: one per CU (four waves, one per SIMD),
// fewer when N is small, so every wave has at least one column.
static int num_cus()
{
    static int cus = 0;
    if (cus == 0) {
        int dev = 0, v = 0;
        if (hipGetDevice(&dev) == hipSuccess &&
            hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && v > 0)
            cus = v;
        else
            cus = 256;
    }
    return cus;
}

static int m1_grid(int N) { return std::max(1, std::min(num_cus(), (N + 3) / 4)); }

template <int BITS, int RPL, int D, int IPT, bool PGZ, int FMT = 0>
static hipError_t gemv_m1_go(const GemvArgs &a, hipStream_t st)
{
    static bool attr_set = false;
    if (!attr_set) {
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(&gemv_m1_kernel<BITS, RPL, D, IPT, PGZ, FMT>),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
        if (e != hipSuccess) return e;
        attr_set = true;
    }
    const size_t lds = m1_lds_bytes(RPL > 8 ? 32 * 64 * RPL : a.K, PGZ);   // RPL 16: runs staged up to 64 RPL
    const dim3 block(256), grid(m1_grid(a.N));
    hipLaunchKernelGGL((gemv_m1_kernel<BITS, RPL, D, IPT, PGZ, FMT>), grid, block, lds, st, a.X, a.wq, a.s, a.z, a.Y, a.K,
                       a.N, a.G);
    return hipGetLastError();
}

// M = 1 with K <= 32768 and at most 64 columns per wave: RPL = runs per lane
// (1, 2, 4, 8; 12 and 16 with X read from LDS per column), D = 8 / RPL
// columns in flight per wave (1 beyond 8); 4 for RPL = 4 and
// k <= 2, whose columns carry few bytes (k = 2 on the 70B MLP-up shape: 19.4
// -> 17.2 us; 8 in flight, or two workgroups per CU, measured slower).
template <int BITS, bool PGZ>
static hipError_t gemv_m1_launch(const GemvArgs &a, hipStream_t st)
{
    const int R = a.K / 32;
    const int rpl_need = (R + 63) / 64;
    if (rpl_need <= 1) return gemv_m1_go<BITS, 1, m1_depth(BITS, 1), m1_ipt(1), PGZ>(a, st);
    if (rpl_need <= 2) return gemv_m1_go<BITS, 2, m1_depth(BITS, 2), m1_ipt(2), PGZ>(a, st);
    if (rpl_need <= 4) return gemv_m1_go<BITS, 4, m1_depth(BITS, 4), m1_ipt(4), PGZ>(a, st);
    if (rpl_need <= 8) return gemv_m1_go<BITS, 8, m1_depth(BITS, 8), m1_ipt(8), PGZ>(a, st);
    if (rpl_need <= 12) return gemv_m1_go<BITS, 12, m1_depth(BITS, 12), m1_ipt(12), PGZ>(a, st);
    return gemv_m1_go<BITS, 16, m1_depth(BITS, 16), m1_ipt(16), PGZ>(a, st);
}

// Grouped M = 1 products: the CUs are shared out in proportion to each
// problem's estimated time, N (bits + 3): packed bytes plus a per-code share
// for the unpack and dot products, which make the narrow codes relatively
// costlier (on the 7B MLP shapes at k = 3, 4, 6 this split measured 15.7 us
// against 17.5 us for a split by bytes alone); at least one workgroup each
// and enough that no wave takes more than 64 columns.
template <int RPL>
static hipError_t grouped_go(const GroupArgs &ga, int grid, hipStream_t st)
{
    static bool attr_set = false;
    if (!attr_set) {
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(&gemv_m1_grouped_kernel<RPL>),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
        if (e != hipSuccess) return e;
        attr_set = true;
    }
    hipLaunchKernelGGL((gemv_m1_grouped_kernel<RPL>), dim3(grid), dim3(256), m1_lds_bytes(ga.K, true), st, ga);
    return hipGetLastError();
}

hipError_t launch_gemv_grouped(const GroupArgs &in, hipStream_t st)
{
    GroupArgs ga = in;
    const int n = ga.count, cus = num_cus();
    double cost[QMM_GROUP_MAX], total = 0.0;
    for (int p = 0; p < n; ++p) {
        cost[p] = (double)ga.p[p].N * ((double)ga.p[p].bits + 3.0);
        total += cost[p];
    }
    int nwg[QMM_GROUP_MAX], sum = 0, big = 0;
    for (int p = 0; p < n; ++p) {
        const int need = (ga.p[p].N + 255) / 256;   // 4 waves x at most 64 columns each
        nwg[p] = std::max(need, std::max(1, (int)(cus * cost[p] / total + 0.5)));
        sum += nwg[p];
        if (cost[p] > cost[big]) big = p;
    }
    if (sum > cus) {   // trim the largest share while it keeps its minimum
        const int need = (ga.p[big].N + 255) / 256;
        const int cut = std::min(sum - cus, nwg[big] - std::max(1, need));
        nwg[big] -= cut;
        sum -= cut;
    } else if (sum < cus) {
        nwg[big] += cus - sum;
        sum = cus;
    }
    ga.wg0[0] = 0;
    for (int p = 0; p < n; ++p) ga.wg0[p + 1] = ga.wg0[p] + nwg[p];
    const int rpl = (ga.K / 32 + 63) / 64;
    if (rpl <= 1) return grouped_go<1>(ga, sum, st);
    if (rpl <= 2) return grouped_go<2>(ga, sum, st);
    if (rpl <= 4) return grouped_go<4>(ga, sum, st);
    return grouped_go<8>(ga, sum, st);
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
    return b + (size_t)ks * 4 * 16 * 4 + 16;
}

template <int BITS, int T, int IPT, int SPT, bool G128, bool PGZ>
static hipError_t gemv_rows_go(const GemvArgs &a, int ks, size_t lds, hipStream_t st)
{
    static bool attr_set = false;   // raise the dynamic-LDS limit once per instantiation
    if (!attr_set) {
        hipError_t e =
            hipFuncSetAttribute(reinterpret_cast<const void *>(&gemv_rows_kernel<BITS, T, IPT, SPT, G128, PGZ>),
                                hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
        if (e != hipSuccess) return e;
        attr_set = true;
    }
    const dim3 block(64 * ks), grid((a.N + 15) / 16);
    hipLaunchKernelGGL((gemv_rows_kernel<BITS, T, IPT, SPT, G128, PGZ>), grid, block, lds, st, a.X, a.wq, a.s, a.z,
                       a.Y, a.M, a.K, a.N, a.G, ks);
    return hipGetLastError();
}

template <int BITS, int IPT, bool G128, bool PGZ>
static hipError_t gemv_rows_pick_t(const GemvArgs &a, int T, int ks, size_t lds, hipStream_t st)
{
    switch (T) {
        case 1: return gemv_rows_go<BITS, 1, IPT, 1, G128, PGZ>(a, ks, lds, st);
        case 2: return gemv_rows_go<BITS, 2, IPT, 2, G128, PGZ>(a, ks, lds, st);
        case 4: return gemv_rows_go<BITS, 4, IPT, 4, G128, PGZ>(a, ks, lds, st);
        default: return gemv_rows_go<BITS, 8, IPT, 4, G128, PGZ>(a, ks, lds, st);
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
    if (a.M == 1 && R <= 1024 && (size_t)a.N * R * 4 * BITS < 0x7fffffffu &&
        (a.N + 4 * m1_grid(a.N) - 1) / (4 * m1_grid(a.N)) <= 64)
        return a.z ? gemv_m1_launch<BITS, true>(a, st) : gemv_m1_launch<BITS, false>(a, st);
    if (a.M >= 2 && a.G % 128 == 0 && (size_t)a.N * R * 4 * BITS < 0x7fffffffu)
        return a.z ? gemv_mma_launch<BITS, true>(a, st) : gemv_mma_launch<BITS, false>(a, st);
    if (a.M <= 4) {
        int T = 1;
        while (T < 8 && T < TT) T <<= 1;
        const int ks = (TT + T - 1) / T;
        const size_t lds = rows_lds_bytes(a.M, a.K, a.G, ks, a.z != nullptr);
        const int R4 = (R + 3) & ~3;
        // scales per thread: 16 * ng halves over 64 * ks threads, within the SPT the
        // instantiation for T carries (1, 2, 4, 4 for T = 1, 2, 4, 8; enough for any
        // G at T <= 4 and for G >= 64 at T = 8)
        const int spt_max = T == 1 ? 1 : T == 2 ? 2 : 4;
        if (ks <= 8 && lds <= 160 * 1024 && 16 * (a.K / a.G) <= spt_max * 64 * ks) {
            if (a.M * R4 <= 64 * ks) return gemv_rows_pick<BITS, 1>(a, T, ks, lds, st);
            if (a.M * R4 <= 2 * 64 * ks) return gemv_rows_pick<BITS, 2>(a, T, ks, lds, st);
        }
    }
    return a.z ? gemv_mfma_launch<BITS, true>(a, st) : gemv_mfma_launch<BITS, false>(a, st);
}

// Floating-point codes (FMT 1: E2M1, 2: E4M3, 3: E3M2, 4: E2M3; no zero-point) at M = 1 on the
// decode kernel and at 2 <= M <= 16 on the MFMA GEMV: hipErrorNotSupported
// outside their shapes.
template <int BITS, int FMT>
static hipError_t gemv_small_fp(const GemvArgs &a, hipStream_t st)
{
    const int R = a.K / 32;
    if (a.M >= 2 && a.M <= 16 && a.G % 128 == 0 && (size_t)a.N * R * 4 * BITS < 0x7fffffffu)
        return gemv_mma_launch<BITS, false, FMT>(a, st);
    if (!(a.M == 1 && R <= 512 && (size_t)a.N * R * 4 * BITS < 0x7fffffffu &&
          (a.N + 4 * m1_grid(a.N) - 1) / (4 * m1_grid(a.N)) <= 64))
        return hipErrorNotSupported;
    const int rpl_need = (R + 63) / 64;
    if (rpl_need <= 1) return gemv_m1_go<BITS, 1, 8, 1, false, FMT>(a, st);
    if (rpl_need <= 2) return gemv_m1_go<BITS, 2, 4, 1, false, FMT>(a, st);
    if (rpl_need <= 4) return gemv_m1_go<BITS, 4, 2, 1, false, FMT>(a, st);
    return gemv_m1_go<BITS, 8, 1, 2, false, FMT>(a, st);
}

hipError_t launch_gemv_fp(const GemvArgs &a, int fmt, hipStream_t st)
{
    if (fmt == 0 && a.bits == 4) return gemv_small_fp<4, 1>(a, st);
    if (fmt == 1 && a.bits == 8) return gemv_small_fp<8, 2>(a, st);
    if (fmt == 2 && a.bits == 6) return gemv_small_fp<6, 3>(a, st);
    if (fmt == 3 && a.bits == 6) return gemv_small_fp<6, 4>(a, st);
    if (fmt == 4 && a.bits == 3) return gemv_small_fp<3, 5>(a, st);
    if (fmt == 5 && a.bits == 5) return gemv_small_fp<5, 6>(a, st);
    if (fmt == 6 && a.bits == 7) return gemv_small_fp<7, 7>(a, st);
    return hipErrorInvalidValue;
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
