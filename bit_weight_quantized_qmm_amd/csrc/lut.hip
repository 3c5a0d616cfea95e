// lut.hip -- M = 1 product for 1-bit codes by table lookup instead of unpacking.
//
// The table-lookup alternative to unpack-and-multiply that BitLLM's related
// work names for low-bit weights (Sec. 8, T-MAC): four consecutive 1-bit
// codes of a column form a 4-bit index c, and the sum of the four matching
// activations selected by c, T[c] = sum_b bit_b(c) x_(4j+b), is read from a
// table of all 16 subsets built once per workgroup in LDS.  A run of 32 codes
// (one dword) is then 8 lookups and 8 adds instead of 32 multiplies:
//   sum_i x_i q_i  (run)  =  sum_t T_(r,t)[nibble t of the run's dword],
// and the dequantisation of BitLLM Sec. 2.2, eq. (5) is applied per run:
//   y += s_g (sum_i x_i q_i - z_g sum_i x_i).
//
// Table layout: fp32 T[c][t][r] for c = 0..15 (rows of 8 KB), nibble t = 0..7
// of run r = 0..255, so K <= 8192.  Lane l of a wave handles runs l, l + 64,
// ... of its column; at nibble t the 64 lanes read 64 consecutive dwords of
// row c_l (one per run), i.e. 64 different banks whatever their indices c_l,
// and the address is (c_l << 13) | 4 l plus an immediate offset.
#include <algorithm>

#include "launch.hpp"
#include "qmm_device.hpp"

namespace qmm {

constexpr int LUT_ROW = 8192;       // bytes per table row c (2048 fp32 slots)
constexpr int LUT_MAXR = 256;       // runs per column (K <= 8192)

template <int CTRL, int ROWM, int BANKM, bool BC>
__device__ __forceinline__ float lut_dpp_add(float v)
{
    const int t = __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, ROWM, BANKM, BC);
    return v + __builtin_bit_cast(float, t);
}

// Sum over the 64 lanes of a wave with DPP (no LDS round trips); the total
// lands in lane 63.
__device__ __forceinline__ float lut_wave_sum(float v)
{
    v = lut_dpp_add<0xB1, 0xF, 0xF, true>(v);    // quad_perm [1,0,3,2]
    v = lut_dpp_add<0x4E, 0xF, 0xF, true>(v);    // quad_perm [2,3,0,1]
    v = lut_dpp_add<0x141, 0xF, 0xF, true>(v);   // row_half_mirror
    v = lut_dpp_add<0x140, 0xF, 0xF, true>(v);   // row_mirror: every lane holds its row's sum
    v = lut_dpp_add<0x142, 0xA, 0xF, false>(v);  // row_bcast:15 into rows 1 and 3
    v = lut_dpp_add<0x143, 0xC, 0xF, false>(v);  // row_bcast:31 into rows 2 and 3
    return v;
}

// Persistent: one workgroup of 4 waves per CU; wave w of W takes columns
// w, w + W, ... (at most 64) with D columns of loads in flight; lane l owns
// runs l + 64 i, i < RPL.
template <int RPL, int D, bool PGZ>
__global__ __launch_bounds__(256) void lut_m1_kernel(const uint16_t *__restrict__ X, const uint32_t *__restrict__ wq,
                                                     const uint16_t *__restrict__ s, const uint16_t *__restrict__ z,
                                                     uint16_t *__restrict__ Y, int K, int N, int G)
{
    // static LDS (the kernel's only allocation, at address 0): table reads then
    // need no base add, only the VGPR address and an immediate offset
    __shared__ __attribute__((aligned(16))) uint8_t smem[16 * LUT_ROW + 4 * LUT_MAXR];
    float *T = reinterpret_cast<float *>(smem);                          // [16][8][256]
    float *xsum = reinterpret_cast<float *>(smem + 16 * LUT_ROW);        // [LUT_MAXR] per-run sums of x
    const int tid = threadIdx.x, lane = tid & 63, wave = wave_id();
    const int R = K >> 5, ng = K / G;
    const uint32_t col_bytes = (uint32_t)R * 4u;
    const int W = (int)gridDim.x * 4;
    const int w = (int)blockIdx.x * 4 + wave;
    const int ncw = w < N ? (N - 1 - w) / W + 1 : 0;

    // 1. the first D columns' weights and scales go out before the tables are built
    const __amdgpu_buffer_rsrc_t wr = make_rsrc(wq, (uint32_t)min((size_t)N * col_bytes, (size_t)0x7fffffffu));
    const __amdgpu_buffer_rsrc_t sr = make_rsrc(s, (uint32_t)(N * ng * 2));
    const __amdgpu_buffer_rsrc_t zr = make_rsrc(PGZ ? z : s, PGZ ? (uint32_t)(N * ng * 2) : 0u);
    int gi[RPL];
#pragma unroll
    for (int i = 0; i < RPL; ++i) gi[i] = min(((lane + 64 * i) * 32) / G, ng - 1);
    uint32_t d[D][RPL];
    uint16_t sv[D][RPL], zv[D][RPL];
    auto issue = [&](int slot, int i) {
        const uint32_t n = (uint32_t)(w + i * W);
#pragma unroll
        for (int j = 0; j < RPL; ++j) {
            const int r = lane + 64 * j;
            // a run past K reads some other bits of the stream (or zeros past its
            // end); its tables are all zero, so whatever nibbles it holds add nothing
            d[slot][j] = __builtin_amdgcn_raw_buffer_load_b32(wr, n * col_bytes + (uint32_t)r * 4u, 0, 0);
            const uint32_t so = (n * (uint32_t)ng + (uint32_t)gi[j]) * 2u;
            sv[slot][j] = __builtin_amdgcn_raw_buffer_load_b16(sr, so, 0, 0);
            zv[slot][j] = PGZ ? __builtin_amdgcn_raw_buffer_load_b16(zr, so, 0, 0) : (uint16_t)0;
        }
        __builtin_amdgcn_sched_barrier(0);
    };
#pragma unroll
    for (int q = 0; q < D; ++q) issue(q, q);
    __builtin_amdgcn_sched_barrier(0);

    // 2. tables: thread r builds the 8 tables of run r (its 32 activations are
    //    one 64-byte load) and the run's sum of x; consecutive lanes write
    //    consecutive slots of a row (no bank conflicts).  Runs past K get
    //    all-zero tables and zero sums, so whatever codes they meet add nothing.
    const __amdgpu_buffer_rsrc_t xr = make_rsrc(X, (uint32_t)K * 2u);
    {
        const int r = tid;   // 256 threads = LUT_MAXR runs
        uint32_t raw[16];
        load_dwords<LOAD_DEFAULT>(xr, r < R ? (uint32_t)r * 64u : 0x80000000u, raw, 16);
        float xa = 0.f;
#pragma unroll
        for (int t = 0; t < 8; ++t) {
            const half2_t p0 = as_half2(raw[2 * t]), p1 = as_half2(raw[2 * t + 1]);
            const float x0 = (float)p0[0], x1 = (float)p0[1], x2 = (float)p1[0], x3 = (float)p1[1];
            float e[16];
            e[0] = 0.f;
            e[1] = x0;
            e[2] = x1;
            e[3] = x0 + x1;
#pragma unroll
            for (int c = 0; c < 4; ++c) e[4 + c] = x2 + e[c];
#pragma unroll
            for (int c = 0; c < 8; ++c) e[8 + c] = x3 + e[c];
            const int slot = t * LUT_MAXR + r;
#pragma unroll
            for (int c = 0; c < 16; ++c) T[c * (LUT_ROW / 4) + slot] = e[c];
            xa += (x0 + x1) + (x2 + x3);
        }
        xsum[r] = xa;
    }
    __syncthreads();

    float xs[RPL];
#pragma unroll
    for (int j = 0; j < RPL; ++j) xs[j] = xsum[min(lane + 64 * j, LUT_MAXR - 1)];
    const uint32_t base = (uint32_t)lane * 4u;
    const float zdef = 1.0f;   // 2^(k-1) for k = 1

    // 3. stream the wave's columns
    float yout = 0.f;
    for (int i0 = 0; i0 < ncw; i0 += D) {
#pragma unroll
        for (int q = 0; q < D; ++q) {
            const int i = i0 + q;
            // all RPL * 8 reads of the column first, so they are in flight together;
            // the address of nibble t: rotate it to bits 13..16, mask, OR the lane's
            // run offset (two VALU ops), plus an immediate offset for t and the run
            float v[RPL][8];
#pragma unroll
            for (int j = 0; j < RPL; ++j) {
                const uint32_t wv = d[q][j];
                const uint8_t *rowbase = smem + 4 * 64 * j;   // run lane + 64 j: slot t * 256 + r
#pragma unroll
                for (int t = 0; t < 8; ++t) {
                    const uint32_t rot = __builtin_amdgcn_alignbit(wv, wv, (uint32_t)((4 * t + 19) & 31));
                    const uint32_t addr = qmm_and_or(rot, 0x1e000u, base);
                    v[j][t] = *reinterpret_cast<const float *>(rowbase + addr + t * 1024);
                }
            }
            float y = 0.f;
#pragma unroll
            for (int j = 0; j < RPL; ++j) {
                const float a = ((v[j][0] + v[j][1]) + (v[j][2] + v[j][3])) + ((v[j][4] + v[j][5]) + (v[j][6] + v[j][7]));
                const float zz = PGZ ? (float)as_half(zv[q][j]) : zdef;
                y = fmaf((float)as_half(sv[q][j]), fmaf(-zz, xs[j], a), y);
            }
            issue(q, i + D);
            y = lut_wave_sum(y);
            const float tot = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, y), 63));
            if (lane == i) yout = tot;
        }
    }
    if (lane < ncw) Y[w + lane * W] = f32_to_f16_bits(yout);
}

static int lut_cus()
{
    static int cus = 0;
    if (cus == 0) {
        int dev = 0, v = 0;
        cus = (hipGetDevice(&dev) == hipSuccess &&
               hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && v > 0) ? v : 256;
    }
    return cus;
}

template <int RPL, int D, bool PGZ>
static hipError_t lut_go(const GemvArgs &a, int grid, hipStream_t st)
{
    hipLaunchKernelGGL((lut_m1_kernel<RPL, D, PGZ>), dim3(grid), dim3(256), 0, st, a.X, a.wq, a.s, a.z, a.Y, a.K, a.N, a.G);
    return hipGetLastError();
}

// M = 1, 1-bit codes, K <= 8192, at most 64 columns per wave; hipErrorNotSupported otherwise.
hipError_t launch_gemv_lut(const GemvArgs &a, hipStream_t st)
{
    if (a.M != 1 || a.bits != 1 || a.K > 32 * LUT_MAXR) return hipErrorNotSupported;
    const int grid = std::max(1, std::min(lut_cus(), (a.N + 3) / 4));
    if ((a.N + 4 * grid - 1) / (4 * grid) > 64) return hipErrorNotSupported;
    const int R = a.K / 32, rpl = (R + 63) / 64;
    const bool pgz = a.z != nullptr;
#define QMM_LUT(RP, DD) return pgz ? lut_go<RP, DD, true>(a, grid, st) : lut_go<RP, DD, false>(a, grid, st)
    if (rpl <= 1) QMM_LUT(1, 8);
    if (rpl <= 2) QMM_LUT(2, 8);
    QMM_LUT(4, 4);
#undef QMM_LUT
}

}  // namespace qmm
