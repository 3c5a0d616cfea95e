// gemm.hip -- prefill-shaped product Y[M,N] = X[M,K] . dequant(Wq), any M.
//
// f16 MFMA (v_mfma_f32_16x16x32_f16, fp32 accumulation) on weights dequantised
// in registers: each lane unpacks a whole 32-code run of one column into fp16
// patterns h = 1024 + q 2^p and turns them into w = (q - z) s: q - z by an
// exact fp16 step (h 2^-p - (1024 2^-p + z)), then one rounding multiply
// (BitLLM Sec. 2.2, eq. (5), per group).  The X tile goes through LDS,
// double-buffered, permuted into the run's half-slot order (values
// unchanged), so both MFMA operands are plain 16-byte fragments.
//
// Workgroup tile 128 (M) x 256 (N), 8 waves side by side in N, wave tile
// 128 x 32 = 8 x 2 MFMA tiles; products with too few such tiles for the CUs
// take smaller tiles whose waves also split K (2, 4 or 8 parts, summed in LDS
// at the end).  K advances 128 rows per step: lane group g (lanes
// 16g..16g+15) of every MFMA owns run 4t+g.
//
// Floating-point codes (FMT 1: E2M1 in 4-bit streams, FMT 2: E4M3 in 8-bit
// streams, FMT 3 / 4: E3M2 / E2M3 in 6-bit streams; qmm_gemm_fp) keep the
// codes in order, so X is staged unpermuted.  gfx950's packed fp4 / fp8 -> f16
// conversions give two codes' exact values per VALU op, the fp6 one a whole
// run's 32; one multiply applies s (one rounding).
#include "launch.hpp"
#include "qmm_device.hpp"

namespace qmm {

// 32 activations (natural order, two per dword) -> 16 half2 in the
// half-slot order of RunPlan<BITS> (a permutation, no scaling).
template <int BITS>
__device__ __forceinline__ void x_perm_g(const uint32_t (&xr)[16], half2_t (&xs)[16])
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

// X tile in LDS, per K step: run-major, [run g][row][four 16-byte chunks], the
// chunk index XOR-ed with 3g mod 4 and with bits 2..3 of the row.  Chosen by
// measurement (the SQ_LDS_BANK_CONFLICT counter over a family of layouts): with
// it neither the A-fragment reads (16 lanes: rows c .. c + 15 of run g, one
// chunk) nor the staging writes (16 lanes: rows r .. r + 3, runs 0..3) wait on
// bank conflicts, and ds_read_b128 runs at twice the rate of a row-major tile
// with a 272-byte pitch; XOR-ing with g itself leaves the reads 2-way
// conflicted.
constexpr int GEMM_RUNB = 64;   // bytes of one (row, run): 32 codes' activations
__device__ __forceinline__ int gemm_chunk(int row, int run, int q) { return 16 * (q ^ ((3 * run) & 3) ^ ((row >> 2) & 3)); }
constexpr uint32_t GEMM_OOB = 0x80000000u;
// Workgroup tile BM (M) x 16 NS WV (N): WV waves side by side in N, each
// BM x 16 NS = BM/16 x NS MFMA tiles, so every weight run is dequantised by
// exactly one lane.  With 8 waves, two share each SIMD: one wave's
// dequantisation and X staging run while the other's MFMAs issue (the wave's
// accumulators, B fragments and one K slice of A fragments fit in half the
// register file).
template <int BITS, bool PGZ, int FMT, int WV, int NS, int BM, int KP>
__global__ __launch_bounds__(64 * WV) void gemm_kernel(const uint16_t *__restrict__ X, const uint32_t *__restrict__ wq,
                                                   const uint16_t *__restrict__ s, const uint16_t *__restrict__ z,
                                                   uint16_t *__restrict__ Y, int M, int K, int N, int G, int mtiles,
                                                   int ntiles)
{
    using P = RunPlan<BITS>;
    constexpr int CW = WV / KP;                               // waves side by side in N per K part
    constexpr int BN = 16 * NS * CW;   // workgroup columns: CW waves of 16 NS columns
    constexpr int MS = BM / 16;                               // 16-row MFMA tiles per wave
    constexpr int XP = (BM * 4 + 64 * CW - 1) / (64 * CW);   // (row, run) pieces of the X step per thread
    static_assert(WV % KP == 0, "whole waves per K part");
    static_assert((KP - 1) * CW * MS * NS * 64 * 16 <= KP * 2 * BM * 4 * GEMM_RUNB, "partial sums fit the X tiles' LDS");
    __shared__ __attribute__((aligned(16))) uint8_t lds[KP][2][BM * 4 * GEMM_RUNB];

    int mt, nt;
    band_tile(mtiles, ntiles, mt, nt);
    const int m0 = mt * BM, n0 = nt * BN;

    const int tid = threadIdx.x, lane = tid & 63, wave = wave_id();
    const int g = lane >> 4, c = lane & 15;
    const int R = K >> 5, ng = K / G, TT = (R + 3) >> 2;
    // K part kp of the workgroup's waves takes steps kp TS .. kp TS + TS - 1
    // (past the last step every load is out of range and reads zeros)
    const int kp = wave / CW, cw = wave - kp * CW, tp = tid - kp * 64 * CW;
    const int TS = (TT + KP - 1) / KP, t0 = kp * TS;
    const uint32_t run_bytes = 4u * BITS, col_bytes = (uint32_t)R * run_bytes;
    const float zdef = (float)(1u << (BITS - 1));
    const float ginv = run_group_inv(G);

    // X: rows m0.. of the whole K range (rows past M and runs past K read zeros).
    const int mrows = min(BM, M - m0);
    const __amdgpu_buffer_rsrc_t xr = make_rsrc(X + (size_t)m0 * K, (uint32_t)((size_t)mrows * K * 2u));
    // Weights, scales, zero-points of this wave's 16 NS columns.
    const int wn0 = n0 + cw * 16 * NS;
    const int wcols = max(0, min(16 * NS, N - wn0));
    const __amdgpu_buffer_rsrc_t wr = make_rsrc(wq + (size_t)min(wn0, N) * R * BITS, (uint32_t)wcols * col_bytes);
    const __amdgpu_buffer_rsrc_t sr = make_rsrc(s + (size_t)min(wn0, N) * ng, (uint32_t)(wcols * ng * 2));
    const __amdgpu_buffer_rsrc_t zr =
        make_rsrc(PGZ ? z + (size_t)min(wn0, N) * ng : s, PGZ ? (uint32_t)(wcols * ng * 2) : 0u);

    // X staging: BM rows x 4 runs of 64 bytes per step, XP (row, run) pieces per
    // thread, runs fastest (4 lanes load a row's 256 contiguous bytes).
    auto load_x = [&](int tt, uint32_t (&raw)[XP][16]) {
#pragma unroll
        for (int i = 0; i < XP; ++i) {
            const int it = tp + 64 * CW * i;
            const int row = it >> 2, gg = it & 3;
            const int run = 4 * tt + gg;
            const uint32_t off = (run < R && it < BM * 4) ? ((uint32_t)row * K + (uint32_t)run * 32u) * 2u : GEMM_OOB;
            load_dwords<LOAD_DEFAULT>(xr, off, raw[i], 16);
        }
    };
    auto store_x = [&](int buf, const uint32_t (&raw)[XP][16]) {
#pragma unroll
        for (int i = 0; i < XP; ++i) {
            const int it = tp + 64 * CW * i;
            if (it >= BM * 4) break;
            const int row = it >> 2, gg = it & 3;
            half2_t xs[16];
            if constexpr (FMT == 0) {
                x_perm_g<BITS>(raw[i], xs);
            } else {
#pragma unroll
                for (int j = 0; j < 16; ++j) xs[j] = as_half2(raw[i][j]);   // codes in order
            }
            uint8_t *dst = &lds[kp][buf][(gg * BM + row) * GEMM_RUNB];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                int4_t v;
                v[0] = (int)as_u32(xs[4 * q + 0]);
                v[1] = (int)as_u32(xs[4 * q + 1]);
                v[2] = (int)as_u32(xs[4 * q + 2]);
                v[3] = (int)as_u32(xs[4 * q + 3]);
                *reinterpret_cast<int4_t *>(dst + gemm_chunk(row, gg, q)) = v;
            }
        }
    };
    auto load_w = [&](int tt, uint32_t (&d)[NS][BITS], uint16_t (&sv)[NS], uint16_t (&zv)[NS]) {
        const int run = 4 * tt + g;
#pragma unroll
        for (int ns = 0; ns < NS; ++ns) {
            const int col = ns * 16 + c;
            const uint32_t off = (run < R) ? (uint32_t)col * col_bytes + (uint32_t)run * run_bytes : GEMM_OOB;
            load_dwords<LOAD_STREAM>(wr, off, d[ns], BITS);
            const uint32_t soff = (run < R) ? (uint32_t)(col * ng + run_group(run, ginv)) * 2u : GEMM_OOB;
            sv[ns] = __builtin_amdgcn_raw_buffer_load_b16(sr, soff, 0, 0);
            zv[ns] = PGZ ? __builtin_amdgcn_raw_buffer_load_b16(zr, soff, 0, 0) : (uint16_t)0;
        }
    };

    float4_t acc[MS][NS];
#pragma unroll
    for (int i = 0; i < MS; ++i)
#pragma unroll
        for (int j = 0; j < NS; ++j) acc[i][j] = float4_t{0.f, 0.f, 0.f, 0.f};

    // dequantise a step's 4 runs (one per N subtile) into B fragments
    auto dequant = [&](const uint32_t (&d)[NS][BITS], const uint16_t (&sv)[NS], const uint16_t (&zv)[NS],
                       half8_t (&bq)[NS][4]) {
#pragma unroll
        for (int ns = 0; ns < NS; ++ns) {
          if constexpr (FMT != 0) {
            half2_t s2;
            s2[0] = as_half(sv[ns]);
            s2[1] = s2[0];
            uint32_t hf[16];
            fp_run_to_half2<FMT>(d[ns], hf);
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                const half2_t w = as_half2(hf[j]) * s2;   // exact value, one rounding
                bq[ns][j >> 2][2 * (j & 3)] = w[0];
                bq[ns][j >> 2][2 * (j & 3) + 1] = w[1];
            }
          } else {
            uint32_t h[16];
            run_to_half2<BITS>(d[ns], h);
            half2_t s2;
            s2[0] = as_half(sv[ns]);
            s2[1] = s2[0];
            half2_t z2;
            z2[0] = as_half(zv[ns]);
            z2[1] = z2[0];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int j = 4 * u + e;
                    // h = 1024 + q 2^p:  h 2^-p - (1024 2^-p + z) = q - z exactly in
                    // fp16 (small integers and exact powers of two), then one
                    // rounding multiply by s
                    half2_t pinv, base;
                    pinv[0] = (_Float16)pow2neg(P::pos[2 * j]);
                    pinv[1] = (_Float16)pow2neg(P::pos[2 * j + 1]);
                    base[0] = (_Float16)(1024.0f * pow2neg(P::pos[2 * j]) + (PGZ ? 0.0f : zdef));
                    base[1] = (_Float16)(1024.0f * pow2neg(P::pos[2 * j + 1]) + (PGZ ? 0.0f : zdef));
                    if (PGZ) base = base + z2;
                    const half2_t w = (as_half2(h[j]) * pinv - base) * s2;
                    bq[ns][u][2 * e] = w[0];
                    bq[ns][u][2 * e + 1] = w[1];
                }
            }
          }
        }
    };
    // lane (g, c) reads rows c + 16 ms of run g; chunk u of a row lies at a
    // row-dependent slot (the same for every ms: 16 ms leaves bits 2..3 alone)
    const uint8_t *abase0[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) abase0[u] = &lds[kp][0][(g * BM + c) * GEMM_RUNB + gemm_chunk(c, g, u)];
    // per 32-row K slice u: the MS A fragments of the wave's BM rows, then the
    // slice's MFMAs over the column subtiles
    auto mfmas = [&](int cur, const half8_t (&bq)[NS][4]) {
        const int bufoff = cur * (BM * 4 * GEMM_RUNB);
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            half8_t a[MS];
#pragma unroll
            for (int ms = 0; ms < MS; ++ms)
                a[ms] = *reinterpret_cast<const half8_t *>(abase0[u] + bufoff + ms * 16 * GEMM_RUNB);
#pragma unroll
            for (int ns = 0; ns < NS; ++ns)
#pragma unroll
                for (int ms = 0; ms < MS; ++ms) {
                    acc[ms][ns] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[ms], bq[ns][u], acc[ms][ns], 0, 0, 0);
                }
        }
    };

    uint32_t xraw[XP][16];
    uint32_t dcur[NS][BITS], dnext[NS][BITS];
    uint16_t scur[NS], snext[NS], zcur[NS], znext[NS];
    load_x(t0, xraw);
    load_w(t0, dcur, scur, zcur);
    store_x(0, xraw);
    // Nothing stays in flight into the loop: the loop body then starts from the
    // same wait state on every iteration (the waits the compiler inserts for a
    // join of differently-pending paths would otherwise cover the prefetch).
    __builtin_amdgcn_s_waitcnt(0x0070);   // vmcnt(0) lgkmcnt(0)
    __syncthreads();
    for (int tt = 0; tt < TS; ++tt) {
        const int cur = tt & 1;
        // prefetch the part's next step (past the last step every load is out of range: zeros)
        load_x(t0 + tt + 1, xraw);
        load_w(t0 + tt + 1, dnext, snext, znext);
        // issue the prefetch here: the scheduler would otherwise sink it to
        // the end of the step, next to its first use
        __builtin_amdgcn_sched_barrier(0);
        half8_t bq[NS][4];
        dequant(dcur, scur, zcur, bq);
        mfmas(cur, bq);
        // the X permutation waits for this step's prefetch: keep it after the MFMAs
        __builtin_amdgcn_sched_barrier(0);
        store_x(cur ^ 1, xraw);
        __syncthreads();
#pragma unroll
        for (int ns = 0; ns < NS; ++ns) {
#pragma unroll
            for (int b = 0; b < BITS; ++b) dcur[ns][b] = dnext[ns][b];
            scur[ns] = snext[ns];
            zcur[ns] = znext[ns];
        }
    }
    // K parts: parts 1 .. KP - 1 leave their sums in LDS (over the X tiles), part
    // 0 adds them in part order (a fixed order: the result does not depend on
    // timing) and writes Y
    if constexpr (KP > 1) {
        float4_t *red = reinterpret_cast<float4_t *>(&lds[0][0][0]);
        __syncthreads();
        if (kp > 0) {
#pragma unroll
            for (int ms = 0; ms < MS; ++ms)
#pragma unroll
                for (int ns = 0; ns < NS; ++ns) red[((((kp - 1) * CW + cw) * MS + ms) * NS + ns) * 64 + lane] = acc[ms][ns];
        }
        __syncthreads();
        if (kp > 0) return;
#pragma unroll
        for (int q = 1; q < KP; ++q)
#pragma unroll
            for (int ms = 0; ms < MS; ++ms)
#pragma unroll
                for (int ns = 0; ns < NS; ++ns) acc[ms][ns] += red[((((q - 1) * CW + cw) * MS + ms) * NS + ns) * 64 + lane];
    }

    // epilogue: lane (g, c) of MFMA tile (ms, ns) holds rows 4g..4g+3, column c.
#pragma unroll
    for (int ms = 0; ms < MS; ++ms) {
#pragma unroll
        for (int ns = 0; ns < NS; ++ns) {
            const int col = wn0 + ns * 16 + c;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int row = m0 + ms * 16 + 4 * g + i;
                if (row < M && col < N) Y[(size_t)row * N + col] = f32_to_f16_bits(acc[ms][ns][i]);
            }
        }
    }
}

template <int BITS, int FMT, int WV, int NS, int BM, int KP = 1>
static hipError_t gemm_go(const GemvArgs &a, hipStream_t st)
{
    constexpr int BN = 16 * NS * (WV / KP);
    const int mtiles = (a.M + BM - 1) / BM, ntiles = (a.N + BN - 1) / BN;
    const dim3 block(64 * WV), grid((unsigned)(mtiles * ntiles));
    if (FMT == 0 && a.z)
        hipLaunchKernelGGL((gemm_kernel<BITS, true, FMT, WV, NS, BM, KP>), grid, block, 0, st, a.X, a.wq, a.s, a.z, a.Y, a.M,
                           a.K, a.N, a.G, mtiles, ntiles);
    else
        hipLaunchKernelGGL((gemm_kernel<BITS, false, FMT, WV, NS, BM, KP>), grid, block, 0, st, a.X, a.wq, a.s, a.z, a.Y, a.M,
                           a.K, a.N, a.G, mtiles, ntiles);
    return hipGetLastError();
}

static int gemm_cus()
{
    static int cus = 0;
    if (cus == 0) {
        int dev = 0, v = 0;
        cus = (hipGetDevice(&dev) == hipSuccess &&
               hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && v > 0) ? v : 256;
    }
    return cus;
}

// Tile choice.  Each workgroup walks its K range alone, so a grid with fewer
// workgroups than CUs leaves the time of one workgroup's loop for a fraction
// of the work; the candidates go from the largest tile to the smallest, and
// the smaller ones split K among the workgroup's waves (K parts added in LDS
// at the end): 128 x 256 (8 waves of 32 columns), 128 x 128 in 2 K parts,
// 64 x 128 (8 waves of 16 columns), 64 x 64 in 2 parts, 64 x 32 in 4, and
// 32 x 16 in 8 parts.  The first whose grid reaches 4/5 of the CUs is taken,
// else the last.  Measured at K = N = 4096, k 4 (us, without -> with the K
// parts): M 128: 23.7 -> 20.1; M 256: 25.3 -> 25.1; M 1024: 59.2 -> 56.5;
// M 100, N 1000: 22.6 -> 12.6; M 512 and M 2048 keep their tiles.
template <int BITS, int FMT>
static hipError_t gemm_dispatch(const GemvArgs &a, hipStream_t st)
{
    const long long cus = gemm_cus(), need = (4 * cus + 4) / 5;
    auto tiles = [&](int bm, int bn) { return (long long)((a.M + bm - 1) / bm) * ((a.N + bn - 1) / bn); };
    if (tiles(128, 256) >= need) return gemm_go<BITS, FMT, 8, 2, 128, 1>(a, st);
    if (tiles(128, 128) >= need) return gemm_go<BITS, FMT, 8, 2, 128, 2>(a, st);
    if (tiles(64, 128) >= need) return gemm_go<BITS, FMT, 8, 1, 64, 1>(a, st);
    if (tiles(64, 64) >= need) return gemm_go<BITS, FMT, 8, 1, 64, 2>(a, st);
    if (tiles(64, 32) >= need) return gemm_go<BITS, FMT, 8, 1, 64, 4>(a, st);
    return gemm_go<BITS, FMT, 8, 1, 32, 8>(a, st);
}

hipError_t launch_gemm(const GemvArgs &a, hipStream_t st)
{
    switch (a.bits) {
        case 1: return gemm_dispatch<1, 0>(a, st);
        case 2: return gemm_dispatch<2, 0>(a, st);
        case 3: return gemm_dispatch<3, 0>(a, st);
        case 4: return gemm_dispatch<4, 0>(a, st);
        case 5: return gemm_dispatch<5, 0>(a, st);
        case 6: return gemm_dispatch<6, 0>(a, st);
        case 7: return gemm_dispatch<7, 0>(a, st);
        case 8: return gemm_dispatch<8, 0>(a, st);
        default: return hipErrorInvalidValue;
    }
}

// Floating-point codes: fmt 0 = E2M1 (4-bit stream), 1 = E4M3 (8-bit), 2 = E3M2
// and 3 = E2M3 (6-bit), 4 = E1M1 (3-bit), 5 = E2M2 (5-bit), 6 = E3M3 (7-bit);
// a.bits must match, a.z is ignored.
hipError_t launch_gemm_fp(const GemvArgs &a, int fmt, hipStream_t st)
{
    if (fmt == 0 && a.bits == 4) return gemm_dispatch<4, 1>(a, st);
    if (fmt == 1 && a.bits == 8) return gemm_dispatch<8, 2>(a, st);
    if (fmt == 2 && a.bits == 6) return gemm_dispatch<6, 3>(a, st);
    if (fmt == 3 && a.bits == 6) return gemm_dispatch<6, 4>(a, st);
    if (fmt == 4 && a.bits == 3) return gemm_dispatch<3, 5>(a, st);
    if (fmt == 5 && a.bits == 5) return gemm_dispatch<5, 6>(a, st);
    if (fmt == 6 && a.bits == 7) return gemm_dispatch<7, 7>(a, st);
    return hipErrorInvalidValue;
}

}  // namespace qmm
