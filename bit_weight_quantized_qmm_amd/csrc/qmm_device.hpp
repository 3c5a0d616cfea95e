// qmm_device.hpp -- device-side building blocks shared by the gfx950 kernels.
//
// Packed format: column n of Wq is a little-endian bit stream along K; code i
// sits at stream bits [i*k, i*k+k).  Because 32 codes of k bits are exactly k
// dwords, a lane always loads whole "runs" of 32 codes as k dword-aligned
// dwords and unpacks them in registers (no LDS layout conversion).  This is
// the register reinterpretation described on the Tilus verdict page
// (pith.science, arXiv 2504.12984: skeptic critique and referee report on the
// View instruction, Sec. 3.2 / Fig. 2(c)) written out for each k by hand.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qmm {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float float4_t __attribute__((ext_vector_type(4)));
typedef int int4_t __attribute__((ext_vector_type(4)));

// (a & m) | b as one VALU op.  Written out because with two literal constants
// the compiler otherwise emits v_and_b32 + v_or_b32; here the mask goes in an
// SGPR and the OR operand in a VGPR (one constant-bus read, as VOP3 allows).
__device__ __forceinline__ uint32_t qmm_and_or(uint32_t a, uint32_t m, uint32_t b)
{
    uint32_t r;
    asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "s"(m), "v"(b));
    return r;
}

#include "unpack_plan.inc"

__device__ __forceinline__ half2_t as_half2(uint32_t u) { return __builtin_bit_cast(half2_t, u); }
__device__ __forceinline__ uint32_t as_u32(half2_t h) { return __builtin_bit_cast(uint32_t, h); }
__device__ __forceinline__ _Float16 as_half(uint16_t u) { return __builtin_bit_cast(_Float16, u); }
__device__ __forceinline__ uint16_t as_u16(_Float16 h) { return __builtin_bit_cast(uint16_t, h); }

// Exact 2^-p as fp16 for 0 <= p <= 10.
__host__ __device__ constexpr float pow2neg(int p) { return 1.0f / float(1u << p); }

// ---------------------------------------------------------------------------
// Buffer resources: raw buffer loads carry their own range check (lanes whose
// byte offset is past num_records read zeros and never fault), which is how
// ragged column and K tails are handled without divergent branches.
// ---------------------------------------------------------------------------
// Every resource the kernels build is wave-uniform by construction; passing
// base and size through readfirstlane says so to the compiler, which otherwise
// may keep the descriptor in VGPRs and wrap each load in a readfirstlane loop.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t bytes)
{
    const uint64_t p = reinterpret_cast<uint64_t>(base);
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)p);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(p >> 32));
    void *ub = reinterpret_cast<void *>(((uint64_t)hi << 32) | lo);
    const int ubytes = __builtin_amdgcn_readfirstlane((int)bytes);
    return __builtin_amdgcn_make_buffer_rsrc(ub, (short)0, ubytes, 0x00020000);
}

// Cache policy bits for buffer loads: streamed weights are read once.
enum : int { LOAD_DEFAULT = 0, LOAD_STREAM = 2 /* nt */ };

template <int AUX>
__device__ __forceinline__ void load_dwords(__amdgpu_buffer_rsrc_t r, uint32_t off, uint32_t *d, int n)
{
    // n is a compile-time constant after inlining; split into x4/x3/x2/x1 pieces.
    int i = 0;
    for (; i + 4 <= n; i += 4) {
        int4_t v = __builtin_bit_cast(int4_t, __builtin_amdgcn_raw_buffer_load_b128(r, off + 4 * i, 0, AUX));
        d[i] = v[0]; d[i + 1] = v[1]; d[i + 2] = v[2]; d[i + 3] = v[3];
    }
    if (n - i == 3) {
        typedef int int3_t __attribute__((ext_vector_type(3)));
        int3_t v = __builtin_bit_cast(int3_t, __builtin_amdgcn_raw_buffer_load_b96(r, off + 4 * i, 0, AUX));
        d[i] = v[0]; d[i + 1] = v[1]; d[i + 2] = v[2];
    } else if (n - i == 2) {
        typedef int int2_t __attribute__((ext_vector_type(2)));
        int2_t v = __builtin_bit_cast(int2_t, __builtin_amdgcn_raw_buffer_load_b64(r, off + 4 * i, 0, AUX));
        d[i] = v[0]; d[i + 1] = v[1];
    } else if (n - i == 1) {
        d[i] = __builtin_amdgcn_raw_buffer_load_b32(r, off + 4 * i, 0, AUX);
    }
}

// Index of this wave inside its workgroup, as a wave-uniform (SGPR) value.
// Plain threadIdx.x / 64 looks divergent to the compiler; a buffer resource
// built from it would be wrapped in a readfirstlane loop around every load.
__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6)); }

// Index of the group that holds 32-code run r when a group spans gr runs
// (gr = G / 32), i.e. r / gr, without an integer division (which costs about
// 20 VALU instructions): inv = 1 / gr in fp32, then trunc((r + 1/2) inv).
// (r + 1/2) / gr lies at least 1/(2 gr) from any integer, and the fp32
// roundings (a few units in the last place of inv, one of the product) move it
// by at most about (r + 1/2) 2^-21 / gr, less than that for r < 2^20 (run
// indices here stay below 2^16 + 8; checked exhaustively on the host).
__device__ __forceinline__ float run_group_inv(int G) { return 1.0f / (float)(G >> 5); }
__device__ __forceinline__ int run_group(int r, float inv) { return (int)(((float)r + 0.5f) * inv); }

// Tile order of the prefill kernels: workgroup ids go round-robin over the 8
// XCDs, so XCD x gets a contiguous range of the tile sequence; the sequence
// walks bands of TILE_BAND_M M tiles column tile by column tile, so the
// workgroups resident on one XCD share both X row tiles and weight column
// tiles in its L2.
constexpr int TILE_BAND_M = 4;
__device__ __forceinline__ void band_tile(int mtiles, int ntiles, int &mt, int &nt)
{
    const int total = mtiles * ntiles;
    int pid = blockIdx.x;
    if (total % 8 == 0) pid = (blockIdx.x % 8) * (total / 8) + blockIdx.x / 8;
    const int band = pid / (TILE_BAND_M * ntiles);
    const int first = band * TILE_BAND_M;
    const int rows = min(mtiles - first, TILE_BAND_M);
    const int in_band = pid - band * TILE_BAND_M * ntiles;
    mt = first + in_band % rows;
    nt = in_band / rows;
}

// fp32 sum over the 64 lanes of a wave; every lane receives the total.
__device__ __forceinline__ float wave_sum(float v)
{
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) v += __shfl_xor(v, m, 64);
    return v;
}

// Floating-point codes (FMT 1: E2M1 in 4-bit streams, FMT 2: E4M3 in 8-bit
// streams): codes 2j and 2j + 1 of a run d as an fp16 pair holding their exact
// values, by gfx950's packed fp4 / fp8 -> f16 conversions at unit scale (one
// VALU op per pair).  Every E2M1 value and every finite E4M3 value is zero or
// an fp16 normal number.  The byte / word select is an immediate: j must be a
// constant after unrolling.
template <int FMT>
__device__ __forceinline__ half2_t fp_code_pair(const uint32_t *d, int j)
{
    if constexpr (FMT == 1) {   // byte j % 4 of dword j / 4: low nibble first
        const uint32_t w = d[j >> 2];
        switch (j & 3) {
            case 0: return __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 0);
            case 1: return __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 1);
            case 2: return __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 2);
            default: return __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 3);
        }
    } else {                    // 16-bit word j % 2 of dword j / 2: low byte first
        const uint32_t w = d[j >> 1];
        return (j & 1) ? __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, true)
                       : __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, false);
    }
}

// 32 bits of a run's stream starting at bit b (compile-time after unrolling);
// only the low `width` bits are used by the caller.
template <int BITS>
__device__ __forceinline__ uint32_t run_window(const uint32_t (&d)[BITS], int b, int width)
{
    const int i = b >> 5, sh = b & 31;
    if (sh == 0) return d[i];
    if (sh + width <= 32 || i + 1 >= BITS) return d[i] >> sh;
    return __builtin_amdgcn_alignbit(d[i + 1], d[i], (uint32_t)sh);
}

// 3-, 5- and 7-bit float codes (FMT 5: E1M1, 6: E2M2, 7: E3M3) have no
// conversion instruction of their own.  Each code is moved into a container
// format that has one, with the exponent widened by leading zero bits and the
// sign moved to the container's sign bit: E1M1 -> E2M1 nibble, E2M2 -> E5M2
// byte, E3M3 -> E4M3 byte.  Field by field, the container then encodes the
// code's value times 2^(container bias - code bias) (subnormals included:
// both formats put the leading zero exponent at the same place), so the
// converter's scale operand 2^(code bias - container bias) gives the exact
// value: 2, 2^14 and 2^4.  Spreading the k-bit fields to 4- or 8-bit lanes
// takes two mask-and-shift steps (halves, then single codes), the sign move a
// third.
template <int FMT, int BITS>
__device__ __forceinline__ void fp_small_run_to_half2(const uint32_t (&d)[BITS], uint32_t (&h)[16])
{
    if constexpr (FMT == 5) {       // E1M1: 8 codes (24 bits) -> 8 E2M1 nibbles per dword
#pragma unroll
        for (int o = 0; o < 4; ++o) {
            const uint32_t x = run_window<BITS>(d, 24 * o, 24);
            uint32_t t = (x & 0x000fffu) | ((x & 0xfff000u) << 4);
            t = (t & 0x003f003fu) | ((t & 0x0fc00fc0u) << 2);
            t = (t & 0x07070707u) | ((t & 0x38383838u) << 1);
            t = (t & 0x33333333u) | ((t & 0x44444444u) << 1);
            h[4 * o + 0] = as_u32(__builtin_amdgcn_cvt_scalef32_pk_f16_fp4(t, 2.0f, 0));
            h[4 * o + 1] = as_u32(__builtin_amdgcn_cvt_scalef32_pk_f16_fp4(t, 2.0f, 1));
            h[4 * o + 2] = as_u32(__builtin_amdgcn_cvt_scalef32_pk_f16_fp4(t, 2.0f, 2));
            h[4 * o + 3] = as_u32(__builtin_amdgcn_cvt_scalef32_pk_f16_fp4(t, 2.0f, 3));
        }
    } else if constexpr (FMT == 6) {   // E2M2: 4 codes (20 bits) -> 4 E5M2 bytes per dword
#pragma unroll
        for (int o = 0; o < 8; ++o) {
            const uint32_t x = run_window<BITS>(d, 20 * o, 20);
            uint32_t t = (x & 0x003ffu) | ((x & 0xffc00u) << 6);
            t = (t & 0x001f001fu) | ((t & 0x03e003e0u) << 3);
            t = (t & 0x0f0f0f0fu) | ((t & 0x10101010u) << 3);
            h[2 * o + 0] = as_u32(__builtin_amdgcn_cvt_scalef32_pk_f16_bf8(t, 16384.0f, false));
            h[2 * o + 1] = as_u32(__builtin_amdgcn_cvt_scalef32_pk_f16_bf8(t, 16384.0f, true));
        }
    } else {                            // E3M3: 4 codes (28 bits) -> 4 E4M3 bytes per dword
        static_assert(FMT == 7, "float code format");
#pragma unroll
        for (int o = 0; o < 8; ++o) {
            const uint32_t x = run_window<BITS>(d, 28 * o, 28);
            uint32_t t = (x & 0x0003fffu) | ((x & 0xfffc000u) << 2);
            t = (t & 0x007f007fu) | ((t & 0x3f803f80u) << 1);
            t = (t & 0x3f3f3f3fu) | ((t & 0x40404040u) << 1);
            h[2 * o + 0] = as_u32(__builtin_amdgcn_cvt_scalef32_pk_f16_fp8(t, 16.0f, false));
            h[2 * o + 1] = as_u32(__builtin_amdgcn_cvt_scalef32_pk_f16_fp8(t, 16.0f, true));
        }
    }
}

// A whole run of floating-point codes as 16 fp16 pairs (pair p = codes 2p and
// 2p + 1, exact values): per pair for E2M1 / E4M3, one packed conversion of
// all 32 codes for the 6-bit formats (FMT 3: E3M2, 4: E2M3), whose source is
// the run's 6 dwords in stream order, and through a container format for the
// 3-, 5- and 7-bit ones (FMT 5..7).
template <int FMT, int BITS>
__device__ __forceinline__ void fp_run_to_half2(const uint32_t (&d)[BITS], uint32_t (&h)[16])
{
    if constexpr (FMT >= 5) {
        fp_small_run_to_half2<FMT, BITS>(d, h);
    } else if constexpr (FMT == 3 || FMT == 4) {
        static_assert(BITS == 6, "6-bit float codes");
        typedef uint32_t u32x6_t __attribute__((ext_vector_type(6)));
        typedef uint32_t u32x16_t __attribute__((ext_vector_type(16)));
        typedef _Float16 half32_t __attribute__((ext_vector_type(32)));
        const u32x6_t src = {d[0], d[1], d[2], d[3], d[4], d[5]};
        half32_t r;
        if constexpr (FMT == 3)
            r = __builtin_amdgcn_cvt_scalef32_pk32_f16_bf6(src, 1.0f);
        else
            r = __builtin_amdgcn_cvt_scalef32_pk32_f16_fp6(src, 1.0f);
        const u32x16_t w = __builtin_bit_cast(u32x16_t, r);
#pragma unroll
        for (int p = 0; p < 16; ++p) h[p] = w[p];
    } else {
#pragma unroll
        for (int p = 0; p < 16; ++p) h[p] = as_u32(fp_code_pair<FMT>(d, p));
    }
}

// fp32 -> fp16 round to nearest even (v_cvt_f16_f32).
__device__ __forceinline__ uint16_t f32_to_f16_bits(float v) { return as_u16((_Float16)v); }

}  // namespace qmm
