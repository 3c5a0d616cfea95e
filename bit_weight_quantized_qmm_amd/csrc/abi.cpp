// abi.cpp -- the C ABI declared in include/qmm.h: argument validation (host
// only, before any HIP call), then one launch on the caller's stream.
#include "../../include/qmm.h"

#include <hip/hip_runtime.h>
#include <stdio.h>
#include <string.h>

#include "launch.hpp"

namespace {

thread_local char g_last_error[256] = "";

qmm_status fail(qmm_status st, const char *fmt, const char *what)
{
    snprintf(g_last_error, sizeof g_last_error, fmt, what);
    return st;
}

// Largest sizes the kernels index with 32-bit arithmetic: with K <= 2^21 every
// buffer resource the kernels build (at most 256 rows of X, 64 columns of Wq)
// stays below 2^31 bytes, below the out-of-range offset they use for padding.
constexpr int64_t kMaxK = int64_t(1) << 21;
constexpr int64_t kMaxN = int64_t(1) << 24;
constexpr int64_t kMaxM = int64_t(1) << 24;

qmm_status check_shape(const char *fn, int64_t M, int64_t K, int64_t N, int bits, int64_t G, bool need_g)
{
    if (bits < 1 || bits > 8) return fail(QMM_ERR_INVALID_ARG, "%s: bits must be in 1..8", fn);
    if (K < 32 || K % 32 != 0) return fail(QMM_ERR_INVALID_ARG, "%s: K must be a positive multiple of 32", fn);
    if (N < 1) return fail(QMM_ERR_INVALID_ARG, "%s: N must be >= 1", fn);
    if (M < 1) return fail(QMM_ERR_INVALID_ARG, "%s: M must be >= 1", fn);
    if (need_g && (G < 32 || G % 32 != 0 || K % G != 0))
        return fail(QMM_ERR_INVALID_ARG, "%s: G must be a positive multiple of 32 dividing K", fn);
    if (K > kMaxK || N > kMaxN || M > kMaxM)
        return fail(QMM_ERR_UNSUPPORTED, "%s: dimension beyond the supported range", fn);
    if ((K / 32) * N > (int64_t(1) << 31) - 256)
        return fail(QMM_ERR_UNSUPPORTED, "%s: problem beyond the supported range", fn);
    if (((M + 127) / 128) * ((N + 255) / 256) > (int64_t(1) << 31) - 1)   // GEMM tiles of 128 x 256
        return fail(QMM_ERR_UNSUPPORTED, "%s: problem beyond the supported range", fn);
    return QMM_OK;
}

qmm_status hip_status(hipError_t e, const char *fn)
{
    if (e == hipSuccess) {
        g_last_error[0] = '\0';
        return QMM_OK;
    }
    if (e == hipErrorNotSupported) return fail(QMM_ERR_UNSUPPORTED, "%s: shape not supported by the kernel", fn);
    snprintf(g_last_error, sizeof g_last_error, "%s: %s", fn, hipGetErrorString(e));
    return QMM_ERR_HIP;
}

}  // namespace

extern "C" {

size_t qmm_packed_bytes(int64_t K, int64_t N, int bits)
{
    if (bits < 1 || bits > 8 || K < 0 || N < 0 || (K * bits) % 8 != 0) return 0;
    return (size_t)N * (size_t)K * (size_t)bits / 8u;
}

qmm_status qmm_pack(const uint8_t *codes, uint32_t *wq, int64_t K, int64_t N, int bits, qmm_stream stream)
{
    qmm_status st = check_shape("qmm_pack", 1, K, N, bits, 32, false);
    if (st != QMM_OK) return st;
    if (!codes || !wq) return fail(QMM_ERR_INVALID_ARG, "%s: null pointer", "qmm_pack");
    return hip_status(qmm::launch_pack(codes, wq, (int)K, (int)N, bits, false, (hipStream_t)stream), "qmm_pack");
}

qmm_status qmm_pack_signed(const int8_t *codes, uint32_t *wq, int64_t K, int64_t N, int bits, qmm_stream stream)
{
    const char *fn = "qmm_pack_signed";
    qmm_status st = check_shape(fn, 1, K, N, bits, 32, false);
    if (st != QMM_OK) return st;
    if (!codes || !wq) return fail(QMM_ERR_INVALID_ARG, "%s: null pointer", fn);
    return hip_status(qmm::launch_pack(reinterpret_cast<const uint8_t *>(codes), wq, (int)K, (int)N, bits, true,
                                       (hipStream_t)stream),
                      fn);
}

qmm_status qmm_unpack(const uint32_t *wq, uint8_t *codes, int64_t K, int64_t N, int bits, qmm_stream stream)
{
    qmm_status st = check_shape("qmm_unpack", 1, K, N, bits, 32, false);
    if (st != QMM_OK) return st;
    if (!codes || !wq) return fail(QMM_ERR_INVALID_ARG, "%s: null pointer", "qmm_unpack");
    return hip_status(qmm::launch_unpack(wq, codes, (int)K, (int)N, bits, (hipStream_t)stream), "qmm_unpack");
}

static qmm_status product(const char *fn, bool gemv, const qmm_half *X, const uint32_t *wq, const qmm_half *s,
                          const qmm_half *z, qmm_half *Y, int64_t M, int64_t K, int64_t N, int bits, int64_t G,
                          qmm_stream stream)
{
    qmm_status st = check_shape(fn, M, K, N, bits, G, true);
    if (st != QMM_OK) return st;
    if (gemv && M > 16) return fail(QMM_ERR_INVALID_ARG, "%s: M must be <= 16 (use qmm_gemm)", fn);
    if (!X || !wq || !s || !Y) return fail(QMM_ERR_INVALID_ARG, "%s: null pointer", fn);
    qmm::GemvArgs a{X, wq, s, z, Y, (int)M, (int)K, (int)N, bits, (int)G};
    hipError_t e = gemv ? qmm::launch_gemv(a, (hipStream_t)stream) : qmm::launch_gemm(a, (hipStream_t)stream);
    return hip_status(e, fn);
}

qmm_status qmm_gemv(const qmm_half *X, const uint32_t *wq, const qmm_half *s, const qmm_half *z, qmm_half *Y,
                    int64_t M, int64_t K, int64_t N, int bits, int64_t G, qmm_stream stream)
{
    return product("qmm_gemv", true, X, wq, s, z, Y, M, K, N, bits, G, stream);
}

qmm_status qmm_gemv_grouped(const qmm_gemv_problem *probs, int count, int64_t K, int64_t G, qmm_stream stream)
{
    const char *fn = "qmm_gemv_grouped";
    if (!probs) return fail(QMM_ERR_INVALID_ARG, "%s: null problem array", fn);
    if (count < 1 || count > qmm::QMM_GROUP_MAX) return fail(QMM_ERR_INVALID_ARG, "%s: count must be in 1..16", fn);
    qmm::GroupArgs ga{};
    ga.count = count;
    ga.K = (int)K;
    ga.G = (int)G;
    for (int p = 0; p < count; ++p) {
        const qmm_gemv_problem &q = probs[p];
        qmm_status st = check_shape(fn, 1, K, q.N, q.bits, G, true);
        if (st != QMM_OK) return st;
        if (!q.X || !q.wq || !q.s || !q.Y) return fail(QMM_ERR_INVALID_ARG, "%s: null pointer in a problem", fn);
        if (K > 16384 || (K / 32) * q.N * 4 * (int64_t)q.bits >= (int64_t(1) << 31) - 1)
            return fail(QMM_ERR_UNSUPPORTED, "%s: K <= 16384 and a problem's weights below 2 GiB are supported", fn);
        ga.p[p] = qmm::GroupProblem{q.X, q.wq, q.s, q.z, q.Y, (int)q.N, q.bits};
    }
    return hip_status(qmm::launch_gemv_grouped(ga, (hipStream_t)stream), fn);
}

qmm_status qmm_gemv_lut(const qmm_half *X, const uint32_t *wq, const qmm_half *s, const qmm_half *z, qmm_half *Y,
                        int64_t M, int64_t K, int64_t N, int bits, int64_t G, qmm_stream stream)
{
    const char *fn = "qmm_gemv_lut";
    qmm_status st = check_shape(fn, M, K, N, bits, G, true);
    if (st != QMM_OK) return st;
    if (!X || !wq || !s || !Y) return fail(QMM_ERR_INVALID_ARG, "%s: null pointer", fn);
    if (M != 1 || bits != 1 || K > 8192)
        return fail(QMM_ERR_UNSUPPORTED, "%s: implemented for M = 1, bits = 1, K <= 8192", fn);
    qmm::GemvArgs a{X, wq, s, z, Y, (int)M, (int)K, (int)N, bits, (int)G};
    return hip_status(qmm::launch_gemv_lut(a, (hipStream_t)stream), fn);
}

qmm_status qmm_gemm(const qmm_half *X, const uint32_t *wq, const qmm_half *s, const qmm_half *z, qmm_half *Y,
                    int64_t M, int64_t K, int64_t N, int bits, int64_t G, qmm_stream stream)
{
    return product("qmm_gemm", false, X, wq, s, z, Y, M, K, N, bits, G, stream);
}

qmm_status qmm_gemm_fp(const qmm_half *X, const uint32_t *wq, const qmm_half *s, qmm_half *Y, int64_t M, int64_t K,
                       int64_t N, int fmt, int64_t G, qmm_stream stream)
{
    const char *fn = "qmm_gemm_fp";
    static const int kBits[] = {4, 8, 6, 6, 3, 5, 7};   // by format id (qmm.h)
    if (fmt < QMM_FP4_E2M1 || fmt > QMM_FP7_E3M3) return fail(QMM_ERR_INVALID_ARG, "%s: unknown code format", fn);
    const int bits = kBits[fmt];
    qmm_status st = check_shape(fn, M, K, N, bits, G, true);
    if (st != QMM_OK) return st;
    if (!X || !wq || !s || !Y) return fail(QMM_ERR_INVALID_ARG, "%s: null pointer", fn);
    qmm::GemvArgs a{X, wq, s, nullptr, Y, (int)M, (int)K, (int)N, bits, (int)G};
    const int f = fmt;   // 0 E2M1, 1 E4M3, 2 E3M2, 3 E2M3, 4 E1M1, 5 E2M2, 6 E3M3
    if (M <= 16) {   // the decode kernels where they take the shape
        const hipError_t e = qmm::launch_gemv_fp(a, f, (hipStream_t)stream);
        if (e != hipErrorNotSupported) return hip_status(e, fn);
    }
    return hip_status(qmm::launch_gemm_fp(a, f, (hipStream_t)stream), fn);
}

static qmm_status int8_product(const char *fn, const int8_t *Xq, const qmm_half *sx, const uint32_t *wq,
                               const qmm_half *s, const qmm_half *z, qmm_half *Y, int32_t *acc_out, int64_t M,
                               int64_t K, int64_t N, int bits, int64_t G, qmm_stream stream)
{
    qmm_status st = check_shape(fn, M, K, N, bits, G, true);
    if (st != QMM_OK) return st;
    if (!Xq || !sx || !wq || !s || !Y) return fail(QMM_ERR_INVALID_ARG, "%s: null pointer", fn);
    if (G % 128 != 0 || (G / 128 & (G / 128 - 1)) != 0 || G > 1024)
        return fail(QMM_ERR_UNSUPPORTED, "%s: G must be 128, 256, 512 or 1024", fn);
    if ((M + 15) / 16 > 65535) return fail(QMM_ERR_UNSUPPORTED, "%s: M too large", fn);
    if (acc_out && M * (K / G) * N > (int64_t(1) << 31) - 1)
        return fail(QMM_ERR_UNSUPPORTED, "%s: accumulator dump too large", fn);
    qmm::W4A8Args a{Xq, sx, wq, s, z, Y, acc_out, (int)M, (int)K, (int)N, bits, (int)G};
    return hip_status(qmm::launch_w4a8(a, (hipStream_t)stream), fn);
}

qmm_status qmm_gemm_w4a8(const int8_t *Xq, const qmm_half *sx, const uint32_t *wq, const qmm_half *s,
                         const qmm_half *z, qmm_half *Y, int32_t *acc_out, int64_t M, int64_t K, int64_t N,
                         int64_t G, qmm_stream stream)
{
    return int8_product("qmm_gemm_w4a8", Xq, sx, wq, s, z, Y, acc_out, M, K, N, 4, G, stream);
}

qmm_status qmm_gemm_wka8(const int8_t *Xq, const qmm_half *sx, const uint32_t *wq, const qmm_half *s,
                         const qmm_half *z, qmm_half *Y, int32_t *acc_out, int64_t M, int64_t K, int64_t N, int bits,
                         int64_t G, qmm_stream stream)
{
    return int8_product("qmm_gemm_wka8", Xq, sx, wq, s, z, Y, acc_out, M, K, N, bits, G, stream);
}

qmm_status qmm_quantize(const qmm_half *W, uint8_t *codes, qmm_half *s, qmm_half *z, int64_t K, int64_t N, int bits,
                        int64_t G, qmm_stream stream)
{
    const char *fn = "qmm_quantize";
    qmm_status st = check_shape(fn, 1, K, N, bits, G, true);
    if (st != QMM_OK) return st;
    if (!W || !codes || !s || !z) return fail(QMM_ERR_INVALID_ARG, "%s: null pointer", fn);
    if (K / G > 65535) return fail(QMM_ERR_UNSUPPORTED, "%s: more than 65535 groups per column", fn);
    return hip_status(qmm::launch_quantize(W, codes, s, z, (int)K, (int)N, bits, (int)G, (hipStream_t)stream), fn);
}

qmm_status qmm_probe_read(const void *buf, uint64_t bytes, uint32_t *sink, int grid, qmm_stream stream)
{
    const char *fn = "qmm_probe_read";
    if (!buf || !sink) return fail(QMM_ERR_INVALID_ARG, "%s: null pointer", fn);
    if (bytes < 16 || bytes % 16 != 0) return fail(QMM_ERR_INVALID_ARG, "%s: bytes must be a positive multiple of 16", fn);
    if (grid < 1 || grid > 65535) return fail(QMM_ERR_INVALID_ARG, "%s: grid must be in 1..65535", fn);
    return hip_status(qmm::launch_probe_read(buf, bytes, sink, grid, (hipStream_t)stream), fn);
}

qmm_status qmm_probe_mfma(float *sink, int iters, int grid, int shape, qmm_stream stream)
{
    const char *fn = "qmm_probe_mfma";
    if (!sink) return fail(QMM_ERR_INVALID_ARG, "%s: null pointer", fn);
    if (iters < 1 || grid < 1 || grid > 65535 || (shape != 0 && shape != 1))
        return fail(QMM_ERR_INVALID_ARG, "%s: iters >= 1, grid in 1..65535, shape 0 or 1", fn);
    return hip_status(qmm::launch_probe_mfma(sink, iters, grid, shape, (hipStream_t)stream), fn);
}

const char *qmm_status_string(qmm_status status)
{
    switch (status) {
        case QMM_OK: return "ok";
        case QMM_ERR_INVALID_ARG: return "invalid argument";
        case QMM_ERR_UNSUPPORTED: return "unsupported shape";
        case QMM_ERR_HIP: return "HIP launch failure";
        default: return "unknown status";
    }
}

const char *qmm_last_error(void) { return g_last_error; }

const char *qmm_last_hip_error(void) { return g_last_error; }

}  // extern "C"
