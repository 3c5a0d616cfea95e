/*
 * qmm_oracle.c -- TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow, obviously correct CPU definition of the k-bit weight-quantized
 * matrix product
 *
 *     Y[M,N] = X[M,K] . dequant(Wq)[K,N],    w = (q - z) * s,
 *
 * and of the bit packing that carries the codes q.  Only the test suite, the
 * package's smoke check and the benchmark's CPU-baseline leg load this library.
 * The GPU product path never calls it, and it shares no source, header, table or
 * helper with the HIP kernels.  Everything is computed from the definitions,
 * bit by bit and in fp64 (or exact int64), with no blocking, fusion or
 * reordering: a reader can check each function against the passages cited.
 *
 * Passages followed (page titles as published):
 *  - BitLLM: Efficient Low-Bit, Conversion-Hiding LLM Decoding on Mobile GPUs,
 *    Sec. 2.2 "LLM Quantization": eq. (1) (integer zero-point z), eq. (5)
 *    (dequantisation x ~ s * (q - z)) and the per-group granularity paragraph
 *    (one s and z per group of consecutive elements).
 *  - same page, Sec. 4.3 "Quantization-Aware Packing": contiguous packing of
 *    low-bit values inside 32-bit words (Fig. 8(a): the last of eight 4-bit
 *    values is the word's top nibble, i.e. LSB-first order), and the dp4a
 *    definition (exact integer products summed into an int32 accumulator).
 *  - same page, Sec. 4.4 "Type Conversion-Hiding Computation": integer
 *    accumulation per tile with dequantisation deferred to the tile boundary.
 *  - Tilus verdict page (pith.science, arXiv 2504.12984), skeptic critique and
 *    referee report major comment 1 (Sec. 3.2, Fig. 2(c)): a thread's packed
 *    low-bit values are one contiguous bit string (three u8 = four i6).
 *
 * Packed format (the reading this library takes of "contiguous packing"):
 * column n of Wq is one little-endian bit stream along K.  Code i of the column
 * occupies stream bits [i*k, i*k + k), least significant bit first; stream bit p
 * is bit (p mod 8) of byte floor(p / 8) of the column, and column n starts at
 * byte n * K * k / 8.  Codes are given as uint8 [K][N], row-major.
 *
 * Scales s and zero-points z are given as doubles [N][K/G] (the fp16 inputs
 * widened exactly by the caller); z == NULL means z = 2^(k-1).  Group g of a
 * column covers rows [g*G, (g+1)*G).
 *
 * Floating-point codes (qmm_oracle_qmm_fp): the Tilus verdict page lists
 * float3..float8 weight types beside the integer ones without defining a
 * format; the reading here is the two OCP 8-bit-and-below formats in common
 * use: E2M1 (4 bits: sign, 2 exponent bits with bias 1, 1 mantissa bit;
 * subnormal at exponent 0) and E4M3 (8 bits: sign, 4 exponent bits with bias
 * 7, 3 mantissa bits; subnormal at exponent 0; the all-ones exponent and
 * mantissa pattern is NaN, no infinities), and at 6 bits the two OCP FP6
 * formats, E3M2 (3 exponent bits with bias 3, 2 mantissa bits) and E2M3
 * (2 exponent bits with bias 1, 3 mantissa bits), both with subnormals at
 * exponent 0 and every code finite.  The 3-, 5- and 7-bit widths follow the
 * rule those three formats share (of the k - 1 bits after the sign, the
 * extra one goes to the exponent): E1M1 (bias 0), E2M2 (bias 1) and E3M3
 * (bias 3), subnormals at exponent 0, every code finite.  w = value(q) * s,
 * no zero-point.
 *
 * The quantiser (qmm_oracle_quantize) follows eq. (1) of the same section,
 * q = clip(round(w / s) + z, 0, 2^k - 1), with s and z chosen per (column,
 * group) from the group's range; its header states the reading.
 *
 * Status: 0 = ok, -1 = invalid shape or argument, -2 = non-integer zero-point
 * where the integer path needs one, -3 = int32 accumulator range exceeded.
 */
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <math.h>

static int shape_ok(int64_t K, int64_t N, int bits)
{
    if (bits < 1 || bits > 8) return 0;
    if (K < 0 || N < 0) return 0;
    if ((K * bits) % 8 != 0) return 0;   /* every column is a whole number of bytes */
    return 1;
}

static int groups_ok(int64_t K, int64_t G)
{
    return G >= 1 && K % G == 0;
}

/* Stream bit p of one column. */
static unsigned stream_bit(const uint8_t *col, int64_t p)
{
    return (col[p >> 3] >> (p & 7)) & 1u;
}

/* Code i of one column, gathered bit by bit: q = floor(P / 2^(i*k)) mod 2^k. */
static unsigned column_code(const uint8_t *col, int64_t i, int bits)
{
    unsigned q = 0;
    for (int j = 0; j < bits; ++j)
        q |= stream_bit(col, i * bits + j) << j;
    return q;
}

int qmm_oracle_pack(const uint8_t *codes, uint8_t *stream, int64_t K, int64_t N, int bits)
{
    if (!shape_ok(K, N, bits) || ((K > 0 && N > 0) && (!codes || !stream))) return -1;
    const int64_t colbytes = K * bits / 8;
    const unsigned mask = (1u << bits) - 1u;
#pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; ++n) {
        uint8_t *col = stream + n * colbytes;
        memset(col, 0, (size_t)colbytes);
        for (int64_t i = 0; i < K; ++i) {
            unsigned q = codes[i * N + n] & mask;   /* codes wider than k bits are masked */
            for (int j = 0; j < bits; ++j) {
                int64_t p = i * bits + j;
                if ((q >> j) & 1u) col[p >> 3] |= (uint8_t)(1u << (p & 7));
            }
        }
    }
    return 0;
}

int qmm_oracle_unpack(const uint8_t *stream, uint8_t *codes, int64_t K, int64_t N, int bits)
{
    if (!shape_ok(K, N, bits) || ((K > 0 && N > 0) && (!codes || !stream))) return -1;
    const int64_t colbytes = K * bits / 8;
#pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; ++n) {
        const uint8_t *col = stream + n * colbytes;
        for (int64_t i = 0; i < K; ++i)
            codes[i * N + n] = (uint8_t)column_code(col, i, bits);
    }
    return 0;
}

/* Zero-point of (column n, group g); NULL means the mid-range code 2^(k-1). */
static double zero_point(const double *z, int64_t n, int64_t g, int64_t ngroups, int bits)
{
    return z ? z[n * ngroups + g] : (double)(1u << (bits - 1));
}

/* Eq. (5) per element, fp64: W[i][n] = (q[i][n] - z[n][i/G]) * s[n][i/G].
 * Exact: q - z has at most 9 significant bits and s (an fp16) 11. */
int qmm_oracle_dequant(const uint8_t *stream, const double *s, const double *z,
                       int64_t K, int64_t N, int bits, int64_t G, double *W)
{
    if (!shape_ok(K, N, bits) || !groups_ok(K, G) || ((K > 0 && N > 0) && (!stream || !s || !W))) return -1;
    const int64_t colbytes = K * bits / 8, ngroups = K / G;
#pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; ++n) {
        const uint8_t *col = stream + n * colbytes;
        for (int64_t i = 0; i < K; ++i) {
            int64_t g = i / G;
            double q = (double)column_code(col, i, bits);
            W[i * N + n] = (q - zero_point(z, n, g, ngroups, bits)) * s[n * ngroups + g];
        }
    }
    return 0;
}

/* Y[m][n] = sum_{i=0}^{K-1} X[m][i] * W[i][n], fp64, ascending i. */
int qmm_oracle_qmm(const double *X, const uint8_t *stream, const double *s, const double *z,
                   int64_t M, int64_t K, int64_t N, int bits, int64_t G, double *Y)
{
    if (!shape_ok(K, N, bits) || !groups_ok(K, G) || M < 0) return -1;
    if ((M > 0 && N > 0) && (!Y || (K > 0 && (!X || !stream || !s)))) return -1;
    const int64_t colbytes = K * bits / 8, ngroups = K / G;
    int failed = 0;
#pragma omp parallel for schedule(dynamic, 16)
    for (int64_t n = 0; n < N; ++n) {
        const uint8_t *col = stream + n * colbytes;
        double *w = (double *)malloc(sizeof(double) * (size_t)(K ? K : 1));
        if (!w) { failed = 1; continue; }
        for (int64_t i = 0; i < K; ++i) {
            int64_t g = i / G;
            double q = (double)column_code(col, i, bits);
            w[i] = (q - zero_point(z, n, g, ngroups, bits)) * s[n * ngroups + g];
        }
        for (int64_t m = 0; m < M; ++m) {
            double acc = 0.0;
            for (int64_t i = 0; i < K; ++i)
                acc += X[m * K + i] * w[i];
            Y[m * N + n] = acc;
        }
        free(w);
    }
    return failed ? -1 : 0;
}

/* The same definition evaluated only at the listed (m, n) outputs. */
int qmm_oracle_qmm_sampled(const double *X, const uint8_t *stream, const double *s, const double *z,
                           int64_t M, int64_t K, int64_t N, int bits, int64_t G,
                           const int64_t *ms, const int64_t *ns, int64_t count, double *out)
{
    if (!shape_ok(K, N, bits) || !groups_ok(K, G) || count < 0) return -1;
    for (int64_t t = 0; t < count; ++t)
        if (ms[t] < 0 || ms[t] >= M || ns[t] < 0 || ns[t] >= N) return -1;
    const int64_t colbytes = K * bits / 8, ngroups = K / G;
#pragma omp parallel for schedule(dynamic, 4)
    for (int64_t t = 0; t < count; ++t) {
        const int64_t m = ms[t], n = ns[t];
        const uint8_t *col = stream + n * colbytes;
        double acc = 0.0;
        for (int64_t i = 0; i < K; ++i) {
            int64_t g = i / G;
            double q = (double)column_code(col, i, bits);
            double w = (q - zero_point(z, n, g, ngroups, bits)) * s[n * ngroups + g];
            acc += X[m * K + i] * w;
        }
        out[t] = acc;
    }
    return 0;
}

/* Integer-activation product (int8 activations with one scale per token):
 *   A[m][g][n] = sum_{i in group g} Xq[m][i] * (q[i][n] - z[n][g])      (exact, int64)
 *   Y[m][n]    = sx[m] * sum_g s[n][g] * A[m][g][n]                      (fp64)
 * The integer sum is the dp4a definition applied along the group; the scale is
 * applied once per group, after the integer accumulation (Sec. 4.4).  z must be
 * integer-valued (eq. (1)); every |A| must fit an int32 accumulator. */
int qmm_oracle_w4a8(const int8_t *Xq, const double *sx, const uint8_t *stream,
                    const double *s, const double *z, int64_t M, int64_t K, int64_t N,
                    int bits, int64_t G, int64_t *A, double *Y)
{
    if (!shape_ok(K, N, bits) || !groups_ok(K, G) || M < 0) return -1;
    if ((M > 0 && N > 0) && (!Y || !sx || (K > 0 && (!Xq || !stream || !s)))) return -1;
    const int64_t colbytes = K * bits / 8, ngroups = K / G;
    if (z)
        for (int64_t t = 0; t < N * ngroups; ++t)
            if (z[t] != floor(z[t])) return -2;
    int overflow = 0, failed = 0;
#pragma omp parallel for schedule(dynamic, 16)
    for (int64_t n = 0; n < N; ++n) {
        const uint8_t *col = stream + n * colbytes;
        int64_t *q = (int64_t *)malloc(sizeof(int64_t) * (size_t)(K ? K : 1));
        if (!q) { failed = 1; continue; }
        for (int64_t i = 0; i < K; ++i) q[i] = (int64_t)column_code(col, i, bits);
        for (int64_t m = 0; m < M; ++m) {
            double y = 0.0;
            for (int64_t g = 0; g < ngroups; ++g) {
                const int64_t zg = (int64_t)zero_point(z, n, g, ngroups, bits);
                int64_t a = 0;
                for (int64_t i = g * G; i < (g + 1) * G; ++i)
                    a += (int64_t)Xq[m * K + i] * (q[i] - zg);
                if (a >= 2147483648LL || a < -2147483648LL) overflow = 1;
                if (A) A[(m * ngroups + g) * N + n] = a;
                y += s[n * ngroups + g] * (double)a;
            }
            Y[m * N + n] = sx[m] * y;
        }
        free(q);
    }
    if (failed) return -1;
    return overflow ? -3 : 0;
}

/* Nearest fp16 value to x >= 0 (ties to even significand), as a double; +inf
 * past the largest finite fp16 value.  fp16 values in [2^e, 2^(e+1)) are the
 * multiples of 2^(e-10) (e >= -14; below 2^-14 the multiples of 2^-24), so x is
 * rounded to a whole number of that quantum. */
static double round_to_fp16(double x)
{
    if (x == 0.0) return 0.0;
    int e;
    frexp(x, &e);              /* x = f * 2^e, f in [0.5, 1): x in [2^(e-1), 2^e) */
    e -= 1;
    if (e < -14) e = -14;
    const double quantum = ldexp(1.0, e - 10);
    const double r = rint(x / quantum) * quantum;   /* x / quantum is exact */
    return r > 65504.0 ? INFINITY : r;
}

/* Quantiser, BitLLM Sec. 2.2, eq. (1): q = clip(round(w / s) + z, qmin, qmax)
 * with s > 0 and integer z.  The page does not say how s and z are chosen;
 * the reading here is the min-max affine mapping of each (column n, group g)
 * with zero kept representable, unsigned codes and round half to even:
 *   lo = min(0, min w),  hi = max(0, max w)           over the group's G rows
 *   s  = fp16((hi - lo) / (2^k - 1)),  1 if that is 0,  65504 if it overflows
 *   z  = clamp(round(-lo / s), 0, 2^k - 1)
 *   q  = clamp(round(w / s) + z, 0, 2^k - 1)
 * W is fp16 [K][N] widened to doubles (row-major, the orientation of the
 * codes); codes are uint8 [K][N]; s and z are [N][K/G] doubles holding fp16
 * values.  The quotients are taken in fp64: for fp16 operands the fp64
 * quotient never lands on a rounding tie that the exact quotient is not on. */
int qmm_oracle_quantize(const double *W, int64_t K, int64_t N, int bits, int64_t G,
                        uint8_t *codes, double *s, double *z)
{
    if (bits < 1 || bits > 8 || K < 0 || N < 0 || !groups_ok(K, G)) return -1;
    if (K > 0 && N > 0 && (!W || !codes || !s || !z)) return -1;
    const int64_t ngroups = K / G;
    const double qmax = (double)((1 << bits) - 1);
    for (int64_t n = 0; n < N; ++n) {
        for (int64_t g = 0; g < ngroups; ++g) {
            double lo = 0.0, hi = 0.0;
            for (int64_t i = g * G; i < (g + 1) * G; ++i) {
                const double w = W[i * N + n];
                if (w < lo) lo = w;
                if (w > hi) hi = w;
            }
            double sg = round_to_fp16((hi - lo) / qmax);
            if (sg == 0.0) sg = 1.0;
            if (isinf(sg)) sg = 65504.0;
            const double zg = fmin(fmax(rint(-lo / sg), 0.0), qmax);
            for (int64_t i = g * G; i < (g + 1) * G; ++i) {
                const double q = fmin(fmax(rint(W[i * N + n] / sg) + zg, 0.0), qmax);
                codes[i * N + n] = (uint8_t)q;
            }
            s[n * ngroups + g] = sg;
            z[n * ngroups + g] = zg;
        }
    }
    return 0;
}

/* Value of a floating-point code: fmt 0 = E2M1 (4-bit), fmt 1 = E4M3 (8-bit),
 * fmt 2 = E3M2 and fmt 3 = E2M3 (6-bit), fmt 4 = E1M1 (3-bit), fmt 5 = E2M2
 * (5-bit), fmt 6 = E3M3 (7-bit), from the sign / exponent / mantissa fields
 * as defined above. */
static double float_code_value(unsigned q, int fmt)
{
    if (fmt == 0) {
        const double sign = (q & 8u) ? -1.0 : 1.0;
        const unsigned e = (q >> 1) & 3u, m = q & 1u;
        return sign * (e == 0 ? ldexp((double)m, -1) : ldexp(1.0 + (double)m / 2.0, (int)e - 1));
    }
    if (fmt == 2 || fmt == 3) {
        const int mb = fmt == 2 ? 2 : 3, bias = fmt == 2 ? 3 : 1;
        const double sign = (q & 0x20u) ? -1.0 : 1.0;
        const unsigned e = (q & 0x1fu) >> mb, m = q & ((1u << mb) - 1u);
        const double frac = ldexp((double)m, -mb);
        return sign * (e == 0 ? ldexp(frac, 1 - bias) : ldexp(1.0 + frac, (int)e - bias));
    }
    if (fmt >= 4 && fmt <= 6) {   /* E1M1, E2M2, E3M3: k = 3, 5, 7 */
        const int eb = fmt - 3, mbits = fmt - 3, k = 1 + eb + mbits, bias = (1 << (eb - 1)) - 1;
        const double sign = ((q >> (k - 1)) & 1u) ? -1.0 : 1.0;
        const unsigned e = (q >> mbits) & ((1u << eb) - 1u), m = q & ((1u << mbits) - 1u);
        const double frac = ldexp((double)m, -mbits);
        return sign * (e == 0 ? ldexp(frac, 1 - bias) : ldexp(1.0 + frac, (int)e - bias));
    }
    const double sign = (q & 0x80u) ? -1.0 : 1.0;
    const unsigned e = (q >> 3) & 15u, m = q & 7u;
    if (e == 15 && m == 7) return NAN;
    return sign * (e == 0 ? ldexp((double)m / 8.0, -6) : ldexp(1.0 + (double)m / 8.0, (int)e - 7));
}

double qmm_oracle_float_code_value(unsigned q, int fmt) { return float_code_value(q, fmt); }

/* Y = X . W with W[i][n] = value(q[i][n]) * s[n][i / G] for floating-point codes
 * (fmt 0: E2M1 in 4-bit streams, fmt 1: E4M3 in 8-bit streams, fmt 2 / 3:
 * E3M2 / E2M3 in 6-bit streams, fmt 4 / 5 / 6: E1M1 / E2M2 / E3M3 in 3-, 5-
 * and 7-bit streams), fp64. */
int qmm_oracle_qmm_fp(const double *X, const uint8_t *stream, const double *s, int64_t M, int64_t K, int64_t N,
                      int fmt, int64_t G, double *Y)
{
    const int bits = fmt == 0 ? 4 : fmt == 1 ? 8 : (fmt == 2 || fmt == 3) ? 6 : (fmt >= 4 && fmt <= 6) ? 2 * fmt - 5 : 0;
    if (!shape_ok(K, N, bits) || !groups_ok(K, G) || M < 0) return -1;
    if ((M > 0 && N > 0) && (!Y || (K > 0 && (!X || !stream || !s)))) return -1;
    const int64_t colbytes = K * bits / 8, ngroups = K / G;
    int failed = 0;
#pragma omp parallel for schedule(dynamic, 16)
    for (int64_t n = 0; n < N; ++n) {
        const uint8_t *col = stream + n * colbytes;
        double *w = (double *)malloc(sizeof(double) * (size_t)(K ? K : 1));
        if (!w) { failed = 1; continue; }
        for (int64_t i = 0; i < K; ++i)
            w[i] = float_code_value(column_code(col, i, bits), fmt) * s[n * ngroups + i / G];
        for (int64_t m = 0; m < M; ++m) {
            double acc = 0.0;
            for (int64_t i = 0; i < K; ++i)
                acc += X[m * K + i] * w[i];
            Y[m * N + n] = acc;
        }
        free(w);
    }
    return failed ? -1 : 0;
}
