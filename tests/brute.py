"""Independent brute-force references used to pin the CPU oracle.

Nothing here imports the oracle or the GPU path.  Packing is written as one
Python big integer per column (the stream's value P_n = sum_i q_i * 2^(i*k),
stored little-endian), and products as exact rationals (``fractions.Fraction``)
or exact integers, so a mistake in the oracle's bit loops or fp64 sums cannot
hide behind the same mistake here.
"""
from __future__ import annotations

from fractions import Fraction

import numpy as np


def bigint_pack_column(codes_col, bits: int) -> bytes:
    """P = sum_i q_i * 2^(i*k) as K*k/8 little-endian bytes (codes masked to k bits)."""
    P = 0
    for i, q in enumerate(codes_col):
        P += (int(q) & ((1 << bits) - 1)) << (i * bits)
    return P.to_bytes(len(codes_col) * bits // 8, "little")


def bigint_pack(codes: np.ndarray, bits: int) -> np.ndarray:
    K, N = codes.shape
    out = np.zeros((N, K * bits // 8), dtype=np.uint8)
    for n in range(N):
        out[n] = np.frombuffer(bigint_pack_column(codes[:, n], bits), dtype=np.uint8)
    return out


def bigint_unpack(stream: np.ndarray, K: int, N: int, bits: int) -> np.ndarray:
    """q_i = floor(P / 2^(i*k)) mod 2^k for each column's big integer P."""
    b = np.ascontiguousarray(stream).view(np.uint8).reshape(N, K * bits // 8)
    out = np.zeros((K, N), dtype=np.uint8)
    for n in range(N):
        P = int.from_bytes(b[n].tobytes(), "little")
        for i in range(K):
            out[i, n] = (P >> (i * bits)) & ((1 << bits) - 1)
    return out


def frac(x) -> Fraction:
    return Fraction(float(x))


def exact_qmm(X, codes, s, z, bits: int, G: int):
    """Exact rational Y[m][n] = sum_i X[m][i] * (q[i][n] - z[n][i/G]) * s[n][i/G],
    plus the sum of |terms| (for the fp64 summation error bound)."""
    M, K = X.shape
    N = codes.shape[1]
    Y = [[Fraction(0)] * N for _ in range(M)]
    A = [[Fraction(0)] * N for _ in range(M)]
    zdef = 1 << (bits - 1)
    for n in range(N):
        w = []
        for i in range(K):
            g = i // G
            zz = frac(z[n, g]) if z is not None else Fraction(zdef)
            w.append((int(codes[i, n]) - zz) * frac(s[n, g]))
        for m in range(M):
            acc = Fraction(0)
            aabs = Fraction(0)
            for i in range(K):
                t = frac(X[m, i]) * w[i]
                acc += t
                aabs += abs(t)
            Y[m][n] = acc
            A[m][n] = aabs
    return Y, A


def exact_w4a8(Xq, sx, codes, s, z, bits: int, G: int):
    """Integer A[m][g][n] and exact rational Y[m][n] = sx[m] * sum_g s[n][g] * A[m][g][n]."""
    M, K = Xq.shape
    N = codes.shape[1]
    ng = K // G
    zdef = 1 << (bits - 1)
    A = np.zeros((M, ng, N), dtype=np.int64)
    Y = [[Fraction(0)] * N for _ in range(M)]
    for m in range(M):
        for n in range(N):
            y = Fraction(0)
            for g in range(ng):
                zz = int(z[n, g]) if z is not None else zdef
                a = 0
                for i in range(g * G, (g + 1) * G):
                    a += int(Xq[m, i]) * (int(codes[i, n]) - zz)
                A[m, g, n] = a
                y += frac(s[n, g]) * a
            Y[m][n] = frac(sx[m]) * y
    return A, Y


def fp64_sum_bound(n_terms: int, abs_sum: Fraction) -> float:
    """Recursive fp64 summation of n exact terms errs by at most gamma_{n-1} * sum|terms|
    with gamma_j = j u / (1 - j u), u = 2^-53."""
    u = 2.0 ** -53
    j = max(n_terms - 1, 1)
    return float(abs_sum) * (j * u / (1 - j * u)) * 1.000001 + 1e-300


def read_page_facts(path: str) -> dict:
    facts = {}
    with open(path) as fh:
        for line in fh:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            name, *kvs = line.split()
            facts[name] = {k: int(v) for k, v in (kv.split("=") for kv in kvs)}
    return facts


def _fp16_positive_table():
    """Every finite fp16 value >= 0, ascending, as exact Fractions with its bit pattern."""
    bits = np.arange(0, 0x7C00, dtype=np.uint16)
    vals = bits.view(np.float16).astype(np.float64)
    return [Fraction(float(v)) for v in vals], bits


_FP16 = None


def nearest_fp16(r: Fraction):
    """Nearest finite fp16 value to r >= 0 by search over the whole table (ties to
    the even bit pattern); None past the largest finite value plus half its spacing."""
    global _FP16
    if _FP16 is None:
        _FP16 = _fp16_positive_table()
    vals, bits = _FP16
    top = vals[-1]
    if r >= top + (top - vals[-2]) / 2:
        return None
    import bisect
    j = bisect.bisect_left(vals, r)
    if j < len(vals) and vals[j] == r:
        return vals[j]
    lo, hi = vals[j - 1], vals[j]
    if r - lo < hi - r:
        return lo
    if hi - r < r - lo:
        return hi
    return lo if int(bits[j - 1]) % 2 == 0 else hi


def exact_quantize(W, bits: int, G: int):
    """Quantiser of eq. (1) with the min-max (zero-including) reading, in exact rational
    arithmetic: codes [K][N], s and z [N][K/G] as Fractions."""
    K, N = W.shape
    qmax = (1 << bits) - 1
    ng = K // G
    codes = np.zeros((K, N), dtype=np.int64)
    s = [[None] * ng for _ in range(N)]
    z = [[None] * ng for _ in range(N)]
    for n in range(N):
        for g in range(ng):
            col = [Fraction(float(W[i, n])) for i in range(g * G, (g + 1) * G)]
            lo = min([Fraction(0)] + col)
            hi = max([Fraction(0)] + col)
            sg = nearest_fp16((hi - lo) / qmax)
            if sg is None:
                sg = Fraction(65504)
            elif sg == 0:
                sg = Fraction(1)
            zg = min(max(round(-lo / sg), 0), qmax)
            for r, w in enumerate(col):
                codes[g * G + r, n] = min(max(round(w / sg) + zg, 0), qmax)
            s[n][g] = sg
            z[n][g] = Fraction(zg)
    return codes, s, z
