"""Pins of the CPU oracle against facts that do not come from the oracle itself.

Each ``pin_*`` function takes an :class:`oracle.Oracle` and raises
``AssertionError`` when the oracle disagrees with the pages, the mathematics or
an independent brute force.  ``test_oracle_pins.py`` runs them on the real
oracle; ``test_oracle_mutants.py`` runs them on copies of the oracle with
planted mistakes and requires each mistake to be caught.
"""
from __future__ import annotations

import os
from fractions import Fraction

import numpy as np

import brute
import synthetic

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "page_facts.txt")
ALL_BITS = range(1, 9)


def _case(M, K, N, bits, G, seed, per_group_z):
    return synthetic.make_case(M, K, N, bits, G, seed, per_group_z=per_group_z, s_range=(0.002, 0.02))


# ---------------------------------------------------------------- packing ---
def pin_pack_matches_bigint(orc):
    """pack == the big-integer definition P_n = sum_i q_i 2^(i k), little-endian."""
    for bits in ALL_BITS:
        for K, N in ((32, 3), (64, 5), (8 * 7, 2)):
            if (K * bits) % 8:
                continue
            g = synthetic.rng(11 * bits + K)
            codes = synthetic.codes_uniform(g, bits, K, N)
            assert np.array_equal(orc.pack(codes, bits), brute.bigint_pack(codes, bits)), (bits, K, N)


def pin_unpack_matches_bigint(orc):
    """unpack == floor(P / 2^(i k)) mod 2^k on arbitrary byte streams."""
    for bits in ALL_BITS:
        K, N = 64, 4
        g = synthetic.rng(100 + bits)
        stream = g.integers(0, 256, size=(N, K * bits // 8), dtype=np.uint8)
        assert np.array_equal(orc.unpack(stream, K, N, bits), brute.bigint_unpack(stream, K, N, bits)), bits


def pin_exhaustive_single_code(orc):
    """Every value 0..2^k-1 at every position 0..31 of a 32-code run, alone in its column,
    lands exactly at stream bits [i k, i k + k)."""
    for bits in ALL_BITS:
        K = 32
        vals = np.arange(1 << bits)
        N = 32 * vals.size
        codes = np.zeros((K, N), dtype=np.uint8)
        expect = np.zeros((N, K * bits // 8), dtype=np.uint8)
        for pos in range(32):
            for v in vals:
                n = pos * vals.size + v
                codes[pos, n] = v
                expect[n] = np.frombuffer((int(v) << (pos * bits)).to_bytes(K * bits // 8, "little"), np.uint8)
        got = orc.pack(codes, bits)
        assert np.array_equal(got, expect), bits
        assert np.array_equal(orc.unpack(got, K, N, bits), codes), bits


def pin_round_trips(orc):
    """unpack(pack(q)) == q and pack(unpack(b)) == b (a bijection when K k % 8 == 0)."""
    for bits in ALL_BITS:
        K, N = 96, 7
        g = synthetic.rng(200 + bits)
        codes = synthetic.codes_uniform(g, bits, K, N)
        assert np.array_equal(orc.unpack(orc.pack(codes, bits), K, N, bits), codes), bits
        stream = g.integers(0, 256, size=(N, K * bits // 8), dtype=np.uint8)
        assert np.array_equal(orc.pack(orc.unpack(stream, K, N, bits), bits), stream), bits


def pin_codes_masked(orc):
    """Codes wider than k bits contribute only their low k bits."""
    for bits in range(1, 8):
        g = synthetic.rng(300 + bits)
        wide = g.integers(0, 256, size=(32, 3), dtype=np.uint8)
        low = (wide & ((1 << bits) - 1)).astype(np.uint8)
        assert np.array_equal(orc.pack(wide, bits), orc.pack(low, bits)), bits


def pin_k8_is_byte_identity(orc):
    """For k = 8 the stream of a column is its codes, byte for byte."""
    g = synthetic.rng(400)
    codes = synthetic.codes_uniform(g, 8, 64, 5)
    assert np.array_equal(orc.pack(codes, 8), codes.T)


def pin_page_facts(orc):
    """Packing facts the pages state (tests/golden/page_facts.txt, cited there)."""
    facts = brute.read_page_facts(GOLDEN)
    # BitLLM Fig. 8(a): last of eight 4-bit values of a word = word >> 28.
    f = facts["contiguous_last_value"]
    g = synthetic.rng(500)
    codes = synthetic.codes_uniform(g, f["bits"], f["values_per_word"], 16)
    words = orc.pack(codes, f["bits"]).view("<u4").reshape(-1)
    assert np.array_equal(words >> f["shift"], codes[f["index"]].astype(np.uint32))
    # Tilus: four 6-bit values are exactly three bytes, and every 24-bit pattern is one
    # arrangement of four codes (a bijection; sampled).
    f = facts["same_bits_view"]
    g = synthetic.rng(501)
    codes = synthetic.codes_uniform(g, f["bits"], f["codes"], 64)
    st = orc.pack(codes, f["bits"])
    assert st.shape == (64, f["bytes"])
    assert np.array_equal(orc.unpack(st, f["codes"], 64, f["bits"]), codes)
    pats = g.integers(0, 256, size=(64, f["bytes"]), dtype=np.uint8)
    assert np.array_equal(orc.pack(orc.unpack(pats, f["codes"], 64, f["bits"]), f["bits"]), pats)
    # BitLLM dp4a: a word of four 8-bit values is sum_i a_i * 256^i.
    f = facts["dp4a_word"]
    codes = synthetic.codes_uniform(g, f["bits"], f["values_per_word"], 32)
    words = orc.pack(codes, f["bits"]).view("<u4").reshape(-1).astype(np.int64)
    expect = sum(codes[i].astype(np.int64) * f["weight_base"] ** i for i in range(f["values_per_word"]))
    assert np.array_equal(words, expect)


# ------------------------------------------------------------ dequantise ---
def pin_dequant_exact_rational(orc):
    """W == (q - z) * s exactly (the products are exact in fp64), default and per-group z."""
    for bits in ALL_BITS:
        for pgz in (False, True):
            c = _case(1, 64, 6, bits, 32, 600 + bits, pgz)
            st = brute.bigint_pack(c["codes"], bits)
            W = orc.dequant(st, c["s"], c["z"], 64, 6, bits, 32)
            zdef = 1 << (bits - 1)
            for i in range(64):
                for n in range(6):
                    zz = brute.frac(c["z"][n, i // 32]) if pgz else Fraction(zdef)
                    w = (int(c["codes"][i, n]) - zz) * brute.frac(c["s"][n, i // 32])
                    assert Fraction(W[i, n]) == w, (bits, pgz, i, n)


def pin_k8_is_int8_dequant(orc):
    """k = 8 with z = 128 is plain symmetric int8 dequantisation: W = int8(q ^ 0x80) * s."""
    c = _case(1, 128, 9, 8, 64, 700, False)
    st = brute.bigint_pack(c["codes"], 8)
    W = orc.dequant(st, c["s"], None, 128, 9, 8, 64)
    as_int8 = (c["codes"] ^ 0x80).astype(np.uint8).view(np.int8).astype(np.float64)
    s_rows = np.repeat(c["s"].astype(np.float64).T, 64, axis=0)   # [K][N]
    assert np.array_equal(W, as_int8 * s_rows)


def pin_codes_equal_zero_point_give_zero(orc):
    """q == z everywhere => W == 0 and Y == 0 exactly."""
    for bits in ALL_BITS:
        K, N, G = 128, 5, 32
        g = synthetic.rng(800 + bits)
        z = synthetic.zeros_uniform(g, bits, N, K // G)
        codes = np.repeat(z.astype(np.uint8).T, G, axis=0)          # [K][N], q[i][n] = z[n][i/G]
        s = synthetic.fp16_uniform(g, 0.002, 0.02, (N, K // G))
        X = synthetic.fp16_normal(g, (3, K))
        st = brute.bigint_pack(codes, bits)
        assert not orc.dequant(st, s, z, K, N, bits, G).any()
        Y = orc.qmm(X, st, s, z, bits, G)
        assert np.array_equal(Y, np.zeros_like(Y))
        mid = np.full((K, N), 1 << (bits - 1), dtype=np.uint8)
        Y = orc.qmm(X, brute.bigint_pack(mid, bits), s, None, bits, G)
        assert np.array_equal(Y, np.zeros_like(Y))


# ---------------------------------------------------------------- matmul ---
def pin_qmm_exact_rational(orc):
    """fp64 Y within the recursive-summation bound of the exact rational Y (tiny shapes,
    every k, >= 2 groups, default and per-group z)."""
    for bits in ALL_BITS:
        for (M, K, N, G, pgz) in ((2, 64, 3, 32, False), (1, 128, 4, 64, True)):
            c = _case(M, K, N, bits, G, 900 + bits + K, pgz)
            st = brute.bigint_pack(c["codes"], bits)
            Y = orc.qmm(c["X"], st, c["s"], c["z"], bits, G)
            Yx, Aabs = brute.exact_qmm(c["X"], c["codes"], c["s"], c["z"], bits, G)
            for m in range(M):
                for n in range(N):
                    err = abs(Fraction(Y[m, n]) - Yx[m][n])
                    assert err <= Fraction(brute.fp64_sum_bound(K, Aabs[m][n])), (bits, m, n, float(err))


def pin_integer_special_case(orc):
    """s = 1, z = 0, G = K and integer X: Y = X_int @ Q exactly (numpy int64 matmul)."""
    for bits in ALL_BITS:
        M, K, N = 3, 64, 7
        g = synthetic.rng(1000 + bits)
        Xi = g.integers(-20, 21, size=(M, K))
        codes = synthetic.codes_uniform(g, bits, K, N)
        s = np.ones((N, 1), dtype=np.float16)
        z = np.zeros((N, 1), dtype=np.float16)
        Y = orc.qmm(Xi.astype(np.float16), brute.bigint_pack(codes, bits), s, z, bits, K)
        assert np.array_equal(Y, (Xi @ codes.astype(np.int64)).astype(np.float64)), bits


def pin_one_hot_rows(orc):
    """A one-hot row of X selects the matching row of dequant(W) exactly."""
    bits, K, N, G = 5, 96, 6, 32
    c = _case(1, K, N, bits, G, 1100, True)
    st = brute.bigint_pack(c["codes"], bits)
    W = orc.dequant(st, c["s"], c["z"], K, N, bits, G)
    rows = [0, 31, 32, 95]
    X = np.zeros((len(rows), K), dtype=np.float16)
    for r, i in enumerate(rows):
        X[r, i] = 1
    Y = orc.qmm(X, st, c["s"], c["z"], bits, G)
    assert np.array_equal(Y, W[rows]), rows


def pin_sampled_matches_full(orc):
    """The sampled entry point computes the same numbers as the full product."""
    c = _case(3, 128, 9, 3, 64, 1200, True)
    st = brute.bigint_pack(c["codes"], 3)
    Y = orc.qmm(c["X"], st, c["s"], c["z"], 3, 64)
    ms = np.array([0, 1, 2, 2, 0])
    ns = np.array([0, 8, 3, 7, 5])
    got = orc.qmm_sampled(c["X"], st, c["s"], c["z"], 3, 64, ms, ns)
    assert np.array_equal(got, Y[ms, ns])


# ------------------------------------------------------------------ W4A8 ---
def pin_w4a8_bruteforce(orc):
    """Integer A bit-exact vs Python integers; Y within the fp64 bound of the exact value."""
    for (M, K, N, G, pgz) in ((2, 128, 5, 64, False), (3, 64, 4, 32, True)):
        c = synthetic.make_w4a8_case(M, K, N, G, 1300 + K, per_group_z=pgz)
        st = brute.bigint_pack(c["codes"], 4)
        A, Y = orc.w4a8(c["Xq"], c["sx"], st, c["s"], c["z"], G)
        Ax, Yx = brute.exact_w4a8(c["Xq"], c["sx"], c["codes"], c["s"], c["z"], 4, G)
        assert np.array_equal(A, Ax)
        ng = K // G
        for m in range(M):
            for n in range(N):
                terms = sum(abs(brute.frac(c["s"][n, g]) * int(Ax[m, g, n])) for g in range(ng))
                bound = brute.frac(c["sx"][m]) * terms * Fraction(2.0 ** -52 * (ng + 2)) + Fraction(1, 10 ** 300)
                assert abs(Fraction(Y[m, n]) - Yx[m][n]) <= bound, (m, n)


def pin_wka8_every_width_bruteforce(orc):
    """The integer product for every code width: A bit-exact vs Python integers
    (codes at both ends of their range included), Y within the fp64 bound."""
    for bits in range(1, 9):
        M, K, N, G = 2, 64, 3, 32
        pgz = bits % 2 == 1
        c = synthetic.make_w4a8_case(M, K, N, G, 1600 + bits, bits=bits, per_group_z=pgz)
        c["codes"][:, 0] = (1 << bits) - 1
        c["codes"][:, 1] = 0
        st = brute.bigint_pack(c["codes"], bits)
        A, Y = orc.w4a8(c["Xq"], c["sx"], st, c["s"], c["z"], G, bits=bits)
        Ax, Yx = brute.exact_w4a8(c["Xq"], c["sx"], c["codes"], c["s"], c["z"], bits, G)
        assert np.array_equal(A, Ax), bits
        ng = K // G
        for m in range(M):
            for n in range(N):
                terms = sum(abs(brute.frac(c["s"][n, g]) * int(Ax[m, g, n])) for g in range(ng))
                bound = brute.frac(c["sx"][m]) * terms * Fraction(2.0 ** -52 * (ng + 2)) + Fraction(1, 10 ** 300)
                assert abs(Fraction(Y[m, n]) - Yx[m][n]) <= bound, (bits, m, n)


def pin_w8a8_matches_integer_matmul(orc):
    """k = 8 with the default zero-point 128: per group A = Xq[:, g] @ (Q[g] - 128)."""
    M, K, N, G = 3, 256, 5, 128
    c = synthetic.make_w4a8_case(M, K, N, G, 1700, bits=8)
    st = brute.bigint_pack(c["codes"], 8)
    A, _ = orc.w4a8(c["Xq"], c["sx"], st, c["s"], None, G, bits=8)
    Q = c["codes"].astype(np.int64) - 128
    for g in range(K // G):
        assert np.array_equal(A[:, g, :], c["Xq"][:, g * G:(g + 1) * G].astype(np.int64) @ Q[g * G:(g + 1) * G])


def pin_w4a8_matches_integer_matmul(orc):
    """Per group, A = Xq[:, g] @ (Q[g] - z): numpy int64 matmul as the library special case."""
    M, K, N, G = 4, 256, 6, 128
    c = synthetic.make_w4a8_case(M, K, N, G, 1400)
    st = brute.bigint_pack(c["codes"], 4)
    A, _ = orc.w4a8(c["Xq"], c["sx"], st, c["s"], None, G)
    Q = c["codes"].astype(np.int64) - 8
    for g in range(K // G):
        assert np.array_equal(A[:, g, :], c["Xq"][:, g * G:(g + 1) * G].astype(np.int64) @ Q[g * G:(g + 1) * G])


def pin_w4a8_rejects_fractional_z(orc):
    """Eq. (1) zero-points are integers; the integer path refuses anything else."""
    c = synthetic.make_w4a8_case(1, 64, 2, 32, 1500, per_group_z=True)
    z = c["z"].copy()
    z[0, 0] = np.float16(2.5)
    st = brute.bigint_pack(c["codes"], 4)
    try:
        orc.w4a8(c["Xq"], c["sx"], st, c["s"], z, 32)
    except ValueError:
        return
    raise AssertionError("fractional zero-point accepted")


# ------------------------------------------------------------ signed codes ---
def pin_signed_codes_dequantise_to_q_times_s(orc):
    """Two's-complement codes stored offset-binary: with the default zero-point the
    dequantised weight is q s exactly, and a signed zero-point z_s passed as
    z_s + 2^(k-1) gives (q - z_s) s (numpy closed forms)."""
    rng = np.random.default_rng(2100)
    for bits in range(1, 9):
        K, N, G = 64, 5, 32
        lo, hi = -(1 << (bits - 1)), (1 << (bits - 1)) - 1
        q = rng.integers(lo, hi + 1, (K, N))
        q[0, :], q[1, :] = lo, hi
        s = rng.uniform(0.01, 0.1, (N, K // G)).astype(np.float16)
        st = orc.pack_signed(q.astype(np.int8), bits)
        s_rows = np.repeat(s.astype(np.float64).T, G, axis=0)
        assert np.array_equal(orc.dequant(st, s, None, K, N, bits, G), q * s_rows), bits
        zs = rng.integers(lo, hi + 1, (N, K // G))
        z_rows = np.repeat(zs.T, G, axis=0)
        got = orc.dequant(st, s, (zs + (1 << (bits - 1))).astype(np.float16), K, N, bits, G)
        assert np.array_equal(got, (q - z_rows) * s_rows), bits


# ---------------------------------------------------- floating-point codes ---
E2M1_MAGNITUDES = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]   # the eight E2M1 magnitudes, codes 0..7


def pin_e2m1_values(orc):
    """E2M1 codes 0..7 are the eight magnitudes in order; bit 3 is the sign."""
    for q in range(16):
        v = orc.float_code_value(q, 0)
        assert abs(v) == E2M1_MAGNITUDES[q & 7] and (np.signbit(v) == bool(q & 8)), q


def pin_e4m3_landmarks(orc):
    """E4M3 facts: 1.0 = 0x38, 2^-6 = 0x08 (smallest normal), 2^-9 = 0x01 (smallest
    subnormal), 448 = 0x7E (largest), NaN only at 0x7F / 0xFF, bit 7 the sign,
    magnitudes strictly increasing over 0x00..0x7E with 8 equal steps per binade
    (steps of 2^-9 through the subnormals and the first normal binade)."""
    v = [orc.float_code_value(q, 1) for q in range(256)]
    assert v[0x38] == 1.0 and v[0x08] == 2.0 ** -6 and v[0x01] == 2.0 ** -9 and v[0x7E] == 448.0
    assert np.isnan(v[0x7F]) and np.isnan(v[0xFF]) and sum(np.isnan(x) for x in v) == 2
    for q in range(0x7F):
        assert v[q + 0x80] == -v[q] and np.signbit(v[q + 0x80])
    mags = v[:0x7F]
    assert all(b > a for a, b in zip(mags, mags[1:]))
    for q in range(0, 0x78, 8):   # each run of 8 codes has equal steps
        steps = {mags[q + j + 1] - mags[q + j] for j in range(7)}
        assert len(steps) == 1, q
    assert mags[1] - mags[0] == 2.0 ** -9 and mags[9] - mags[8] == 2.0 ** -9


def _float_landmarks(v, one, min_normal, min_sub, max_code, max_val, per_binade):
    """Checks for a format whose codes (len(v) of them) carry the sign in the top
    bit, every code finite, subnormals at exponent 0."""
    half = len(v) // 2
    assert v[one] == 1.0 and v[per_binade] == min_normal and v[1] == min_sub and v[max_code] == max_val
    assert not any(np.isnan(x) or np.isinf(x) for x in v)     # every code finite
    for q in range(half):
        assert v[q + half] == -v[q] and np.signbit(v[q + half])
    mags = v[:half]
    assert all(b > a for a, b in zip(mags, mags[1:]))
    for q in range(0, half, per_binade):   # equal steps inside each binade
        assert len({mags[q + j + 1] - mags[q + j] for j in range(per_binade - 1)}) == 1, q
    # subnormals continue the first normal binade's step
    assert mags[1] - mags[0] == min_sub and mags[per_binade + 1] - mags[per_binade] == min_sub


def pin_e3m2_landmarks(orc):
    """E3M2 (6-bit, bias 3): 1.0 = 0x0C, 0.25 = 0x04 (smallest normal),
    0.0625 = 0x01 (smallest subnormal), 28 = 0x1F (largest), bit 5 the sign,
    4 codes per binade, every code finite."""
    _float_landmarks([orc.float_code_value(q, 2) for q in range(64)], 0x0C, 0.25, 0.0625, 0x1F, 28.0, 4)


def pin_e2m3_landmarks(orc):
    """E2M3 (6-bit, bias 1): 1.0 = 0x08 (smallest normal), 0.125 = 0x01
    (smallest subnormal), 7.5 = 0x1F (largest), bit 5 the sign, 8 codes per
    binade, every code finite."""
    _float_landmarks([orc.float_code_value(q, 3) for q in range(64)], 0x08, 1.0, 0.125, 0x1F, 7.5, 8)


def pin_e1m1_values(orc):
    """E1M1 (3-bit, bias 0): codes 0..3 are 0, 1, 2, 3; bit 2 the sign."""
    v = [orc.float_code_value(q, 4) for q in range(8)]
    assert v[:4] == [0.0, 1.0, 2.0, 3.0]
    _float_landmarks(v, 0x1, 2.0, 1.0, 0x3, 3.0, 2)


def pin_e2m2_landmarks(orc):
    """E2M2 (5-bit, bias 1): 0.25 = 0x01 (smallest subnormal), 1.0 = 0x04
    (smallest normal), 7 = 0x0F (largest), bit 4 the sign, 4 codes per binade."""
    _float_landmarks([orc.float_code_value(q, 5) for q in range(32)], 0x04, 1.0, 0.25, 0x0F, 7.0, 4)


def pin_e3m3_landmarks(orc):
    """E3M3 (7-bit, bias 3): 2^-5 = 0x01 (smallest subnormal), 0.25 = 0x08
    (smallest normal), 1.0 = 0x18, 30 = 0x3F (largest), bit 6 the sign, 8 codes
    per binade."""
    _float_landmarks([orc.float_code_value(q, 6) for q in range(128)], 0x18, 0.25, 2.0 ** -5, 0x3F, 30.0, 8)


def pin_float_code_product_bruteforce(orc):
    """Y = X (value(q) s) for every format against exact rational arithmetic
    (E2M1 values from the magnitude table, the others from the landmark-checked
    decode)."""
    rng = np.random.default_rng(2200)
    for fmt, bits in ((0, 4), (1, 8), (2, 6), (3, 6), (4, 3), (5, 5), (6, 7)):
        M, K, N, G = 2, 64, 3, 32
        hi = 1 << bits
        codes = rng.integers(0, hi, (K, N))
        if fmt == 1:
            codes[(codes & 0x7F) == 0x7F] = 0x3A   # NaN codes are not inputs
        X = rng.normal(0, 1, (M, K)).astype(np.float16)
        s = rng.uniform(0.01, 0.1, (N, K // G)).astype(np.float16)
        st = brute.bigint_pack(codes.astype(np.uint8), bits)
        Y = orc.qmm_fp(X, st, s, fmt, G)
        for m in range(M):
            for n in range(N):
                exact = Fraction(0)
                aabs = Fraction(0)
                for i in range(K):
                    q = int(codes[i, n])
                    val = (Fraction(E2M1_MAGNITUDES[q & 7]) * (-1 if q & 8 else 1)) if fmt == 0 else \
                        Fraction(orc.float_code_value(q, fmt))
                    t = Fraction(float(X[m, i])) * val * Fraction(float(s[n, i // G]))
                    exact += t
                    aabs += abs(t)
                assert abs(Fraction(Y[m, n]) - exact) <= brute.fp64_sum_bound(K, aabs) * 2, (fmt, m, n)


# --------------------------------------------------------------- quantiser ---
def _quantize_cases():
    """Tiny fp16 weight matrices with the special groups of the reading: random
    normals, exact rounding ties, constant (zero, positive, negative) groups,
    ranges that overflow or underflow the fp16 scale."""
    rng = np.random.default_rng(1800)
    K, N, G = 64, 6, 16
    W = rng.normal(0.0, 0.05, (K, N)).astype(np.float16)
    W[0:16, 1] = 0                                   # all-zero group
    W[16:32, 1] = np.float16(0.75)                   # constant positive group
    W[32:48, 1] = np.float16(-3.0)                   # constant negative group
    W[0:16, 2] = np.arange(16, dtype=np.float16) * np.float16(0.5)   # w / s on half steps at k = 5
    W[16:32, 2] = np.float16(-60000.0)               # range past the fp16 scale at k = 1
    W[17, 2] = np.float16(60000.0)
    W[32:48, 2] = np.float16(2.0 ** -24)             # a scale that underflows fp16
    W[48:64, 3] = np.linspace(-1, 1, 16).astype(np.float16)
    W[48:64, 2] = np.array([0, 3, 0.5, 1.5, 2.5, 0.5, 1.5, 2.5, 1, 2, 0, 3, 2.5, 0.5, 1.5, 3],
                           dtype=np.float16)      # s = 1 at k = 2: every w / s a tie or a whole number
    return W, G


def pin_quantize_bruteforce(orc):
    """Codes, s and z bit-exact against exact rational arithmetic and a search
    over every fp16 value, for every code width."""
    W, G = _quantize_cases()
    for bits in range(1, 9):
        codes, s, z = orc.quantize(W, bits, G)
        cx, sx, zx = brute.exact_quantize(W, bits, G)
        assert np.array_equal(codes.astype(np.int64), cx), bits
        for n in range(W.shape[1]):
            for g in range(W.shape[0] // G):
                assert Fraction(float(s[n, g])) == sx[n][g], (bits, n, g)
                assert Fraction(float(z[n, g])) == zx[n][g], (bits, n, g)


def pin_quantize_round_trip(orc):
    """Weights already on a grid s (q - z), with both code ends present in every
    group and s a power of two, come back as exactly q, s and z."""
    rng = np.random.default_rng(1900)
    for bits in range(1, 9):
        qmax = (1 << bits) - 1
        K, N, G = 64, 5, 32
        q = rng.integers(0, qmax + 1, (K, N))
        q[0::G, :] = 0
        q[1::G, :] = qmax
        z = rng.integers(0, qmax + 1, (N, K // G))
        sc = 2.0 ** -6
        W = np.zeros((K, N))
        for g in range(K // G):
            W[g * G:(g + 1) * G] = sc * (q[g * G:(g + 1) * G] - z[:, g][None, :])
        W16 = W.astype(np.float16)
        assert np.array_equal(W16.astype(np.float64), W)
        codes, s, zz = orc.quantize(W16, bits, G)
        assert np.array_equal(codes.astype(np.int64), q), bits
        assert np.all(s.astype(np.float64) == sc) and np.array_equal(zz.astype(np.int64), z), bits


def pin_quantize_error_bound(orc):
    """Every weight is reproduced within one step s (half a step from rounding,
    at most half more from the fp16 rounding of s at the clipped ends), and zero
    exactly."""
    rng = np.random.default_rng(2000)
    K, N, G = 256, 7, 64
    W = rng.normal(0.0, 0.02, (K, N)).astype(np.float16)
    W[5, :] = 0
    for bits in range(1, 9):
        codes, s, z = orc.quantize(W, bits, G)
        s64 = np.repeat(s.astype(np.float64).T, G, axis=0)
        z64 = np.repeat(z.astype(np.float64).T, G, axis=0)
        deq = (codes.astype(np.float64) - z64) * s64
        assert np.all(np.abs(deq - W.astype(np.float64)) <= s64 * 1.0), bits
        assert np.all(deq[5, :] == 0), bits


ALL_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]
