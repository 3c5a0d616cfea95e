"""The quantiser kernels' rounding step, checked exhaustively on the host.

The kernels take round(w / s), ties to even (BitLLM Sec. 2.2, eq. (1)), as
t = rint(w * inv) with inv = 1 / s rounded to fp32, then fix only an exact
tie: the residual r = w - t s from one fma equals +-s / 2 there, and the
result is the even one of t and t + sign(r), 2 rint(t / 2 + sign(r) / 4).
The claim is that every code the kernel can form, clamp(round + z, 0,
2^k - 1) with 0 <= z <= 255, is then the same as with the exact quotient,
for every finite fp16 w and every positive fp16 s: equal rounding wherever
|w / s| <= 256.5, and beyond that a result past +-255 on the quotient's
side.  numpy's float32 multiply and rint round to nearest even like v_mul_f32
and v_rndne_f32; each fma is a float64 product and sum (exact for these
operands) rounded once to float32.
"""
import numpy as np
import pytest

H = np.arange(65536, dtype=np.uint32).astype(np.uint16).view(np.float16)
W16 = H[np.isfinite(H)]
S16 = H[np.isfinite(H) & (H > 0)]


def kernel_round(w32, w64, s16, tie_fix=True):
    s32, s64 = np.float32(s16), np.float64(s16)
    inv = np.float32(1.0) / s32
    half = np.float32(0.5) * s32
    t = np.rint(w32 * inv)
    if not tie_fix:
        return t
    r = (w64 - t.astype(np.float64) * s64).astype(np.float32)
    # at a tie, the even one of t and t + sign(r): 2 rint(t / 2 + sign(r) / 4),
    # the inner step one fma rounded to float32
    q4 = (t.astype(np.float64) * 0.5 + np.copysign(0.25, r).astype(np.float64)).astype(np.float32)
    even = np.float32(2.0) * np.rint(q4)
    return np.where(np.abs(r) == half, even, t)


def mismatches(tie_fix=True, step=1):
    w32, w64 = W16.astype(np.float32), W16.astype(np.float64)
    near = far = 0
    for s16 in S16[::step]:
        got = kernel_round(w32, w64, s16, tie_fix)
        q = w64 / np.float64(s16)
        exact = np.rint(q)   # exact: a half-integer quotient is representable, others sit far from one
        inr = np.abs(q) <= 256.5
        near += int(np.count_nonzero(inr & (got != exact)))
        far += int(np.count_nonzero(~inr & (((q > 0) & (got < 255)) | ((q < 0) & (got > -255)))))
    return near, far


def test_rounding_gives_every_code_exactly():
    """All 63488 finite fp16 w against all 31743 positive fp16 s."""
    assert mismatches() == (0, 0)


def test_without_the_tie_fix_it_would_fail():
    """Planted mistake: dropping the tie step leaves ties rounded wrongly (on
    a sample of s), so the check above would catch it."""
    near, _ = mismatches(tie_fix=False, step=97)
    assert near > 0
