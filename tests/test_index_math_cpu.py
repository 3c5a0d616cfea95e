"""The kernels' division-free group index, checked exhaustively on the host.

The kernels find the quantisation group of 32-code run r as
trunc((r + 1/2) * inv) with inv = 1 / gr rounded to fp32 (gr = G / 32 runs
per group) instead of the integer division r / gr.  The claim is that this is
exact for every run index the library can meet (K <= 2^21, so r < 2^16 + 8)
and every group size, also when the reciprocal is off by a few units in the
last place.  numpy's float32 multiply rounds to nearest even like the GPU's
v_mul_f32, and the float -> int conversion truncates like v_cvt_i32_f32.
"""
import numpy as np
import pytest

R_MAX = (1 << 16) + 8          # run indices: K <= 2^21 gives R <= 2^16, plus padding
R = np.arange(R_MAX, dtype=np.int64)
RF = R.astype(np.float32) + np.float32(0.5)   # exact in fp32


def group_index(gr: int, ulps: int) -> np.ndarray:
    inv = np.float32(1.0) / np.float32(gr)
    if ulps:
        inv = np.nextafter(inv, np.float32(np.inf if ulps > 0 else 0.0))
        for _ in range(abs(ulps) - 1):
            inv = np.nextafter(inv, np.float32(np.inf if ulps > 0 else 0.0))
    return np.trunc(RF * inv).astype(np.int64)


GROUPS = list(range(1, 257)) + [384, 416, 512, 1000, 1024, 2048, 4095, 4096, 8192, 32768, 65535, 65536]


@pytest.mark.parametrize("ulps", [0, -2, -1, 1, 2])
def test_run_group_matches_integer_division(ulps):
    for gr in GROUPS:
        got = group_index(gr, ulps)
        want = R // gr
        bad = np.nonzero(got != want)[0]
        assert bad.size == 0, f"gr={gr} ulps={ulps}: r={int(R[bad[0]])} gives {int(got[bad[0]])}, not {int(want[bad[0]])}"


def test_the_plain_product_would_fail():
    """Without the half-run offset, trunc(r * inv) goes wrong where r / gr is
    an integer and fp32(1 / gr) rounds below 1 / gr (gr = 41 is the first such
    group size): the check above would catch a dropped offset."""
    gr = 41
    inv = np.float32(1.0) / np.float32(gr)
    got = np.trunc(R.astype(np.float32) * inv).astype(np.int64)
    assert np.any(got != R // gr)
