"""The register decode of 3-, 5- and 7-bit float codes, run on the CPU.

The kernels have no conversion instruction for E1M1, E2M2 or E3M3 codes: they
spread a run's k-bit fields into 4- or 8-bit lanes with mask-and-shift steps,
move each sign to the lane's top bit, and convert the lanes as E2M1, E5M2 or
E4M3 values with a power-of-two scale.  This file replays those steps (the
constants of ``fp_small_run_to_half2`` in ``qmm_device.hpp``) on integers and
checks, for every code and for random runs, that the container values times
the scale are the oracle's code values: the field placement, the sign move
and the scale are all pinned here without a GPU.
"""
import numpy as np
import pytest

import oracle
import synthetic

# kernel format id -> (bits, codes per output dword, lane width, container, scale)
FORMATS = {4: (3, 8, 4, "e2m1", 2.0), 5: (5, 4, 8, "e5m2", 2.0 ** 14), 6: (7, 4, 8, "e4m3", 2.0 ** 4)}


def spread(x, fmt):
    """The kernels' mask-and-shift steps on one 32-bit window (Python ints)."""
    if fmt == 4:
        t = (x & 0x000FFF) | ((x & 0xFFF000) << 4)
        t = (t & 0x003F003F) | ((t & 0x0FC00FC0) << 2)
        t = (t & 0x07070707) | ((t & 0x38383838) << 1)
        t = (t & 0x33333333) | ((t & 0x44444444) << 1)
    elif fmt == 5:
        t = (x & 0x003FF) | ((x & 0xFFC00) << 6)
        t = (t & 0x001F001F) | ((t & 0x03E003E0) << 3)
        t = (t & 0x0F0F0F0F) | ((t & 0x10101010) << 3)
    else:
        t = (x & 0x0003FFF) | ((x & 0xFFFC000) << 2)
        t = (t & 0x007F007F) | ((t & 0x3F803F80) << 1)
        t = (t & 0x3F3F3F3F) | ((t & 0x40404040) << 1)
    return t & 0xFFFFFFFF


def container_value(v, kind):
    """Textbook decodes of the container formats (independent of the oracle)."""
    if kind == "e2m1":
        s, e, m = (v >> 3) & 1, (v >> 1) & 3, v & 1
        mag = m / 2.0 if e == 0 else 2.0 ** (e - 1) * (1 + m / 2.0)
    elif kind == "e5m2":
        s, e, m = (v >> 7) & 1, (v >> 2) & 31, v & 3
        mag = 2.0 ** -14 * m / 4.0 if e == 0 else 2.0 ** (e - 15) * (1 + m / 4.0)
    else:
        s, e, m = (v >> 7) & 1, (v >> 3) & 15, v & 7
        mag = 2.0 ** -6 * m / 8.0 if e == 0 else 2.0 ** (e - 7) * (1 + m / 8.0)
    return -mag if s else mag


def decode_run(stream_bits, fmt):
    """32 code values of one run (given as one integer of 32*k bits), the kernels' way."""
    bits, per, lane, kind, scale = FORMATS[fmt]
    vals = []
    for o in range(32 // per):
        x = (stream_bits >> (per * bits * o)) & 0xFFFFFFFF
        t = spread(x, fmt)
        for j in range(per):
            vals.append(container_value((t >> (lane * j)) & ((1 << lane) - 1), kind) * scale)
    return vals


@pytest.mark.parametrize("fmt", sorted(FORMATS))
def test_every_code_at_every_position(fmt):
    orc = oracle.default()
    bits = FORMATS[fmt][0]
    for code in range(1 << bits):
        want = orc.float_code_value(code, fmt)
        for pos in range(32):
            got = decode_run(code << (bits * pos), fmt)
            assert got[pos] == want, (code, pos)
            assert all(v == 0.0 for i, v in enumerate(got) if i != pos)


@pytest.mark.parametrize("fmt", sorted(FORMATS))
def test_random_runs_match_the_oracle(fmt):
    orc = oracle.default()
    bits = FORMATS[fmt][0]
    g = synthetic.rng(700 + fmt)
    for _ in range(200):
        codes = g.integers(0, 1 << bits, 32)
        stream = sum(int(c) << (bits * i) for i, c in enumerate(codes))
        got = decode_run(stream, fmt)
        assert got == [orc.float_code_value(int(c), fmt) for c in codes]
