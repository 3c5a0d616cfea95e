"""Host-side check of the generated in-register unpack (unpack_plan.inc).

The device code for each k is straight-line: views of the run made with
v_alignbit_b32 / shifts, then v_and_or_b32 (or v_perm_b32 for k = 8) building
two fp16 patterns per word.  Here that code is interpreted in Python with the
instructions' documented semantics and checked against the big-integer
definition of the stream: every half-slot must hold 0x6400 | (q << p) for the
code and shift the slot table names, every code exactly once, p + k <= 10.
"""
import os
import re

import numpy as np
import pytest

import brute

INC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                   "bit_weight_quantized_qmm_amd", "csrc", "unpack_plan.inc")
MASK32 = 0xFFFFFFFF


def alignbit(hi, lo, t):
    return (((hi << 32) | lo) >> (t & 31)) & MASK32


def perm(s0, s1, sel):
    src = (s0 << 32) | s1
    out = 0
    for i in range(4):
        b = (sel >> (8 * i)) & 0xFF
        if b < 8:
            v = (src >> (8 * b)) & 0xFF
        elif b == 12:
            v = 0
        elif b >= 13:
            v = 0xFF
        else:
            raise ValueError("sign-extension selectors are not used")
        out |= v << (8 * i)
    return out


def and_or(a, m, b):
    return ((a & m) | b) & MASK32


def parse():
    text = open(INC).read()
    plans = {}
    for k in range(1, 9):
        st = re.search(r"struct RunPlan<%d> \{(.*?)\n\};" % k, text, re.S).group(1)
        code = [int(v) for v in re.search(r"code\[32\] = \{([^}]*)\}", st).group(1).split(",")]
        pos = [int(v) for v in re.search(r"pos\[32\] = \{([^}]*)\}", st).group(1).split(",")]
        ops = int(re.search(r"ops = (\d+);", st).group(1))
        body = re.search(r"run_to_half2<%d>\(const uint32_t \(&d\)\[%d\], uint32_t \(&h\)\[16\]\)\n\{(.*?)\n\}" % (k, k),
                         text, re.S).group(1)
        plans[k] = (code, pos, ops, [l.strip() for l in body.strip().splitlines()])
    return plans


def run_plan(lines, d):
    env = {"d": list(d), "h": [None] * 16, "alignbit": alignbit, "perm": perm, "qmm_and_or": and_or}
    for line in lines:
        line = line.rstrip(";")
        line = re.sub(r"(0x[0-9a-fA-F]+)u\b", r"\1", line)
        line = line.replace("__builtin_amdgcn_alignbit", "alignbit").replace("__builtin_amdgcn_perm", "perm")
        line = line.replace("const uint32_t ", "")
        lhs, rhs = [p.strip() for p in line.split("=", 1)]
        val = eval(rhs, {}, env) & MASK32
        if lhs.startswith("h["):
            env["h"][int(lhs[2:-1])] = val
        else:
            env[lhs] = val
    return env["h"]


PLANS = parse()


@pytest.mark.parametrize("k", range(1, 9))
def test_slot_tables(k):
    code, pos, ops, _ = PLANS[k]
    assert sorted(code) == list(range(32))
    assert all(0 <= p and p + k <= 10 for p in pos)
    assert ops <= 32


@pytest.mark.parametrize("k", range(1, 9))
def test_generated_unpack_matches_stream_definition(k):
    code, pos, _, lines = PLANS[k]
    g = np.random.default_rng(77 + k)
    runs = [g.integers(0, 1 << k, size=32) for _ in range(64)]
    runs += [np.full(32, (1 << k) - 1), np.zeros(32, dtype=np.int64)]
    for q in runs:
        stream = brute.bigint_pack_column(q, k)                       # k*4 bytes
        d = [int.from_bytes(stream[4 * j:4 * j + 4], "little") for j in range(k)]
        h = run_plan(lines, d)
        for s in range(32):
            half = (h[s // 2] >> (16 * (s % 2))) & 0xFFFF
            assert half == (0x6400 | (int(q[code[s]]) << pos[s])), (k, s)
