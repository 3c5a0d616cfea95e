#!/usr/bin/env python3
"""Build step: plan the in-register conversion of one 32-code run into fp16 pairs.

A lane holds one run of 32 k-bit codes of a column as k dwords (32*k bits is
always exactly k dwords).  The kernels turn the run into 16 "half2" words in
which each 16-bit half is the fp16 bit pattern 0x6400 | (q << p): the value
1024 + q * 2^p, exact for any code q < 2^k as long as p + k <= 10 (the code
sits inside the 10-bit mantissa of an fp16 whose exponent makes one mantissa
unit worth 1).  The activation that meets this half is pre-scaled by 2^-p, so
the product contributes x * q plus a bias that does not depend on the code.

One VALU op v_and_or_b32 (src & mask) | 0x64006400 builds a whole pair when
both codes sit inside the 10-bit windows [w, w+10) and [w+16, w+26) of one
32-bit view of the stream starting at bit w.  A view at a dword boundary is
free (it is the loaded dword); any other view costs one v_alignbit_b32 (or one
shift at the ends of the run).  This script picks, for each k, the views and
the pairing that minimise VALU ops per run (ties: smaller total shift p), and
emits straight-line device code plus the slot tables that say which code and
which p each half holds.  For k = 8 one v_perm_b32 builds each pair directly.

Output: unpack_plan.inc (included by qmm_device.hpp).  Run without arguments to
regenerate; `--check` exits non-zero if the committed file is stale.
"""
from __future__ import annotations

import functools
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
OUT = os.path.join(HERE, "unpack_plan.inc")


def slots(k: int, w: int):
    lo = [i for i in range(32) if w <= k * i and k * i + k <= w + 10]
    hi = [i for i in range(32) if w + 16 <= k * i and k * i + k <= w + 26]
    return lo, hi


def solve(k: int, ws):
    """Best cover of the 32 codes by the views `ws`.

    Returns (ops, possum, items) where items are ('pair', w, lo, hi) or
    ('single', w, code, side).  Singles are later merged two at a time (one lo,
    one hi) into one half2 at one op each, so lo- and hi-singles must balance.
    """
    lo_of = {w: slots(k, w)[0] for w in ws}
    hi_of = {w: slots(k, w)[1] for w in ws}
    opts = {i: [] for i in range(32)}          # per code: ways to consume it first
    for w in ws:
        for a in lo_of[w]:
            opts[a].append(("single", w, a, 0))
            for b in hi_of[w]:
                opts[a].append(("pair", w, a, b))
        for b in hi_of[w]:
            opts[b].append(("single", w, b, 1))
            for a in lo_of[w]:
                opts[b].append(("pair", w, a, b))

    def pos(item):
        if item[0] == "pair":
            _, w, a, b = item
            return (k * a - w) + (k * b - w - 16)
        _, w, c, side = item
        return k * c - w - 16 * side

    @functools.lru_cache(None)
    def rec(rem: int, bal: int):
        if rem == 0:
            return (0, 0, ()) if bal == 0 else None
        i = (rem & -rem).bit_length() - 1
        best = None
        for it in opts[i]:
            if it[0] == "pair":
                other = it[3] if it[2] == i else it[2]
                if not (rem >> other) & 1 or other == i:
                    continue
                sub = rec(rem & ~(1 << i) & ~(1 << other), bal)
                cost = 1
            else:
                sub = rec(rem & ~(1 << i), bal + (1 if it[3] == 0 else -1))
                cost = 1
            if sub is None:
                continue
            cand = (sub[0] + cost, sub[1] + pos(it), sub[2] + (it,))
            if best is None or cand[:2] < best[:2]:
                best = cand
        return best

    r = rec((1 << 32) - 1, 0)
    rec.cache_clear()
    return r


def plan(k: int):
    free = [32 * j for j in range(k)]
    cands = [w for w in range(-9, 32 * k) if w not in free]

    def score(ws):
        r = solve(k, ws)
        if r is None:
            covered = set()
            for w in ws:
                lo, hi = slots(k, w)
                covered |= set(lo) | set(hi)
            return (10 ** 6 + 100 * (32 - len(covered)), 0), None
        extra = len([w for w in ws if w not in free])
        return (r[0] + extra, r[1]), r

    ws = list(free)
    cur, res = score(ws)
    while True:
        best, bw, br = cur, None, None
        for w in cands:
            if w in ws:
                continue
            sc, r = score(ws + [w])
            if sc < best:
                best, bw, br = sc, w, r
        if bw is None:
            break
        ws.append(bw)
        cur, res = best, br
    # drop views that the final cover does not use
    used = sorted({it[1] for it in res[2]})
    return used, res


def emit_generic(k: int, used, res):
    items = list(res[2])
    pairs = [it for it in items if it[0] == "pair"]
    lo_s = [it for it in items if it[0] == "single" and it[3] == 0]
    hi_s = [it for it in items if it[0] == "single" and it[3] == 1]
    assert len(lo_s) == len(hi_s) and len(pairs) + len(lo_s) == 16
    words = []   # (lo view, lo code, lo pos, hi view, hi code, hi pos)
    for _, w, a, b in pairs:
        words.append((w, a, k * a - w, w, b, k * b - w - 16))
    for (_, wa, a, _), (_, wb, b, _) in zip(sorted(lo_s, key=lambda t: t[2]), sorted(hi_s, key=lambda t: t[2])):
        words.append((wa, a, k * a - wa, wb, b, k * b - wb - 16))
    words.sort(key=lambda t: (t[1], t[4]))
    lines = []

    def view(w):
        if w % 32 == 0:
            return f"d[{w // 32}]"
        return f"v{w if w >= 0 else 'm' + str(-w)}"

    for w in used:
        if w % 32 == 0:
            continue
        j, t = divmod(w, 32)
        name = view(w)
        if w < 0:
            lines.append(f"    const uint32_t {name} = d[0] << {-w};")
        elif j + 1 < k:
            lines.append(f"    const uint32_t {name} = __builtin_amdgcn_alignbit(d[{j + 1}], d[{j}], {t});")
        else:
            lines.append(f"    const uint32_t {name} = d[{j}] >> {t};")
    cm = (1 << k) - 1
    for idx, (wl, a, pl, wh, b, ph) in enumerate(words):
        ml, mh = cm << pl, cm << (16 + ph)
        assert 0 <= pl and pl + k <= 10 and 0 <= ph and ph + k <= 10
        if wl == wh:
            lines.append(f"    h[{idx}] = qmm_and_or({view(wl)}, 0x{ml | mh:08x}u, 0x64006400u);")
        else:
            lines.append(f"    h[{idx}] = qmm_and_or({view(wl)}, 0x{ml:08x}u, "
                         f"qmm_and_or({view(wh)}, 0x{mh:08x}u, 0x64006400u));")
    code = [0] * 32
    pos = [0] * 32
    for idx, (wl, a, pl, wh, b, ph) in enumerate(words):
        code[2 * idx], pos[2 * idx], code[2 * idx + 1], pos[2 * idx + 1] = a, pl, b, ph
    nviews = len([w for w in used if w % 32])
    ops = nviews + sum(1 if t[0] == t[3] else 2 for t in words)
    return lines, code, pos, ops


def emit_k8():
    lines, code, pos = [], [0] * 32, [0] * 32
    for j in range(8):
        lines.append(f"    h[{2 * j}] = __builtin_amdgcn_perm(d[{j}], 0x64646464u, 0x00060004u);")
        lines.append(f"    h[{2 * j + 1}] = __builtin_amdgcn_perm(d[{j}], 0x64646464u, 0x00070005u);")
        for h, (a, b) in enumerate(((0, 2), (1, 3))):
            s = 2 * (2 * j + h)
            code[s], code[s + 1] = 4 * j + a, 4 * j + b
    return lines, code, pos, 16


def render() -> str:
    out = [
        "// Generated by gen_unpack_plan.py -- do not edit by hand.",
        "//",
        "// run_to_half2<k>(d, h): the 32 k-bit codes of one run (k dwords, LSB-first",
        "// stream) -> 16 words of two fp16 bit patterns 0x6400 | (q << p) each.",
        "// RunPlan<k>::code[s] / pos[s]: code index (0..31 inside the run) and shift p",
        "// held by half-slot s = 2*word + (0 = low half, 1 = high half).",
        "// RunPlan<k>::ops: VALU ops per run spent by run_to_half2.",
        "",
        "template <int BITS> struct RunPlan;",
        "template <int BITS> __device__ __forceinline__ void run_to_half2(const uint32_t (&d)[BITS], uint32_t (&h)[16]);",
        "",
    ]
    for k in range(1, 9):
        if k == 8:
            lines, code, pos, ops = emit_k8()
        else:
            used, res = plan(k)
            lines, code, pos, ops = emit_generic(k, used, res)
        assert sorted(code) == list(range(32)), k
        out.append(f"template <> struct RunPlan<{k}> {{")
        out.append(f"    static constexpr int ops = {ops};")
        out.append("    static constexpr uint8_t code[32] = {" + ", ".join(map(str, code)) + "};")
        out.append("    static constexpr uint8_t pos[32] = {" + ", ".join(map(str, pos)) + "};")
        out.append("};")
        out.append("template <>")
        out.append(f"__device__ __forceinline__ void run_to_half2<{k}>(const uint32_t (&d)[{k}], uint32_t (&h)[16])")
        out.append("{")
        out.extend(lines)
        out.append("}")
        out.append("")
    return "\n".join(out)


def main(argv):
    text = render()
    if "--check" in argv:
        cur = open(OUT).read() if os.path.exists(OUT) else ""
        if cur != text:
            print("unpack_plan.inc is stale; run gen_unpack_plan.py", file=sys.stderr)
            return 1
        return 0
    with open(OUT, "w") as fh:
        fh.write(text)
    return 0


if __name__ == "__main__":
    sys.exit(main(sys.argv[1:]))
