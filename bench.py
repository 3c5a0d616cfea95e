#!/usr/bin/env python3
"""Throughput of the k-bit weight-quantized matmul on one MI355X.

Workload (one "step"): the decode product Y[1, 11008] = x[1, 4096] . dequant(Wq)
for 7B-MLP-shaped weights at k = 3, 4 and 6 bits, G = 128 (three qmm_gemv
launches).  Inputs are seeded synthetic data already resident in HBM; each
launch reads its own copy of the packed weights and scales out of a rotating
set larger than 1 GiB, so no launch finds its weights in the 256 MB Infinity
Cache or the L2 (the pages' protocol clears the cache between runs; here every
launch simply reads weights nothing else has touched recently).

Timing: two HIP events on the launch stream (torch's current stream) bracket
a region of back-to-back launches; the stream is first held by a spin kernel
so the host queues the whole region before the GPU starts it.  `value` is
packed-weight bytes per second over K steps.  Each kernel is then timed alone
over K back-to-back launches; the `roofline` object prices the dominant
kernel's algorithmic bytes (packed weights + scales + x + y) per launch
against that mean launch duration and the 8 TB/s HBM peak.  The same JSON line carries the M = 2048
prefill product (qmm_gemm) in TFLOP/s against the 2.5 PFLOP/s dense fp16 MFMA
peak, the batched-decode (70B MLP-up shapes, M = 1, 8, 16, k = 1, 2, 5, 7, 8) and
W4A8 / W8A8 (8B MLP shapes, M = 16, 4- and 8-bit weights) products and the
quantiser (7B MLP weight) as a "suite" object, and the CPU oracle timed on
this host on a bounded sample.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu] [--no-suite]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, HERE)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
FP16_MFMA_PEAK_TFS = 2516.6    # MI355X dense fp16 MFMA, published (2.5 PFLOP/s)
INT8_MFMA_PEAK_TOPS = 5033.2
METRIC = "packed-weight HBM GB/s (% peak) at M=1; TFLOP/s (% MFMA peak) at M=2048"
ROTATE_BYTES = 1 << 30
PROFILE_TRAFFIC = os.path.join(HERE, "profiles", "traffic.json")
PROFILE_VALU = os.path.join(HERE, "profiles", "valu.json")
# VALU issue peak: 256 CUs x 4 SIMDs x 2.4 GHz, one wave64 VALU instruction per
# 4 cycles on a 16-lane SIMD = 614.4 G instructions/s = 39.3 T lane-ops/s
VALU_PEAK_TLANEOPS = 256 * 4 * 2.4e9 / 4 * 64 / 1e12


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU-oracle baseline leg")
    ap.add_argument("--no-suite", action="store_true", help="skip the suite (batched decode, int8 activations, quantiser, float codes)")
    ap.add_argument("--copy-probe", action="store_true", help="run a plain 1 GiB device copy (counter calibration)")
    ap.add_argument("--only", default=None,
                    help="run one leg and print its JSON (for profiling): decode, grouped, gemm, batched, w4a8, w8a8, w4a8p, "
                         "quantize, fp, lut, probes")
    ap.add_argument("--bits", type=int, default=None, help="with --only: restrict to one code width")
    ap.add_argument("--M", type=int, default=None, help="with --only batched: restrict to one M")
    return ap.parse_args()


# Sources each profiled kernel is built from: a counter run stays valid for a
# kernel only while these files are unchanged.
KERNEL_SOURCES = {
    "gemv_m1": ("gemv.hip", "qmm_device.hpp", "unpack_plan.inc", "launch.hpp"),
    "lut": ("lut.hip", "qmm_device.hpp", "launch.hpp"),
    "gemm": ("gemm.hip", "qmm_device.hpp", "unpack_plan.inc", "launch.hpp"),
    "w4a8": ("w4a8.hip", "qmm_device.hpp", "launch.hpp"),
    "quantize": ("quantize.hip", "qmm_device.hpp", "launch.hpp"),
}


def source_digest(names=None) -> str:
    """sha256 (16 hex digits) over the named kernel sources, all of them by default."""
    h = hashlib.sha256()
    csrc = os.path.join(HERE, "bit_weight_quantized_qmm_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        if name.endswith((".hip", ".hpp", ".cpp", ".inc")) and (names is None or name in names):
            h.update(name.encode())
            h.update(open(os.path.join(csrc, name), "rb").read())
    return h.hexdigest()[:16]


class Timer:
    """HIP events on the launch stream (torch's current stream) bracketing a
    region of back-to-back launches.  The stream is first held by a spin
    kernel so the host can queue the whole region before the GPU starts it;
    the region then measures GPU time only (kernels plus the dispatch gaps
    between consecutive kernels on one stream)."""

    def __init__(self, torch):
        self.torch = torch
        self.quick = False   # --only runs (under a profiler): a few regions instead of 50

    def region_ms(self, launch, count):
        torch = self.torch
        torch.cuda.synchronize()
        torch.cuda._sleep(200_000_000)
        ev0 = torch.cuda.Event(enable_timing=True)
        ev1 = torch.cuda.Event(enable_timing=True)
        ev0.record()
        for i in range(count):
            launch(i)
        ev1.record()
        torch.cuda.synchronize()
        return ev0.elapsed_time(ev1)

    def median_us(self, launch, per_region=10, regions=50):
        """Median and mean per-launch time (us) over `regions` regions of
        `per_region` back-to-back launches each (the median of 50 of the
        pages' protocol, taken over short regions because a single launch is
        too short to bracket with events without inflating it)."""
        torch = self.torch
        if self.quick:
            regions = min(regions, 2)
        vals = []
        for r in range(regions):
            torch.cuda.synchronize()
            torch.cuda._sleep(20_000_000)
            ev0 = torch.cuda.Event(enable_timing=True)
            ev1 = torch.cuda.Event(enable_timing=True)
            ev0.record()
            for i in range(per_region):
                launch(r * per_region + i)
            ev1.record()
            torch.cuda.synchronize()
            vals.append(ev0.elapsed_time(ev1) * 1e3 / per_region)
        vals.sort()
        return float(np.median(vals)), float(np.mean(vals))


def decode_setup(torch, q, synthetic, bits):
    w = synthetic.DECODE_7B
    c = synthetic.make_case(1, w["K"], w["N"], bits, w["G"], synthetic.seed_for(2, bits), s_range=w["s_range"])
    dev = "cuda:0"
    wq0 = q.pack(torch.from_numpy(c["codes"]).to(dev), bits)
    s0 = torch.from_numpy(c["s"]).to(dev)
    per = wq0.numel() * 4 + s0.numel() * 2
    copies = max(2, -(-ROTATE_BYTES // per))
    bufs = [(wq0.clone(), s0.clone()) for _ in range(copies)]
    del wq0
    x = torch.from_numpy(c["X"]).to(dev)
    y = torch.empty((1, w["N"]), dtype=torch.float16, device=dev)
    wq_bytes = w["N"] * w["K"] * bits // 8
    alg = wq_bytes + s0.numel() * 2 + x.numel() * 2 + y.numel() * 2
    return dict(bits=bits, bufs=bufs, x=x, y=y, K=w["K"], N=w["N"], G=w["G"], wq_bytes=wq_bytes, alg_bytes=alg,
                case=c, i=0)


def decode_launch(q, d):
    wq, s = d["bufs"][d["i"] % len(d["bufs"])]
    d["i"] += 1
    q.gemv(d["x"], wq, s, None, d["bits"], d["G"], out=d["y"])


def grouped_launch(q, decs):
    """The decode step as one qmm_gemv_grouped launch over the three products,
    each reading its next rotating copy of the weights."""
    probs = []
    for d in decs:
        wq, s = d["bufs"][d["i"] % len(d["bufs"])]
        d["i"] += 1
        probs.append((d["x"], wq, s, None, d["bits"]))
    q.gemv_grouped(probs, decs[0]["G"], outs=[d["y"] for d in decs])


def traffic_for(kernel_key):
    """HBM bytes per launch (FETCH_SIZE + WRITE_SIZE, calibrated) from the
    committed rocprofv3 counter runs, or None unless those runs were taken on
    the kernel's current sources."""
    try:
        with open(PROFILE_TRAFFIC) as fh:
            t = json.load(fh)
    except (OSError, ValueError):
        return None
    e = t.get("kernels", {}).get(kernel_key)
    if e is None:
        return None
    family = e.get("family")
    if family not in KERNEL_SOURCES or e.get("source_digest") != source_digest(KERNEL_SOURCES[family]):
        return None
    return e.get("bytes_per_launch")


def valu_for(kernel_key):
    """VALU instructions per launch (rocprofv3 SQ_INSTS_VALU, summed over the
    GPU) from the committed counter run, or None unless it was taken on the
    kernel's current sources."""
    try:
        with open(PROFILE_VALU) as fh:
            t = json.load(fh)
    except (OSError, ValueError):
        return None
    e = t.get("kernels", {}).get(kernel_key)
    if e is None:
        return None
    family = e.get("family")
    if family not in KERNEL_SOURCES or e.get("source_digest") != source_digest(KERNEL_SOURCES[family]):
        return None
    return e.get("valu_insts_per_launch")


def alu_roofline(kernel_key, us, codes):
    """The plain-ALU roofline of a launch: VALU lane-ops per second against the
    VALU issue peak, and lane-ops per weight code."""
    insts = valu_for(kernel_key)
    if insts is None:
        return None
    achieved = insts * 64 / (us * 1e-6) / 1e12
    return {"bound": "alu", "achieved": round(achieved, 2), "peak": round(VALU_PEAK_TLANEOPS, 2), "unit": "Tlane-op/s",
            "frac": round(achieved / VALU_PEAK_TLANEOPS, 4), "valu_lane_ops_per_code": round(insts * 64 / codes, 3)}


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(synthetic, budget_s=12.0):
    """The oracle as it stands, timed on this host.  `value`: the same decode
    step as the GPU's (k = 3, 4, 6) repeated until about budget_s seconds have
    passed.  `configs`: one timing each of the tiny case, one 70B MLP-up
    batched-decode row, the W4A8 product and a bounded row sample of the
    prefill product (scaled to the full shape), each a few seconds at most."""
    import oracle
    cores = int(os.environ.get("OMP_NUM_THREADS", len(os.sched_getaffinity(0))))
    orc = oracle.default()
    w = synthetic.DECODE_7B
    cases = []
    for bits in w["bits"]:
        c = synthetic.make_case(1, w["K"], w["N"], bits, w["G"], synthetic.seed_for(2, bits), s_range=w["s_range"])
        cases.append((c, orc.pack(c["codes"], bits)))
    done_bytes, reps = 0, 0
    t0 = time.perf_counter()
    while True:
        for c, st in cases:
            orc.qmm(c["X"], st, c["s"], None, c["bits"], c["G"])
            done_bytes += st.size
        reps += 1
        if time.perf_counter() - t0 >= budget_s:
            break
    dt = time.perf_counter() - t0
    del cases
    configs = {}

    def timed(fn):
        t = time.perf_counter()
        fn()
        return time.perf_counter() - t

    t = synthetic.TINY
    c = synthetic.make_case(1, t["K"], t["N"], 4, t["G"], synthetic.seed_for(1, 4), s_range=t["s_range"])
    st = orc.pack(c["codes"], 4)
    n = 200
    sec = timed(lambda: [orc.qmm(c["X"], st, c["s"], None, 4, t["G"]) for _ in range(n)]) / n
    configs["tiny"] = {"workload": t["name"], "ms": round(sec * 1e3, 4), "packed_GBs": round(st.size / sec / 1e9, 4)}
    b = synthetic.BATCHED_70B
    c = synthetic.make_case(1, b["K"], b["N"], 1, b["G"], synthetic.seed_for(3, 1), per_group_z=True, s_range=b["s_range"])
    st = orc.pack(c["codes"], 1)
    del c["codes"]
    sec = timed(lambda: orc.qmm(c["X"], st, c["s"], c["z"], 1, b["G"]))
    configs["batched_70b_k1_M1"] = {"workload": "batched-decode 70B-MLP-up M1 K8192 N28672 k1 G128 per-group z",
                                    "ms": round(sec * 1e3, 2), "packed_GBs": round(st.size / sec / 1e9, 4)}
    del st
    a = synthetic.W4A8_8B
    c = synthetic.make_w4a8_case(a["M"], a["K"], a["N"], a["G"], synthetic.seed_for(5, 4), s_range=a["s_range"])
    st = orc.pack(c["codes"], 4)
    del c["codes"]
    sec = timed(lambda: orc.w4a8(c["Xq"], c["sx"], st, c["s"], None, a["G"]))
    configs["w4a8_8b"] = {"workload": a["name"], "ms": round(sec * 1e3, 2), "packed_GBs": round(st.size / sec / 1e9, 4),
                          "GOPs": round(2.0 * a["M"] * a["K"] * a["N"] / sec / 1e9, 3)}
    del st
    p = synthetic.PREFILL
    c = synthetic.make_case(p["M"], p["K"], p["N"], 4, p["G"], synthetic.seed_for(4, 4), s_range=p["s_range"])
    st = orc.pack(c["codes"], 4)
    rows = 16
    sec = timed(lambda: orc.qmm(c["X"][:rows], st, c["s"], None, 4, p["G"]))
    full = sec * p["M"] / rows
    configs["prefill"] = {"workload": p["name"], "sample": f"{rows} of {p['M']} rows, time scaled to all rows",
                          "s_full_estimate": round(full, 2), "GFLOPs": round(2.0 * p["M"] * p["K"] * p["N"] / full / 1e9, 3)}
    return {"value": round(done_bytes / dt / 1e9, 4), "unit": "GB/s", "cores": cores, "cpu_model": cpu_model(),
            "kind": "oracle",
            "sample": f"{reps} x the full decode step (k=3,4,6; M=1 K=4096 N=11008): bit-serial unpack, "
                      f"fp64 dequant and fp64 dot products, {dt:.1f} s wall",
            "configs": configs}


def rotating(torch, tensors):
    """Enough copies of the weight-side tensors that the copies together exceed
    1 GiB, so consecutive launches never find their weights in a cache."""
    per = sum(t.numel() * t.element_size() for t in tensors)
    copies = max(2, -(-ROTATE_BYTES // per))
    return [tuple(t.clone() for t in tensors) for _ in range(copies)]


def batched_suite(torch, q, synthetic, timer, reps, only_bits=None, only_m=None):
    """70B MLP-up batched decode (K 8192, N 28672, G 128, per-group z) at M = 1, 8, 16
    for k = 1, 2, 5, 7, 8: us per launch and HBM GB/s of the algorithmic bytes."""
    w = synthetic.BATCHED_70B
    K, N, G = w["K"], w["N"], w["G"]
    out = {}
    for bits in w["bits"]:
        if only_bits is not None and bits != only_bits:
            continue
        c = synthetic.make_case(max(w["Ms"]), K, N, bits, G, synthetic.seed_for(3, bits), per_group_z=True,
                                s_range=w["s_range"])
        wq = q.pack(torch.from_numpy(c["codes"]).to("cuda:0"), bits)
        bufs = rotating(torch, (wq, torch.from_numpy(c["s"]).to("cuda:0"), torch.from_numpy(c["z"]).to("cuda:0")))
        del wq, c["codes"]
        X = torch.from_numpy(c["X"]).to("cuda:0")
        row = {}
        for M in w["Ms"]:
            if only_m is not None and M != only_m:
                continue
            x = X[:M].contiguous()
            y = torch.empty((M, N), dtype=torch.float16, device="cuda:0")
            state = {"i": 0}

            def launch(i, x=x, y=y, state=state):
                b = bufs[state["i"] % len(bufs)]
                state["i"] += 1
                q.gemv(x, b[0], b[1], b[2], bits, G, out=y)

            for i in range(3):
                launch(i)
            ms = timer.region_ms(launch, reps) / reps
            wq_bytes = N * K * bits // 8
            alg = wq_bytes + 2 * N * (K // G) * 2 + M * K * 2 + M * N * 2
            row[f"M{M}"] = {"us": round(ms * 1e3, 2), "packed_GBs": round(wq_bytes / ms / 1e6, 1),
                            "algorithmic_GBs": round(alg / ms / 1e6, 1),
                            "algorithmic_frac_of_hbm_peak": round(alg / ms / 1e6 / HBM_PEAK_GBS, 4)}
            if bits <= 2:
                row[f"M{M}"]["alu_roofline"] = alu_roofline(f"batched_70b_k{bits}_m{M}", ms * 1e3, K * N)
        out[f"k{bits}"] = row
        del bufs
        torch.cuda.empty_cache()
    return {"workload": w["name"], "per_bits": out}


def w4a8_suite(torch, q, synthetic, timer, reps, bits=4):
    """8B MLP int8-activation product (M 16, K 4096, N 14336, G 128): W4A8 at
    bits = 4 (qmm_gemm_w4a8), W8A8 at bits = 8 (qmm_gemm_wka8)."""
    w = synthetic.W4A8_8B
    M, K, N, G = w["M"], w["K"], w["N"], w["G"]
    c = synthetic.make_w4a8_case(M, K, N, G, synthetic.seed_for(5, bits), bits=bits, s_range=w["s_range"])
    wq = q.pack(torch.from_numpy(c["codes"]).to("cuda:0"), bits)
    bufs = rotating(torch, (wq, torch.from_numpy(c["s"]).to("cuda:0")))
    del wq
    Xq = torch.from_numpy(c["Xq"]).to("cuda:0")
    sx = torch.from_numpy(c["sx"]).to("cuda:0")
    y = torch.empty((M, N), dtype=torch.float16, device="cuda:0")
    state = {"i": 0}

    def launch(i):
        b = bufs[state["i"] % len(bufs)]
        state["i"] += 1
        if bits == 4:
            q.gemm_w4a8(Xq, sx, b[0], b[1], None, G, out=y)
        else:
            q.gemm_wka8(Xq, sx, b[0], b[1], None, bits, G, out=y)

    for i in range(3):
        launch(i)
    ms = timer.region_ms(launch, reps) / reps
    wq_bytes = N * K * bits // 8
    alg = wq_bytes + N * (K // G) * 2 + M * K + M * 2 + M * N * 2
    name = w["name"] if bits == 4 else w["name"].replace("w4a8", f"w{bits}a8").replace(" k4 ", f" k{bits} ")
    return {"workload": name, "us": round(ms * 1e3, 2), "packed_GBs": round(wq_bytes / ms / 1e6, 1),
            "algorithmic_GBs": round(alg / ms / 1e6, 1),
            "algorithmic_frac_of_hbm_peak": round(alg / ms / 1e6 / HBM_PEAK_GBS, 4),
            "TOPs": round(2.0 * M * N * K / ms / 1e9, 2)}


def w4a8_prefill_suite(torch, q, synthetic, timer, reps):
    """W4A8 at prefill size (M 2048, K = N = 4096, k 4, G 128; the tiled i8-MFMA
    kernel): TOPS against the dense int8 MFMA peak, Xq, Wq and s rotated."""
    w = synthetic.PREFILL
    M, K, N, G = w["M"], w["K"], w["N"], w["G"]
    c = synthetic.make_w4a8_case(M, K, N, G, synthetic.seed_for(5, 4, 7), s_range=w["s_range"])
    wq = q.pack(torch.from_numpy(c["codes"]).to("cuda:0"), 4)
    bufs = rotating(torch, (torch.from_numpy(c["Xq"]).to("cuda:0"), wq, torch.from_numpy(c["s"]).to("cuda:0")))
    del wq
    sx = torch.from_numpy(c["sx"]).to("cuda:0")
    y = torch.empty((M, N), dtype=torch.float16, device="cuda:0")
    state = {"i": 0}

    def launch(i):
        b = bufs[state["i"] % len(bufs)]
        state["i"] += 1
        q.gemm_w4a8(b[0], sx, b[1], b[2], None, G, out=y)

    for i in range(3):
        launch(i)
    ms = timer.region_ms(launch, reps) / reps
    med, _ = timer.median_us(launch, 5, 50)
    tops = 2.0 * M * N * K / (ms * 1e-3) / 1e12
    del bufs
    torch.cuda.empty_cache()
    return {"workload": f"w4a8 prefill M{M} K{K} N{N} k4 G{G}", "cache": "cold (rotating Xq, Wq, s copies > 1 GiB)",
            "us": round(ms * 1e3, 2), "us_median_of_50": round(med, 2), "TOPs": round(tops, 1),
            "frac_of_int8_mfma_peak": round(tops / INT8_MFMA_PEAK_TOPS, 4)}


FP_NAMES = {0: "E2M1", 1: "E4M3", 2: "E3M2", 3: "E2M3", 4: "E1M1", 5: "E2M2", 6: "E3M3"}
FP_BITS = {0: 4, 1: 8, 2: 6, 3: 6, 4: 3, 5: 5, 6: 7}


def gemm_fp_suite(torch, q, synthetic, timer, reps, fmt):
    """qmm_gemm_fp on the prefill shape (M 2048, K = N = 4096, G 128) with E2M1
    (fmt 0), E4M3 (fmt 1) or E3M2 (fmt 2) codes: TFLOP/s against the dense fp16 MFMA peak."""
    w = synthetic.PREFILL
    M, K, N, G = w["M"], w["K"], w["N"], w["G"]
    bits = FP_BITS[fmt]
    g = synthetic.rng(synthetic.seed_for(4, bits, 11 + fmt))
    codes = g.integers(0, 1 << bits, (K, N))
    if fmt == 1:
        codes[(codes & 0x7F) == 0x7F] = 0x30
    wq = q.pack(torch.from_numpy(codes.astype(np.uint8)).to("cuda:0"), bits)
    s = torch.from_numpy(synthetic.fp16_uniform(g, 0.002, 0.02, (N, K // G))).to("cuda:0")
    X = torch.from_numpy(synthetic.fp16_normal(g, (M, K))).to("cuda:0")
    Y = torch.empty((M, N), dtype=torch.float16, device="cuda:0")
    bufs = rotating(torch, (X, wq, s))
    state = {"i": 0}

    def launch(i):
        b = bufs[state["i"] % len(bufs)]
        state["i"] += 1
        q.gemm_fp(b[0], b[1], b[2], fmt, G, out=Y)

    for _ in range(3):
        launch(0)
    ms = timer.region_ms(launch, reps) / reps
    tfs = 2.0 * M * N * K / (ms * 1e-3) / 1e12
    del bufs
    torch.cuda.empty_cache()
    return {"workload": f"prefill-gemm {FP_NAMES[fmt]} codes M{M} K{K} N{N} G{G}",
            "cache": "cold (rotating X, Wq, s copies > 1 GiB)",
            "us": round(ms * 1e3, 2), "TFLOPs": round(tfs, 1), "frac_of_fp16_mfma_peak": round(tfs / FP16_MFMA_PEAK_TFS, 4)}


def decode_fp_suite(torch, q, synthetic, timer, reps, fmt):
    """qmm_gemm_fp at M = 1, 8, 16 on the 7B MLP shape (K 4096, N 11008, G 128)
    with E2M1 (fmt 0), E4M3 (fmt 1) or E3M2 (fmt 2) codes: weights streamed from HBM
    (rotating copies); HBM GB/s of the algorithmic bytes."""
    w = synthetic.DECODE_7B
    K, N, G = w["K"], w["N"], w["G"]
    bits = FP_BITS[fmt]
    g = synthetic.rng(synthetic.seed_for(2, bits, 13 + fmt))
    codes = g.integers(0, 1 << bits, (K, N))
    if fmt == 1:
        codes[(codes & 0x7F) == 0x7F] = 0x30
    wq = q.pack(torch.from_numpy(codes.astype(np.uint8)).to("cuda:0"), bits)
    s = torch.from_numpy(synthetic.fp16_uniform(g, 0.002, 0.02, (N, K // G))).to("cuda:0")
    bufs = rotating(torch, (wq, s))
    X = torch.from_numpy(synthetic.fp16_normal(g, (16, K))).to("cuda:0")
    out = {"workload": f"decode {FP_NAMES[fmt]} codes 7B-MLP K{K} N{N} G{G}"}
    for M in (1, 8, 16):
        x = X[:M].contiguous()
        Y = torch.empty((M, N), dtype=torch.float16, device="cuda:0")
        state = {"i": 0}

        def launch(i, x=x, Y=Y, state=state):
            b = bufs[state["i"] % len(bufs)]
            state["i"] += 1
            q.gemm_fp(x, b[0], b[1], fmt, G, out=Y)

        for i in range(3):
            launch(i)
        ms = timer.region_ms(launch, reps) / reps
        alg = K * N * bits // 8 + N * (K // G) * 2 + M * K * 2 + M * N * 2
        out[f"M{M}"] = {"us": round(ms * 1e3, 2), "algorithmic_GBs": round(alg / ms / 1e6, 1),
                        "algorithmic_frac_of_hbm_peak": round(alg / ms / 1e6 / HBM_PEAK_GBS, 4)}
    return out


def quantize_suite(torch, q, synthetic, timer, reps):
    """qmm_quantize on the 7B MLP weight (K 4096, N 11008, G 128, k 4): fp16 W in,
    codes, s and z out; HBM-bound."""
    w = synthetic.DECODE_7B
    K, N, G, bits = w["K"], w["N"], w["G"], 4
    g = synthetic.rng(synthetic.seed_for(2, bits, 9))
    W = (torch.from_numpy(synthetic.fp16_normal(g, (K, N))).to("cuda:0") * 0.02).to(torch.float16)
    per = K * N * 2
    Ws = [W] + [W.clone() for _ in range(max(1, -(-(1 << 30) // per)) - 1)]
    codes = torch.empty((K, N), dtype=torch.uint8, device="cuda:0")
    s = torch.empty((N, K // G), dtype=torch.float16, device="cuda:0")
    z = torch.empty_like(s)
    state = {"i": 0}

    def launch(i):
        state["i"] += 1
        q.quantize(Ws[state["i"] % len(Ws)], bits, G, codes=codes, s=s, z=z)

    for i in range(3):
        launch(i)
    ms = timer.region_ms(launch, reps) / reps
    alg = K * N * 2 + K * N + N * (K // G) * 4
    return {"workload": f"quantize 7B-MLP K{K} N{N} k{bits} G{G}", "us": round(ms * 1e3, 2),
            "algorithmic_GBs": round(alg / ms / 1e6, 1),
            "algorithmic_frac_of_hbm_peak": round(alg / ms / 1e6 / HBM_PEAK_GBS, 4)}


def probes_leg(torch, q, timer):
    """Measured ceilings on this GPU: a plain streaming read of the decode
    weights' sizes (and of 1 GiB) from HBM, and back-to-back f16 MFMAs on
    register operands.  Reported beside the datasheet peaks, never instead."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    big = torch.empty(3 << 28, dtype=torch.int32, device="cuda:0").fill_(7)   # 3 GiB, rotated through
    total = big.numel() * 4
    out = {"read": {}, "mfma": {}}
    sink = torch.empty(cus * 16 * 256, dtype=torch.int32, device="cuda:0")
    for name, nbytes in (("7B_k3_16.9MB", 16908288), ("7B_k4_22.5MB", 22544384), ("7B_k6_33.8MB", 33816576),
                         ("7B_step_73.3MB", 16908288 + 22544384 + 33816576), ("1GiB", 1 << 30)):
        best = None
        for wpc in (1, 2, 4, 8, 16):
            grid = cus * wpc
            nslices = max(2, total // nbytes - 1)
            state = {"i": 0}

            def launch(i, nbytes=nbytes, grid=grid, nslices=nslices, state=state):
                off = (state["i"] % nslices) * nbytes
                state["i"] += 1
                q.probe_read(big.view(torch.uint8)[off:off + nbytes], grid, sink)

            launch(0)
            per = 4 if nbytes >= (1 << 30) else 10
            med, mean = timer.median_us(launch, per_region=per, regions=10 if nbytes >= (1 << 30) else 30)
            r = {"workgroups_per_cu": wpc, "us_median": round(med, 3), "GBs": round(nbytes / med / 1e3, 1)}
            if best is None or r["GBs"] > best["GBs"]:
                best = r
        best["frac_of_datasheet"] = round(best["GBs"] / HBM_PEAK_GBS, 4)
        out["read"][name] = best
    del big
    torch.cuda.empty_cache()
    msink = torch.empty(cus * 2 * 512, dtype=torch.float32, device="cuda:0")
    for shape, name in ((0, "f16_16x16x32"), (1, "f16_32x32x16")):
        best = None
        for wpc in (1, 2):
            grid = cus * wpc
            iters = 4096 // wpc
            flops = q.probe_mfma(iters, grid, shape, msink)
            med, mean = timer.median_us(lambda i: q.probe_mfma(iters, grid, shape, msink), per_region=3, regions=10)
            tfs = flops / (med * 1e-6) / 1e12
            r = {"workgroups_per_cu": wpc, "us_median": round(med, 2), "TFLOPs": round(tfs, 1)}
            if best is None or r["TFLOPs"] > best["TFLOPs"]:
                best = r
        best["frac_of_datasheet"] = round(best["TFLOPs"] / FP16_MFMA_PEAK_TFS, 4)
        out["mfma"][name] = best
    return out


def blas_context(torch, timer):
    """The library fp16 GEMM (torch.matmul -> hipBLASLt) on the prefill shape
    with dense fp16 weights: context for the quantised GEMM, not part of the path."""
    M, K, N = 2048, 4096, 4096
    g = torch.Generator(device="cuda:0").manual_seed(5)
    A = torch.randn((M, K), device="cuda:0", dtype=torch.float16, generator=g)
    B = torch.randn((K, N), device="cuda:0", dtype=torch.float16, generator=g)
    C = torch.empty((M, N), device="cuda:0", dtype=torch.float16)
    for _ in range(3):
        torch.matmul(A, B, out=C)
    med, mean = timer.median_us(lambda i: torch.matmul(A, B, out=C), per_region=5, regions=20)
    tfs = 2.0 * M * N * K / (med * 1e-6) / 1e12
    return {"workload": "torch.matmul fp16 M2048 K4096 N4096 (dense weights, warm caches)", "us_median": round(med, 2),
            "TFLOPs": round(tfs, 1), "frac_of_fp16_mfma_peak": round(tfs / FP16_MFMA_PEAK_TFS, 4)}


def lut_leg(torch, q, synthetic, timer):
    """1-bit codes on the 70B MLP-up shape at M = 1 (K 8192, N 28672, G 128,
    per-group z): the table-lookup kernel (qmm_gemv_lut) beside the unpack
    kernel (qmm_gemv), both streaming rotating weight copies from HBM."""
    w = synthetic.BATCHED_70B
    K, N, G = w["K"], w["N"], w["G"]
    c = synthetic.make_case(1, K, N, 1, G, synthetic.seed_for(3, 1), per_group_z=True, s_range=w["s_range"])
    wq = q.pack(torch.from_numpy(c["codes"]).to("cuda:0"), 1)
    bufs = rotating(torch, (wq, torch.from_numpy(c["s"]).to("cuda:0"), torch.from_numpy(c["z"]).to("cuda:0")))
    x = torch.from_numpy(c["X"]).to("cuda:0")
    y = torch.empty((1, N), dtype=torch.float16, device="cuda:0")
    alg = N * K // 8 + 2 * N * (K // G) * 2 + K * 2 + N * 2
    out = {"workload": "70B MLP-up M1 K8192 N28672 k1 G128 per-group z"}
    for name, fn in (("lut", q.gemv_lut), ("unpack", q.gemv)):
        state = {"i": 0}

        def launch(i, fn=fn, state=state):
            b = bufs[state["i"] % len(bufs)]
            state["i"] += 1
            fn(x, b[0], b[1], b[2], 1, G, out=y)

        for _ in range(3):
            launch(0)
        med, _ = timer.median_us(launch, per_region=10, regions=20)
        out[name] = {"us_median": round(med, 2), "algorithmic_GBs": round(alg / med / 1e3, 1),
                     "algorithmic_frac_of_hbm_peak": round(alg / med / 1e3 / HBM_PEAK_GBS, 4),
                     "alu_roofline": alu_roofline("lut_70b_k1" if name == "lut" else "batched_70b_k1_m1", med, K * N)}
    del bufs
    torch.cuda.empty_cache()
    return out


def gemm_leg(torch, q, synthetic, timer, reps):
    """The prefill product (M 2048, K = N = 4096, k 4, G 128) on the MFMA path.
    Cold: every launch reads its own copy of X, Wq and s out of a rotating set
    above 1 GiB (nothing is found in the 256 MB Infinity Cache); hot: the same
    inputs every launch, labelled as such."""
    w = synthetic.PREFILL
    c = synthetic.make_case(w["M"], w["K"], w["N"], 4, w["G"], synthetic.seed_for(4, 4), s_range=w["s_range"])
    X = torch.from_numpy(c["X"]).to("cuda:0")
    wq = q.pack(torch.from_numpy(c["codes"]).to("cuda:0"), 4)
    s = torch.from_numpy(c["s"]).to("cuda:0")
    Y = torch.empty((w["M"], w["N"]), dtype=torch.float16, device="cuda:0")
    bufs = rotating(torch, (X, wq, s))
    state = {"i": 0}

    def cold(i):
        b = bufs[state["i"] % len(bufs)]
        state["i"] += 1
        q.gemm(b[0], b[1], b[2], None, 4, w["G"], out=Y)

    for _ in range(3):
        cold(0)
    flops = 2.0 * w["M"] * w["N"] * w["K"]
    gms = timer.region_ms(cold, reps) / reps
    med, mean = timer.median_us(cold, per_region=5, regions=50)
    hmed, hmean = timer.median_us(lambda i: q.gemm(X, wq, s, None, 4, w["G"], out=Y), per_region=5, regions=20)
    tfs = flops / (gms * 1e-3) / 1e12
    del bufs
    torch.cuda.empty_cache()
    return {"workload": w["name"], "cache": "cold (rotating X, Wq, s copies > 1 GiB)",
            "us_per_launch": round(gms * 1e3, 2), "us_median_of_50": round(med, 2), "TFLOPs": round(tfs, 1),
            "hot_cache": {"us_median": round(hmed, 2), "TFLOPs": round(flops / (hmed * 1e-6) / 1e12, 1)},
            "roofline": {"bound": "mfma", "achieved": round(tfs, 1), "peak": FP16_MFMA_PEAK_TFS, "unit": "TFLOP/s",
                         "frac": round(tfs / FP16_MFMA_PEAK_TFS, 4), "traffic": traffic_for("gemm_k4"),
                         "kernel": "qmm_gemm M=2048 k=4 (gemm_kernel)", "flops_per_launch": flops}}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported here "
              f"(the product shards by output column: one process per GPU, each with its own slice of N).", file=sys.stderr)
        return 2
    import torch
    import bit_weight_quantized_qmm_amd as q
    import synthetic

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2
    torch.cuda.set_device(0)
    timer = Timer(torch)

    if args.copy_probe:
        a = torch.empty(1 << 28, dtype=torch.int32, device="cuda:0").fill_(1)
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"copy_probe_bytes_read": a.numel() * 4, "copies": 3}))
        return 0

    reps = max(10, args.steps // 2)
    if args.only is not None:
        return run_only(args, torch, q, synthetic, timer, reps)

    print(f"bench: setting up decode workload", file=sys.stderr, flush=True)
    decs = [decode_setup(torch, q, synthetic, bits) for bits in synthetic.DECODE_7B["bits"]]
    for _ in range(args.warmup):
        for d in decs:
            decode_launch(q, d)
    torch.cuda.synchronize()

    # the step: the three decode products (k = 3, 4, 6) as one grouped launch
    print(f"bench: timing {args.steps} decode steps", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        grouped_launch(q, decs)
    span = timer.region_ms(lambda i: grouped_launch(q, decs), args.steps)
    ms_per_step = span / args.steps
    wq_step = sum(d["wq_bytes"] for d in decs)
    alg_step = sum(d["alg_bytes"] for d in decs)
    value = wq_step / (ms_per_step * 1e-3) / 1e9
    step_median_us, _ = timer.median_us(lambda i: grouped_launch(q, decs), per_region=10, regions=50)
    # the same products as three separate qmm_gemv launches, for comparison
    sep = timer.region_ms(lambda i: [decode_launch(q, d) for d in decs], args.steps) / args.steps
    separate = {"ms_per_step": round(sep, 5), "packed_GBs": round(wq_step / (sep * 1e-3) / 1e9, 1),
                "packed_frac_of_peak": round(wq_step / (sep * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}

    # each kernel on its own: mean launch duration over the same number of
    # launches, and the median over 50 short regions
    per_bits, mean_ms = {}, {}
    for d in decs:
        ms = timer.region_ms(lambda i, d=d: decode_launch(q, d), args.steps) / args.steps
        med, _ = timer.median_us(lambda i, d=d: decode_launch(q, d), per_region=10, regions=50)
        mean_ms[d["bits"]] = ms
        per_bits[str(d["bits"])] = {
            "us_per_launch": round(ms * 1e3, 3),
            "us_median_of_50": round(med, 3),
            "packed_GBs": round(d["wq_bytes"] / (ms * 1e-3) / 1e9, 1),
            "algorithmic_GBs": round(d["alg_bytes"] / (ms * 1e-3) / 1e9, 1),
            "packed_frac_of_peak": round(d["wq_bytes"] / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        }
    # the step's only kernel is the grouped one: its algorithmic bytes over its
    # mean duration (one launch per step)
    achieved = alg_step / (ms_per_step * 1e-3) / 1e9
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic_for("gemv_grouped_7b"),
                "kernel": "qmm_gemv_grouped k=3,4,6 (gemv_m1_grouped_kernel)",
                "algorithmic_bytes_per_launch": alg_step}
    del decs
    torch.cuda.empty_cache()

    print("bench: measured ceilings (stream read, MFMA) and the library fp16 GEMM", file=sys.stderr, flush=True)
    probes = probes_leg(torch, q, timer)
    probes["library_fp16_gemm"] = blas_context(torch, timer)
    for k, r in per_bits.items():
        name = {"3": "7B_k3_16.9MB", "4": "7B_k4_22.5MB", "6": "7B_k6_33.8MB"}[k]
        r["frac_of_probe_read"] = round(r["packed_GBs"] / probes["read"][name]["GBs"], 4)
    # the step against a plain streaming read of the same packed bytes
    value_frac_of_probe = round(value / probes["read"]["7B_step_73.3MB"]["GBs"], 4)

    print("bench: timing the M=2048 prefill product", file=sys.stderr, flush=True)
    gemm = gemm_leg(torch, q, synthetic, timer, reps)
    mfma_probe = max(v["TFLOPs"] for v in probes["mfma"].values())
    gemm["frac_of_probe_mfma"] = round(gemm["TFLOPs"] / mfma_probe, 4)

    suite = None
    if not args.no_suite:
        print("bench: timing the batched-decode and int8-activation workloads", file=sys.stderr, flush=True)
        suite = run_suite(torch, q, synthetic, timer, reps)

    cpu = None
    if not args.no_cpu:
        print("bench: timing the CPU oracle baseline", file=sys.stderr, flush=True)
        cpu = cpu_baseline(synthetic)

    line = {
        "metric": METRIC, "value": round(value, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f16", "data": "synthetic",
        "config": {"workload": synthetic.DECODE_7B["name"] + " k{3,4,6}", "M": 1, "K": 4096, "N": 11008,
                   "bits": [3, 4, 6], "G": 128, "launches_per_step": 1,
                   "step": "the three products in one qmm_gemv_grouped launch",
                   "weights_read_from": "HBM (rotating copies > 1 GiB)"},
        "value_frac_of_hbm_peak": round(value / HBM_PEAK_GBS, 4),
        "value_frac_of_probe_read": value_frac_of_probe,
        "step_us_median_of_50": round(step_median_us, 3),
        "separate_launches": separate,
        "roofline": roofline,
        "per_bits": per_bits,
        "gemm_m2048": gemm,
        "probes": probes,
        "suite": suite,
        "cpu_baseline": cpu,
        "source_digest": source_digest(),
    }
    print(json.dumps(line), flush=True)
    return 0


def run_suite(torch, q, synthetic, timer, reps):
    return {"batched_decode_70b": batched_suite(torch, q, synthetic, timer, reps),
            "w4a8_8b": w4a8_suite(torch, q, synthetic, timer, reps),
            "w8a8_8b": w4a8_suite(torch, q, synthetic, timer, reps, bits=8),
            "w4a8_prefill": w4a8_prefill_suite(torch, q, synthetic, timer, reps),
            "quantize_7b": quantize_suite(torch, q, synthetic, timer, reps),
            "prefill_fp4_e2m1": gemm_fp_suite(torch, q, synthetic, timer, reps, 0),
            "prefill_fp8_e4m3": gemm_fp_suite(torch, q, synthetic, timer, reps, 1),
            "prefill_fp6_e3m2": gemm_fp_suite(torch, q, synthetic, timer, reps, 2),
            "decode_fp4_e2m1": decode_fp_suite(torch, q, synthetic, timer, reps, 0),
            "decode_fp8_e4m3": decode_fp_suite(torch, q, synthetic, timer, reps, 1),
            "decode_fp6_e3m2": decode_fp_suite(torch, q, synthetic, timer, reps, 2),
            "prefill_fp3_e1m1": gemm_fp_suite(torch, q, synthetic, timer, reps, 4),
            "prefill_fp5_e2m2": gemm_fp_suite(torch, q, synthetic, timer, reps, 5),
            "prefill_fp7_e3m3": gemm_fp_suite(torch, q, synthetic, timer, reps, 6),
            "decode_fp3_e1m1": decode_fp_suite(torch, q, synthetic, timer, reps, 4),
            "decode_fp5_e2m2": decode_fp_suite(torch, q, synthetic, timer, reps, 5),
            "decode_fp7_e3m3": decode_fp_suite(torch, q, synthetic, timer, reps, 6),
            "lut_k1_70b": lut_leg(torch, q, synthetic, timer)}


def run_only(args, torch, q, synthetic, timer, reps):
    """One leg alone (for rocprofv3 runs): few launches, its JSON on stdout."""
    name = args.only
    timer.quick = True
    print(f"bench: --only {name}", file=sys.stderr, flush=True)
    if name == "decode":
        out = {}
        for bits in synthetic.DECODE_7B["bits"]:
            if args.bits is not None and bits != args.bits:
                continue
            d = decode_setup(torch, q, synthetic, bits)
            ms = timer.region_ms(lambda i, d=d: decode_launch(q, d), reps) / reps
            out[f"k{bits}"] = {"us_per_launch": round(ms * 1e3, 3)}
            del d
            torch.cuda.empty_cache()
    elif name == "grouped":
        decs = [decode_setup(torch, q, synthetic, bits) for bits in synthetic.DECODE_7B["bits"]]
        ms = timer.region_ms(lambda i: grouped_launch(q, decs), reps) / reps
        out = {"step_us": round(ms * 1e3, 3)}
    elif name == "lut":
        out = lut_leg(torch, q, synthetic, timer)
    elif name == "gemm":
        out = gemm_leg(torch, q, synthetic, timer, reps)
    elif name == "batched":
        out = batched_suite(torch, q, synthetic, timer, reps, only_bits=args.bits, only_m=args.M)
    elif name in ("w4a8", "w8a8"):
        out = w4a8_suite(torch, q, synthetic, timer, reps, bits=4 if name == "w4a8" else 8)
    elif name == "w4a8p":
        out = w4a8_prefill_suite(torch, q, synthetic, timer, reps)
    elif name == "quantize":
        out = quantize_suite(torch, q, synthetic, timer, reps)
    elif name == "fp":
        out = {f"prefill_{k}": gemm_fp_suite(torch, q, synthetic, timer, reps, k) for k in FP_NAMES}
    elif name == "probes":
        out = probes_leg(torch, q, timer)
        out["library_fp16_gemm"] = blas_context(torch, timer)
    else:
        print(f"unknown leg {name}", file=sys.stderr)
        return 2
    print(json.dumps({"only": name, "result": out}), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
