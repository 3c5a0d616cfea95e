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


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU-oracle baseline leg")
    ap.add_argument("--no-suite", action="store_true", help="skip the suite (batched decode, int8 activations, quantiser, float codes)")
    ap.add_argument("--copy-probe", action="store_true", help="run a plain 1 GiB device copy (counter calibration)")
    return ap.parse_args()


# Sources each profiled kernel is built from: a counter run stays valid for a
# kernel only while these files are unchanged.
KERNEL_SOURCES = {
    "gemv_m1": ("gemv.hip", "qmm_device.hpp", "unpack_plan.inc", "launch.hpp"),
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


def cpu_baseline(synthetic, budget_s=12.0):
    """The oracle as it stands, timed on this host: the same decode step
    (k = 3, 4, 6) repeated until about budget_s seconds have passed."""
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
    return {"value": round(done_bytes / dt / 1e9, 4), "unit": "GB/s", "cores": cores, "kind": "oracle",
            "sample": f"{reps} x the full decode step (k=3,4,6; M=1 K=4096 N=11008): bit-serial unpack, "
                      f"fp64 dequant and fp64 dot products, {dt:.1f} s wall"}


def rotating(torch, tensors):
    """Enough copies of the weight-side tensors that the copies together exceed
    1 GiB, so consecutive launches never find their weights in a cache."""
    per = sum(t.numel() * t.element_size() for t in tensors)
    copies = max(2, -(-ROTATE_BYTES // per))
    return [tuple(t.clone() for t in tensors) for _ in range(copies)]


def batched_suite(torch, q, synthetic, timer, reps):
    """70B MLP-up batched decode (K 8192, N 28672, G 128, per-group z) at M = 1, 8, 16
    for k = 1, 2, 5, 7, 8: us per launch and HBM GB/s of the algorithmic bytes."""
    w = synthetic.BATCHED_70B
    K, N, G = w["K"], w["N"], w["G"]
    out = {}
    for bits in w["bits"]:
        c = synthetic.make_case(max(w["Ms"]), K, N, bits, G, synthetic.seed_for(3, bits), per_group_z=True,
                                s_range=w["s_range"])
        wq = q.pack(torch.from_numpy(c["codes"]).to("cuda:0"), bits)
        bufs = rotating(torch, (wq, torch.from_numpy(c["s"]).to("cuda:0"), torch.from_numpy(c["z"]).to("cuda:0")))
        del wq, c["codes"]
        X = torch.from_numpy(c["X"]).to("cuda:0")
        row = {}
        for M in w["Ms"]:
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


FP_NAMES = {0: "E2M1", 1: "E4M3", 2: "E3M2", 3: "E2M3"}


def gemm_fp_suite(torch, q, synthetic, timer, reps, fmt):
    """qmm_gemm_fp on the prefill shape (M 2048, K = N = 4096, G 128) with E2M1
    (fmt 0), E4M3 (fmt 1) or E3M2 (fmt 2) codes: TFLOP/s against the dense fp16 MFMA peak."""
    w = synthetic.PREFILL
    M, K, N, G = w["M"], w["K"], w["N"], w["G"]
    bits = {0: 4, 1: 8, 2: 6, 3: 6}[fmt]
    g = synthetic.rng(synthetic.seed_for(4, bits, 11 + fmt))
    codes = g.integers(0, 1 << bits, (K, N))
    if fmt == 1:
        codes[(codes & 0x7F) == 0x7F] = 0x30
    wq = q.pack(torch.from_numpy(codes.astype(np.uint8)).to("cuda:0"), bits)
    s = torch.from_numpy(synthetic.fp16_uniform(g, 0.002, 0.02, (N, K // G))).to("cuda:0")
    X = torch.from_numpy(synthetic.fp16_normal(g, (M, K))).to("cuda:0")
    Y = torch.empty((M, N), dtype=torch.float16, device="cuda:0")
    for _ in range(3):
        q.gemm_fp(X, wq, s, fmt, G, out=Y)
    ms = timer.region_ms(lambda i: q.gemm_fp(X, wq, s, fmt, G, out=Y), reps) / reps
    tfs = 2.0 * M * N * K / (ms * 1e-3) / 1e12
    return {"workload": f"prefill-gemm {FP_NAMES[fmt]} codes M{M} K{K} N{N} G{G}",
            "us": round(ms * 1e3, 2), "TFLOPs": round(tfs, 1), "frac_of_fp16_mfma_peak": round(tfs / FP16_MFMA_PEAK_TFS, 4)}


def decode_fp_suite(torch, q, synthetic, timer, reps, fmt):
    """qmm_gemm_fp at M = 1, 8, 16 on the 7B MLP shape (K 4096, N 11008, G 128)
    with E2M1 (fmt 0), E4M3 (fmt 1) or E3M2 (fmt 2) codes: weights streamed from HBM
    (rotating copies); HBM GB/s of the algorithmic bytes."""
    w = synthetic.DECODE_7B
    K, N, G = w["K"], w["N"], w["G"]
    bits = {0: 4, 1: 8, 2: 6, 3: 6}[fmt]
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
    print(f"bench: setting up decode workload", file=sys.stderr, flush=True)

    if args.copy_probe:
        a = torch.empty(1 << 28, dtype=torch.int32, device="cuda:0").fill_(1)
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"copy_probe_bytes_read": a.numel() * 4, "copies": 3}))
        return 0

    decs = [decode_setup(torch, q, synthetic, bits) for bits in synthetic.DECODE_7B["bits"]]
    timer = Timer(torch)
    for _ in range(args.warmup):
        for d in decs:
            decode_launch(q, d)
    torch.cuda.synchronize()

    # the step: three decode products (k = 3, 4, 6), back to back
    print(f"bench: timing {args.steps} decode steps", file=sys.stderr, flush=True)
    span = timer.region_ms(lambda i: [decode_launch(q, d) for d in decs], args.steps)
    ms_per_step = span / args.steps
    wq_step = sum(d["wq_bytes"] for d in decs)
    value = wq_step / (ms_per_step * 1e-3) / 1e9

    # each kernel on its own: mean launch duration over the same number of launches
    per_bits, mean_ms = {}, {}
    for d in decs:
        ms = timer.region_ms(lambda i, d=d: decode_launch(q, d), args.steps) / args.steps
        mean_ms[d["bits"]] = ms
        per_bits[str(d["bits"])] = {
            "us_per_launch": round(ms * 1e3, 3),
            "packed_GBs": round(d["wq_bytes"] / (ms * 1e-3) / 1e9, 1),
            "algorithmic_GBs": round(d["alg_bytes"] / (ms * 1e-3) / 1e9, 1),
            "packed_frac_of_peak": round(d["wq_bytes"] / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        }
    dom = max(decs, key=lambda d: mean_ms[d["bits"]])
    dom_ms = mean_ms[dom["bits"]]
    achieved = dom["alg_bytes"] / (dom_ms * 1e-3) / 1e9
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic_for(f"gemv_m1_k{dom['bits']}"),
                "kernel": f"qmm_gemv M=1 k={dom['bits']} (gemv_m1_kernel)",
                "algorithmic_bytes_per_launch": dom["alg_bytes"]}
    del decs
    torch.cuda.empty_cache()

    # prefill product on the MFMA path
    print("bench: timing the M=2048 prefill product", file=sys.stderr, flush=True)
    w = synthetic.PREFILL
    c = synthetic.make_case(w["M"], w["K"], w["N"], 4, w["G"], synthetic.seed_for(4, 4), s_range=w["s_range"])
    X = torch.from_numpy(c["X"]).to("cuda:0")
    wq = q.pack(torch.from_numpy(c["codes"]).to("cuda:0"), 4)
    s = torch.from_numpy(c["s"]).to("cuda:0")
    Y = torch.empty((w["M"], w["N"]), dtype=torch.float16, device="cuda:0")
    for _ in range(3):
        q.gemm(X, wq, s, None, 4, w["G"], out=Y)
    nrep = max(10, args.steps // 2)
    gms = timer.region_ms(lambda i: q.gemm(X, wq, s, None, 4, w["G"], out=Y), nrep) / nrep
    flops = 2.0 * w["M"] * w["N"] * w["K"]
    tfs = flops / (gms * 1e-3) / 1e12
    gemm = {"workload": w["name"], "us_per_launch": round(gms * 1e3, 2), "TFLOPs": round(tfs, 1),
            "roofline": {"bound": "mfma", "achieved": round(tfs, 1), "peak": FP16_MFMA_PEAK_TFS, "unit": "TFLOP/s",
                         "frac": round(tfs / FP16_MFMA_PEAK_TFS, 4), "traffic": traffic_for("gemm_k4")}}

    suite = None
    if not args.no_suite:
        print("bench: timing the batched-decode and int8-activation workloads", file=sys.stderr, flush=True)
        reps = max(10, args.steps // 2)
        suite = {"batched_decode_70b": batched_suite(torch, q, synthetic, timer, reps),
                 "w4a8_8b": w4a8_suite(torch, q, synthetic, timer, reps),
                 "w8a8_8b": w4a8_suite(torch, q, synthetic, timer, reps, bits=8),
                 "quantize_7b": quantize_suite(torch, q, synthetic, timer, reps),
                 "prefill_fp4_e2m1": gemm_fp_suite(torch, q, synthetic, timer, reps, 0),
                 "prefill_fp8_e4m3": gemm_fp_suite(torch, q, synthetic, timer, reps, 1),
                 "decode_fp4_e2m1": decode_fp_suite(torch, q, synthetic, timer, reps, 0),
                 "decode_fp8_e4m3": decode_fp_suite(torch, q, synthetic, timer, reps, 1),
                 "prefill_fp6_e3m2": gemm_fp_suite(torch, q, synthetic, timer, reps, 2),
                 "decode_fp6_e3m2": decode_fp_suite(torch, q, synthetic, timer, reps, 2)}

    cpu = None
    if not args.no_cpu:
        print("bench: timing the CPU oracle baseline", file=sys.stderr, flush=True)
        cpu = cpu_baseline(synthetic)

    line = {
        "metric": METRIC, "value": round(value, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f16", "data": "synthetic",
        "config": {"workload": synthetic.DECODE_7B["name"] + " k{3,4,6}", "M": 1, "K": 4096, "N": 11008,
                   "bits": [3, 4, 6], "G": 128, "launches_per_step": 3,
                   "weights_read_from": "HBM (rotating copies > 1 GiB)"},
        "value_frac_of_hbm_peak": round(value / HBM_PEAK_GBS, 4),
        "roofline": roofline,
        "per_bits": per_bits,
        "gemm_m2048": gemm,
        "suite": suite,
        "cpu_baseline": cpu,
        "source_digest": source_digest(),
    }
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
