"""Seeded synthetic inputs for the k-bit weight-quantized matmul.

This module only draws random numbers; it holds none of the method's arithmetic
(no packing, no dequantisation, no products), so the CPU oracle and the GPU path
can both start from the same inputs without sharing any code.

Recipe (every draw from numpy's PCG64 with an explicit seed):
  * activations X: fp32 standard normal, rounded to fp16 (round to nearest even);
  * codes q: discrete uniform over [0, 2^k - 1], uint8, layout [K][N];
  * scales s: fp32 uniform over [lo, hi], rounded to fp16, layout [N][K/G];
  * zero-points z (when drawn per group): discrete uniform integers over
    [0, 2^k - 1], stored as fp16 (exact), layout [N][K/G]; otherwise None,
    which means the mid-range code 2^(k-1);
  * int8 activations Xq: discrete uniform over [-127, 127]; per-token scales
    sx: fp32 uniform over [lo, hi] rounded to fp16, layout [M].

The named workloads are LLM-shaped stand-ins (7B-class MLP, 70B-class MLP-up,
8B-class MLP, a 2048-token prefill) for the pages' model workloads, which are
not available here.
"""
from __future__ import annotations

import numpy as np

SEED_BASE = 20261202


def rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def fp16_normal(g: np.random.Generator, shape) -> np.ndarray:
    return g.standard_normal(shape, dtype=np.float32).astype(np.float16)


def fp16_uniform(g: np.random.Generator, lo: float, hi: float, shape) -> np.ndarray:
    return g.uniform(lo, hi, size=shape).astype(np.float32).astype(np.float16)


def codes_uniform(g: np.random.Generator, bits: int, K: int, N: int) -> np.ndarray:
    return g.integers(0, 1 << bits, size=(K, N), dtype=np.uint8)


def zeros_uniform(g: np.random.Generator, bits: int, N: int, ngroups: int) -> np.ndarray:
    return g.integers(0, 1 << bits, size=(N, ngroups)).astype(np.float16)


def make_case(M: int, K: int, N: int, bits: int, G: int, seed: int,
              per_group_z: bool = False, s_range=(0.002, 0.02)) -> dict:
    """fp16-activation case: X [M][K], codes [K][N], s [N][K/G], z [N][K/G] or None."""
    g = rng(seed)
    X = fp16_normal(g, (M, K))
    codes = codes_uniform(g, bits, K, N)
    s = fp16_uniform(g, s_range[0], s_range[1], (N, K // G))
    z = zeros_uniform(g, bits, N, K // G) if per_group_z else None
    return dict(M=M, K=K, N=N, bits=bits, G=G, X=X, codes=codes, s=s, z=z)


def make_w4a8_case(M: int, K: int, N: int, G: int, seed: int, bits: int = 4,
                   per_group_z: bool = False, sx_range=(0.01, 0.05), s_range=(0.002, 0.02)) -> dict:
    """int8-activation case: Xq [M][K], sx [M], codes [K][N], s [N][K/G], z or None."""
    g = rng(seed)
    Xq = g.integers(-127, 128, size=(M, K), dtype=np.int8)
    sx = fp16_uniform(g, sx_range[0], sx_range[1], (M,))
    codes = codes_uniform(g, bits, K, N)
    s = fp16_uniform(g, s_range[0], s_range[1], (N, K // G))
    z = zeros_uniform(g, bits, N, K // G) if per_group_z else None
    return dict(M=M, K=K, N=N, bits=bits, G=G, Xq=Xq, sx=sx, codes=codes, s=s, z=z)


def seed_for(config_index: int, bits: int, extra: int = 0) -> int:
    return SEED_BASE + 100 * config_index + bits + 1000 * extra


# Named workloads (shapes and distributions of the pages' LLM workloads).
TINY = dict(name="tiny M1 K256 N256 k4 G64", M=1, K=256, N=256, bits=(4,), G=64, s_range=(0.005, 0.02),
            per_group_z=False)
DECODE_7B = dict(name="decode-gemv 7B-MLP M1 K4096 N11008 G128", M=1, K=4096, N=11008, bits=(3, 4, 6), G=128,
                 s_range=(0.002, 0.02), per_group_z=False)
BATCHED_70B = dict(name="batched-decode 70B-MLP-up M{1,8,16} K8192 N28672 G128 per-group z", Ms=(1, 8, 16),
                   K=8192, N=28672, bits=(1, 2, 5, 7, 8), G=128, s_range=(0.002, 0.02), per_group_z=True)
PREFILL = dict(name="prefill-gemm M2048 K4096 N4096 k4 G128", M=2048, K=4096, N=4096, bits=(4,), G=128,
               s_range=(0.002, 0.02), per_group_z=False)
W4A8_8B = dict(name="w4a8 8B-MLP M16 K4096 N14336 k4 G128", M=16, K=4096, N=14336, bits=(4,), G=128,
               s_range=(0.002, 0.02), per_group_z=False)
