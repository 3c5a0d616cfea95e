"""CPU oracle for the k-bit weight-quantized matmul -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The GPU product path
(``bit_weight_quantized_qmm_amd``) never imports it and shares no code with it.

The arithmetic lives in ``qmm_oracle.c`` (plain C, fp64 / int64, bit-by-bit
packing; see its header for the passages it follows).  This module only widens
fp16 inputs to float64 exactly (numpy ``astype``) and marshals arrays through
ctypes.

Packed stream layout: uint8 [N][K*bits/8]; column n is a little-endian bit
stream along K with code i at bits [i*bits, i*bits + bits).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(_HERE, "qmm_oracle.c")
LIBRARY = os.path.join(_HERE, "libqmm_oracle.so")
_lock = threading.Lock()


def build(source: str = SOURCE, output: str = LIBRARY, strict: bool = True) -> str:
    """Compile the oracle with gcc (-O2, OpenMP, no fast-math)."""
    cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-Wall"] + (["-Werror"] if strict else []) + [
        "-o", output + ".tmp", source, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(output + ".tmp", output)
    return output


_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_INT = ctypes.c_int


def _ptr(a):
    return None if a is None else a.ctypes.data_as(_P)


class Oracle:
    """ctypes view of one build of the oracle library (the default one, or a test's)."""

    def __init__(self, path: str | None = None):
        path = path or LIBRARY
        if path == LIBRARY:
            with _lock:
                if not os.path.exists(LIBRARY) or os.path.getmtime(LIBRARY) < os.path.getmtime(SOURCE):
                    build()
        self.path = path
        lib = ctypes.CDLL(path)
        for name, args in {
            "qmm_oracle_pack": [_P, _P, _I64, _I64, _INT],
            "qmm_oracle_unpack": [_P, _P, _I64, _I64, _INT],
            "qmm_oracle_dequant": [_P, _P, _P, _I64, _I64, _INT, _I64, _P],
            "qmm_oracle_qmm": [_P, _P, _P, _P, _I64, _I64, _I64, _INT, _I64, _P],
            "qmm_oracle_qmm_sampled": [_P, _P, _P, _P, _I64, _I64, _I64, _INT, _I64, _P, _P, _I64, _P],
            "qmm_oracle_w4a8": [_P, _P, _P, _P, _P, _I64, _I64, _I64, _INT, _I64, _P, _P],
            "qmm_oracle_quantize": [_P, _I64, _I64, _INT, _I64, _P, _P, _P],
            "qmm_oracle_qmm_fp": [_P, _P, _P, _I64, _I64, _I64, _INT, _I64, _P],
        }.items():
            fn = getattr(lib, name)
            fn.argtypes = args
            fn.restype = _INT
        self.lib = lib

    # -- helpers -----------------------------------------------------------
    @staticmethod
    def _f64(a):
        return None if a is None else np.ascontiguousarray(np.asarray(a).astype(np.float64))

    @staticmethod
    def _stream(stream, K, N, bits):
        b = np.ascontiguousarray(stream).view(np.uint8).reshape(-1)
        if b.size != N * K * bits // 8:
            raise ValueError(f"stream holds {b.size} bytes, expected {N * K * bits // 8}")
        return b

    @staticmethod
    def _check(rc, what):
        if rc != 0:
            raise ValueError(f"{what} failed with status {rc}")

    # -- the definition ----------------------------------------------------
    def pack(self, codes, bits: int) -> np.ndarray:
        """uint8 codes [K][N] -> uint8 stream [N][K*bits/8]."""
        codes = np.ascontiguousarray(codes, dtype=np.uint8)
        K, N = codes.shape
        out = np.zeros((N, K * bits // 8), dtype=np.uint8)
        self._check(self.lib.qmm_oracle_pack(_ptr(codes), _ptr(out), K, N, bits), "pack")
        return out

    def pack_signed(self, codes, bits: int) -> np.ndarray:
        """Stream of two's-complement codes [K][N]: stored offset-binary, q + 2^(bits-1)
        (the reading of signed codes this library takes), then packed as unsigned."""
        q = (np.asarray(codes, dtype=np.int64) + (1 << (bits - 1))) & ((1 << bits) - 1)
        return self.pack(q.astype(np.uint8), bits)

    def unpack(self, stream, K: int, N: int, bits: int) -> np.ndarray:
        """stream [N][K*bits/8] -> uint8 codes [K][N]."""
        b = self._stream(stream, K, N, bits)
        out = np.zeros((K, N), dtype=np.uint8)
        self._check(self.lib.qmm_oracle_unpack(_ptr(b), _ptr(out), K, N, bits), "unpack")
        return out

    def dequant(self, stream, s, z, K: int, N: int, bits: int, G: int) -> np.ndarray:
        """float64 W [K][N] = (q - z) * s."""
        b = self._stream(stream, K, N, bits)
        s64, z64 = self._f64(s), self._f64(z)
        out = np.zeros((K, N), dtype=np.float64)
        self._check(self.lib.qmm_oracle_dequant(_ptr(b), _ptr(s64), _ptr(z64), K, N, bits, G, _ptr(out)),
                    "dequant")
        return out

    def qmm(self, X, stream, s, z, bits: int, G: int, N: int | None = None) -> np.ndarray:
        """float64 Y [M][N] = X . dequant(stream); X [M][K] (fp16 or wider)."""
        X64 = self._f64(X)
        M, K = X64.shape
        if N is None:
            N = np.asarray(s).shape[0]
        b = self._stream(stream, K, N, bits)
        s64, z64 = self._f64(s), self._f64(z)
        out = np.zeros((M, N), dtype=np.float64)
        self._check(self.lib.qmm_oracle_qmm(_ptr(X64), _ptr(b), _ptr(s64), _ptr(z64), M, K, N, bits, G,
                                            _ptr(out)), "qmm")
        return out

    def qmm_sampled(self, X, stream, s, z, bits: int, G: int, ms, ns, N: int | None = None) -> np.ndarray:
        """Y[ms[t], ns[t]] for each t, same definition as :meth:`qmm`."""
        X64 = self._f64(X)
        M, K = X64.shape
        if N is None:
            N = np.asarray(s).shape[0]
        b = self._stream(stream, K, N, bits)
        s64, z64 = self._f64(s), self._f64(z)
        ms = np.ascontiguousarray(ms, dtype=np.int64)
        ns = np.ascontiguousarray(ns, dtype=np.int64)
        out = np.zeros(ms.shape[0], dtype=np.float64)
        self._check(self.lib.qmm_oracle_qmm_sampled(_ptr(X64), _ptr(b), _ptr(s64), _ptr(z64), M, K, N, bits, G,
                                                    _ptr(ms), _ptr(ns), ms.shape[0], _ptr(out)), "qmm_sampled")
        return out

    def w4a8(self, Xq, sx, stream, s, z, G: int, bits: int = 4, N: int | None = None):
        """(A int64 [M][K/G][N], Y float64 [M][N]) for int8 activations Xq [M][K]."""
        Xq = np.ascontiguousarray(Xq, dtype=np.int8)
        M, K = Xq.shape
        if N is None:
            N = np.asarray(s).shape[0]
        b = self._stream(stream, K, N, bits)
        sx64, s64, z64 = self._f64(sx), self._f64(s), self._f64(z)
        A = np.zeros((M, K // G, N), dtype=np.int64)
        Y = np.zeros((M, N), dtype=np.float64)
        rc = self.lib.qmm_oracle_w4a8(_ptr(Xq), _ptr(sx64), _ptr(b), _ptr(s64), _ptr(z64), M, K, N, bits, G,
                                      _ptr(A), _ptr(Y))
        self._check(rc, "w4a8")
        return A, Y


    FP_BITS = {0: 4, 1: 8, 2: 6, 3: 6, 4: 3, 5: 5, 6: 7}   # E2M1, E4M3, E3M2, E2M3, E1M1, E2M2, E3M3

    def float_code_value(self, q: int, fmt: int) -> float:
        f = self.lib.qmm_oracle_float_code_value
        f.argtypes = [ctypes.c_uint, _INT]
        f.restype = ctypes.c_double
        return f(q, fmt)

    def qmm_fp(self, X, stream, s, fmt: int, G: int, N: int | None = None) -> np.ndarray:
        """float64 Y = X . (value(q) * s) for floating-point codes (0: E2M1, 1: E4M3, 2: E3M2, 3: E2M3,
        4: E1M1, 5: E2M2, 6: E3M3)."""
        X64 = self._f64(X)
        M, K = X64.shape
        if N is None:
            N = np.asarray(s).shape[0]
        b = self._stream(stream, K, N, self.FP_BITS[fmt])
        Y = np.zeros((M, N), dtype=np.float64)
        self._check(self.lib.qmm_oracle_qmm_fp(_ptr(X64), _ptr(b), _ptr(self._f64(s)), M, K, N, fmt, G, _ptr(Y)),
                    "qmm_fp")
        return Y

    def quantize(self, W, bits: int, G: int):
        """(codes uint8 [K][N], s float16 [N][K/G], z float16 [N][K/G]) for fp16 W [K][N]."""
        W64 = np.ascontiguousarray(np.asarray(W, dtype=np.float16).astype(np.float64))
        K, N = W64.shape
        codes = np.zeros((K, N), dtype=np.uint8)
        s = np.zeros((N, K // G), dtype=np.float64)
        z = np.zeros((N, K // G), dtype=np.float64)
        self._check(self.lib.qmm_oracle_quantize(_ptr(W64), K, N, bits, G, _ptr(codes), _ptr(s), _ptr(z)),
                    "quantize")
        return codes, s.astype(np.float16), z.astype(np.float16)


_default: Oracle | None = None


def default() -> Oracle:
    global _default
    if _default is None:
        _default = Oracle()
    return _default
