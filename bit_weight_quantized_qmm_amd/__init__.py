"""k-bit weight-quantized matmul on AMD MI355X (gfx950): Python binding of libqmm.so.

This module only marshals arguments: it checks tensor dtypes, shapes and
devices, passes raw device pointers and the current HIP stream to the C ABI
(``include/qmm.h``) and raises :class:`QmmError` on a non-zero status.  Every
step of the computation runs in the library's HIP kernels; there is no
fallback.  Importing the package fails loudly if ``libqmm.so`` has not been
built (``python bit_weight_quantized_qmm_amd/_build.py``).

PyTorch is used for device memory and streams only.
"""
from __future__ import annotations

import ctypes
import os

import torch

from ._build import LIBRARY

__all__ = ["QmmError", "packed_bytes", "pack", "pack_signed", "unpack", "gemv", "gemv_grouped", "gemv_lut", "gemm", "gemm_fp", "FP4_E2M1",
           "FP8_E4M3", "FP6_E3M2", "FP6_E2M3", "FP3_E1M1", "FP5_E2M2", "FP7_E3M3", "gemm_w4a8", "gemm_wka8", "quantize",
           "probe_read", "probe_mfma", "library_path", "SYMBOLS"]

SYMBOLS = ("qmm_packed_bytes", "qmm_pack", "qmm_pack_signed", "qmm_unpack", "qmm_gemv", "qmm_gemv_grouped", "qmm_gemv_lut", "qmm_gemm", "qmm_gemm_fp", "qmm_gemm_w4a8", "qmm_gemm_wka8",
           "qmm_quantize", "qmm_status_string", "qmm_last_error", "qmm_last_hip_error", "qmm_probe_read",
           "qmm_probe_mfma")


class QmmError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{message} (status {status})")
        self.status = status


def _load():
    if not os.path.exists(LIBRARY):
        raise ImportError(f"{LIBRARY} is missing: build it first (python bit_weight_quantized_qmm_amd/_build.py)")
    lib = ctypes.CDLL(LIBRARY)
    P, I64, INT = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    sig = {
        "qmm_packed_bytes": ([I64, I64, INT], ctypes.c_size_t),
        "qmm_pack": ([P, P, I64, I64, INT, P], INT),
        "qmm_pack_signed": ([P, P, I64, I64, INT, P], INT),
        "qmm_unpack": ([P, P, I64, I64, INT, P], INT),
        "qmm_gemv": ([P, P, P, P, P, I64, I64, I64, INT, I64, P], INT),
        "qmm_gemm": ([P, P, P, P, P, I64, I64, I64, INT, I64, P], INT),
        "qmm_gemv_lut": ([P, P, P, P, P, I64, I64, I64, INT, I64, P], INT),
        "qmm_gemv_grouped": ([P, INT, I64, I64, P], INT),
        "qmm_gemm_fp": ([P, P, P, P, I64, I64, I64, INT, I64, P], INT),
        "qmm_gemm_w4a8": ([P, P, P, P, P, P, P, I64, I64, I64, I64, P], INT),
        "qmm_gemm_wka8": ([P, P, P, P, P, P, P, I64, I64, I64, INT, I64, P], INT),
        "qmm_quantize": ([P, P, P, P, I64, I64, INT, I64, P], INT),
        "qmm_status_string": ([INT], ctypes.c_char_p),
        "qmm_last_error": ([], ctypes.c_char_p),
        "qmm_last_hip_error": ([], ctypes.c_char_p),
        "qmm_probe_read": ([P, ctypes.c_uint64, P, INT, P], INT),
        "qmm_probe_mfma": ([P, INT, INT, INT, P], INT),
    }
    for name, (args, res) in sig.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = res
    return lib


_lib = _load()


def library_path() -> str:
    return LIBRARY


def _check(status: int):
    if status != 0:
        raise QmmError(status, _lib.qmm_last_error().decode() or _lib.qmm_status_string(status).decode())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _need(t, name, dtype, shape=None, device=None):
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")


def packed_bytes(K: int, N: int, bits: int) -> int:
    return int(_lib.qmm_packed_bytes(K, N, bits))


def pack(codes: torch.Tensor, bits: int, out: torch.Tensor | None = None) -> torch.Tensor:
    """uint8 codes [K, N] -> packed stream as int32 [N, K*bits/32] (bit pattern)."""
    _need(codes, "codes", torch.uint8)
    K, N = codes.shape
    if out is None:
        out = torch.empty((N, K * bits // 32), dtype=torch.int32, device=codes.device)
    _need(out, "out", torch.int32, (N, K * bits // 32), codes.device)
    _check(_lib.qmm_pack(_ptr(codes), _ptr(out), K, N, bits, _stream(codes.device)))
    return out


def pack_signed(codes: torch.Tensor, bits: int, out: torch.Tensor | None = None) -> torch.Tensor:
    """int8 two's-complement codes [K, N] -> packed stream (offset-binary: q + 2^(bits-1))."""
    _need(codes, "codes", torch.int8)
    K, N = codes.shape
    if out is None:
        out = torch.empty((N, K * bits // 32), dtype=torch.int32, device=codes.device)
    _need(out, "out", torch.int32, (N, K * bits // 32), codes.device)
    _check(_lib.qmm_pack_signed(_ptr(codes), _ptr(out), K, N, bits, _stream(codes.device)))
    return out


def unpack(wq: torch.Tensor, K: int, N: int, bits: int, out: torch.Tensor | None = None) -> torch.Tensor:
    """Packed stream [N, K*bits/32] -> uint8 codes [K, N] through the kernels' register unpack."""
    _need(wq, "wq", torch.int32, (N, K * bits // 32))
    if out is None:
        out = torch.empty((K, N), dtype=torch.uint8, device=wq.device)
    _need(out, "out", torch.uint8, (K, N), wq.device)
    _check(_lib.qmm_unpack(_ptr(wq), _ptr(out), K, N, bits, _stream(wq.device)))
    return out


def _product(fn, X, wq, s, z, bits, G, out):
    _need(X, "X", torch.float16)
    M, K = X.shape
    N = s.shape[0] if s.dim() == 2 else -1
    _need(wq, "wq", torch.int32, (N, K * bits // 32), X.device)
    _need(s, "s", torch.float16, (N, K // G), X.device)
    if z is not None:
        _need(z, "z", torch.float16, (N, K // G), X.device)
    if out is None:
        out = torch.empty((M, N), dtype=torch.float16, device=X.device)
    _need(out, "out", torch.float16, (M, N), X.device)
    _check(fn(_ptr(X), _ptr(wq), _ptr(s), _ptr(z), _ptr(out), M, K, N, bits, G, _stream(X.device)))
    return out


def gemv(X, wq, s, z, bits: int, G: int, out=None) -> torch.Tensor:
    """Y [M, N] fp16 = X [M, K] fp16 . dequant(wq); 1 <= M <= 16."""
    return _product(_lib.qmm_gemv, X, wq, s, z, bits, G, out)


class _Problem(ctypes.Structure):
    _fields_ = [("X", ctypes.c_void_p), ("wq", ctypes.c_void_p), ("s", ctypes.c_void_p), ("z", ctypes.c_void_p),
                ("Y", ctypes.c_void_p), ("N", ctypes.c_int64), ("bits", ctypes.c_int)]


def gemv_grouped(problems, G: int, outs=None):
    """Several M = 1 products in one launch.  problems: sequence of (X [1, K], wq, s, z or None,
    bits) sharing K; returns the list of Y [1, N] (or fills outs)."""
    problems = list(problems)
    if not problems:
        raise ValueError("no problems")
    K = problems[0][0].shape[1]
    arr = (_Problem * len(problems))()
    res = []
    for i, (X, wq, s, z, bits) in enumerate(problems):
        _need(X, "X", torch.float16, (1, K))
        N = s.shape[0]
        _need(wq, "wq", torch.int32, (N, K * bits // 32), X.device)
        _need(s, "s", torch.float16, (N, K // G), X.device)
        if z is not None:
            _need(z, "z", torch.float16, (N, K // G), X.device)
        Y = outs[i] if outs is not None else torch.empty((1, N), dtype=torch.float16, device=X.device)
        _need(Y, "out", torch.float16, (1, N), X.device)
        arr[i] = _Problem(X.data_ptr(), wq.data_ptr(), s.data_ptr(), 0 if z is None else z.data_ptr(), Y.data_ptr(),
                          N, bits)
        res.append(Y)
    _check(_lib.qmm_gemv_grouped(ctypes.cast(arr, ctypes.c_void_p), len(problems), K, G,
                                 _stream(problems[0][0].device)))
    return res


def gemv_lut(X, wq, s, z, bits: int, G: int, out=None) -> torch.Tensor:
    """Y [1, N] fp16 = X [1, K] fp16 . dequant(wq) for 1-bit codes by table lookup (K <= 8192)."""
    return _product(_lib.qmm_gemv_lut, X, wq, s, z, bits, G, out)


def gemm(X, wq, s, z, bits: int, G: int, out=None) -> torch.Tensor:
    """Y [M, N] fp16 = X [M, K] fp16 . dequant(wq); any M (f16 MFMA path)."""
    return _product(_lib.qmm_gemm, X, wq, s, z, bits, G, out)


FP4_E2M1, FP8_E4M3, FP6_E3M2, FP6_E2M3, FP3_E1M1, FP5_E2M2, FP7_E3M3 = 0, 1, 2, 3, 4, 5, 6
_FP_BITS = {FP4_E2M1: 4, FP8_E4M3: 8, FP6_E3M2: 6, FP6_E2M3: 6, FP3_E1M1: 3, FP5_E2M2: 5, FP7_E3M3: 7}


def gemm_fp(X, wq, s, fmt: int, G: int, out=None) -> torch.Tensor:
    """Y [M, N] fp16 = X . (value(q) s) for floating-point codes (FP4_E2M1, FP8_E4M3,
    FP6_E3M2, FP6_E2M3, FP3_E1M1, FP5_E2M2 or FP7_E3M3)."""
    if fmt not in _FP_BITS:
        raise ValueError(f"unknown float code format {fmt}: expected one of {sorted(_FP_BITS)}")
    _need(X, "X", torch.float16)
    M, K = X.shape
    N = s.shape[0]
    _need(wq, "wq", torch.int32, (N, K * _FP_BITS[fmt] // 32), X.device)
    _need(s, "s", torch.float16, (N, K // G), X.device)
    if out is None:
        out = torch.empty((M, N), dtype=torch.float16, device=X.device)
    _need(out, "out", torch.float16, (M, N), X.device)
    _check(_lib.qmm_gemm_fp(_ptr(X), _ptr(wq), _ptr(s), _ptr(out), M, K, N, fmt, G, _stream(X.device)))
    return out


def gemm_w4a8(Xq, sx, wq, s, z, G: int, out=None, acc_out=None) -> torch.Tensor:
    """Y [M, N] fp16 for int8 activations Xq [M, K] with per-token fp16 scales sx [M] and
    4-bit weights; acc_out (int32 [M, K/G, N]) optionally receives the exact group sums."""
    return _int8_product(False, Xq, sx, wq, s, z, 4, G, out, acc_out)


def gemm_wka8(Xq, sx, wq, s, z, bits: int, G: int, out=None, acc_out=None) -> torch.Tensor:
    """As gemm_w4a8 for bits-bit weights, bits in 1..8 (8: W8A8)."""
    return _int8_product(True, Xq, sx, wq, s, z, bits, G, out, acc_out)


def _int8_product(any_bits: bool, Xq, sx, wq, s, z, bits: int, G: int, out, acc_out) -> torch.Tensor:
    _need(Xq, "Xq", torch.int8)
    M, K = Xq.shape
    N = s.shape[0]
    _need(sx, "sx", torch.float16, (M,), Xq.device)
    _need(wq, "wq", torch.int32, (N, K * bits // 32), Xq.device)
    _need(s, "s", torch.float16, (N, K // G), Xq.device)
    if z is not None:
        _need(z, "z", torch.float16, (N, K // G), Xq.device)
    if acc_out is not None:
        _need(acc_out, "acc_out", torch.int32, (M, K // G, N), Xq.device)
    if out is None:
        out = torch.empty((M, N), dtype=torch.float16, device=Xq.device)
    _need(out, "out", torch.float16, (M, N), Xq.device)
    ptrs = (_ptr(Xq), _ptr(sx), _ptr(wq), _ptr(s), _ptr(z), _ptr(out), _ptr(acc_out))
    if any_bits:
        _check(_lib.qmm_gemm_wka8(*ptrs, M, K, N, bits, G, _stream(Xq.device)))
    else:
        _check(_lib.qmm_gemm_w4a8(*ptrs, M, K, N, G, _stream(Xq.device)))
    return out


def quantize(W, bits: int, G: int, codes=None, s=None, z=None):
    """(codes uint8 [K, N], s fp16 [N, K/G], z fp16 [N, K/G]) for fp16 weights W [K, N]."""
    _need(W, "W", torch.float16)
    K, N = W.shape
    if codes is None:
        codes = torch.empty((K, N), dtype=torch.uint8, device=W.device)
    if s is None:
        s = torch.empty((N, K // G), dtype=torch.float16, device=W.device)
    if z is None:
        z = torch.empty((N, K // G), dtype=torch.float16, device=W.device)
    _need(codes, "codes", torch.uint8, (K, N), W.device)
    _need(s, "s", torch.float16, (N, K // G), W.device)
    _need(z, "z", torch.float16, (N, K // G), W.device)
    _check(_lib.qmm_quantize(_ptr(W), _ptr(codes), _ptr(s), _ptr(z), K, N, bits, G, _stream(W.device)))
    return codes, s, z


def probe_read(buf: torch.Tensor, grid: int, sink: torch.Tensor | None = None) -> None:
    """Measurement hook: one streaming read of the whole of buf (any dtype, contiguous,
    byte size a multiple of 16) by `grid` workgroups; computes nothing of the product."""
    if not buf.is_cuda or not buf.is_contiguous():
        raise ValueError("buf must be a contiguous GPU tensor")
    if sink is None:
        sink = torch.empty(grid * 256, dtype=torch.int32, device=buf.device)
    _need(sink, "sink", torch.int32, None, buf.device)
    if sink.numel() < grid * 256:
        raise ValueError("sink needs grid * 256 elements")
    _check(_lib.qmm_probe_read(_ptr(buf), buf.numel() * buf.element_size(), _ptr(sink), grid, _stream(buf.device)))


def probe_mfma(iters: int, grid: int, shape: int = 0, sink: torch.Tensor | None = None,
               device: str = "cuda:0") -> int:
    """Measurement hook: back-to-back f16 MFMAs (shape 0: 16x16x32, 1: 32x32x16) on register
    operands in `grid` workgroups of 8 waves; returns the flops enqueued."""
    if sink is None:
        sink = torch.empty(grid * 512, dtype=torch.float32, device=device)
    _need(sink, "sink", torch.float32)
    if sink.numel() < grid * 512:
        raise ValueError("sink needs grid * 512 elements")
    _check(_lib.qmm_probe_mfma(_ptr(sink), iters, grid, shape, _stream(sink.device)))
    return grid * 8 * iters * 8 * 16384
