"""The C-ABI library without a GPU: it loads, exports what include/qmm.h declares,
and rejects invalid arguments before any HIP call (so these run on the CPU)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "qmm.h")
LIB = os.path.join(ROOT, "bit_weight_quantized_qmm_amd", "libqmm.so")

OK, INVALID, UNSUPPORTED, HIPERR = 0, -1, -2, -3
FAKE = ctypes.c_void_p(0x1000)   # never dereferenced: validation fails first


def declared_symbols():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"\b(qmm_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):
        # by path: importing the package needs the library this builds
        import importlib.util
        spec = importlib.util.spec_from_file_location(
            "qmm_build", os.path.join(ROOT, "bit_weight_quantized_qmm_amd", "_build.py"))
        b = importlib.util.module_from_spec(spec)
        spec.loader.exec_module(b)
        b.build()
    lib = ctypes.CDLL(LIB)
    P, I64, INT = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    lib.qmm_packed_bytes.argtypes = [I64, I64, INT]
    lib.qmm_packed_bytes.restype = ctypes.c_size_t
    for f in ("qmm_pack", "qmm_pack_signed", "qmm_unpack"):
        getattr(lib, f).argtypes = [P, P, I64, I64, INT, P]
        getattr(lib, f).restype = INT
    for f in ("qmm_gemv", "qmm_gemm", "qmm_gemv_lut"):
        getattr(lib, f).argtypes = [P, P, P, P, P, I64, I64, I64, INT, I64, P]
        getattr(lib, f).restype = INT
    lib.qmm_gemm_w4a8.argtypes = [P, P, P, P, P, P, P, I64, I64, I64, I64, P]
    lib.qmm_gemm_w4a8.restype = INT
    lib.qmm_gemm_wka8.argtypes = [P, P, P, P, P, P, P, I64, I64, I64, INT, I64, P]
    lib.qmm_gemm_wka8.restype = INT
    lib.qmm_gemm_fp.argtypes = [P, P, P, P, I64, I64, I64, INT, I64, P]
    lib.qmm_gemm_fp.restype = INT
    lib.qmm_quantize.argtypes = [P, P, P, P, I64, I64, INT, I64, P]
    lib.qmm_quantize.restype = INT
    lib.qmm_status_string.argtypes = [INT]
    lib.qmm_status_string.restype = ctypes.c_char_p
    lib.qmm_last_error.restype = ctypes.c_char_p
    lib.qmm_last_hip_error.restype = ctypes.c_char_p
    lib.qmm_probe_read.argtypes = [P, ctypes.c_uint64, P, INT, P]
    lib.qmm_probe_read.restype = INT
    lib.qmm_probe_mfma.argtypes = [P, INT, INT, INT, P]
    lib.qmm_probe_mfma.restype = INT
    return lib


def test_header_declares_the_boundary():
    syms = declared_symbols()
    for name in ("qmm_pack", "qmm_unpack", "qmm_packed_bytes", "qmm_gemv", "qmm_gemm", "qmm_gemm_w4a8",
                 "qmm_gemm_wka8", "qmm_quantize", "qmm_status_string", "qmm_last_error", "qmm_last_hip_error"):
        assert name in syms


def test_every_declared_symbol_is_exported(lib):
    for name in declared_symbols():
        assert hasattr(lib, name), name


def test_binding_lists_every_symbol():
    import bit_weight_quantized_qmm_amd as q
    assert sorted(q.SYMBOLS) == declared_symbols()


def test_packed_bytes(lib):
    assert lib.qmm_packed_bytes(4096, 11008, 4) == 4096 * 11008 // 2
    assert lib.qmm_packed_bytes(8192, 28672, 3) == 8192 * 28672 * 3 // 8
    assert lib.qmm_packed_bytes(32, 1, 1) == 4
    assert lib.qmm_packed_bytes(32, 1, 9) == 0
    assert lib.qmm_packed_bytes(-32, 1, 4) == 0


@pytest.mark.parametrize("K,N,bits,expect", [
    (32, 4, 0, INVALID), (32, 4, 9, INVALID), (48, 4, 4, INVALID), (0, 4, 4, INVALID), (32, 0, 4, INVALID),
    (1 << 22, 4, 4, UNSUPPORTED),
])
def test_pack_validation(lib, K, N, bits, expect):
    assert lib.qmm_pack(FAKE, FAKE, K, N, bits, None) == expect
    assert lib.qmm_unpack(FAKE, FAKE, K, N, bits, None) == expect
    assert lib.qmm_last_error()


def test_pack_null_pointers(lib):
    assert lib.qmm_pack(None, FAKE, 32, 4, 4, None) == INVALID
    assert lib.qmm_unpack(FAKE, None, 32, 4, 4, None) == INVALID


@pytest.mark.parametrize("M,K,N,bits,G,expect", [
    (1, 4096, 8, 0, 128, INVALID),
    (1, 4096, 8, 9, 128, INVALID),
    (1, 4016, 8, 4, 16 * 2, INVALID),   # K % 32
    (1, 4096, 8, 4, 48, INVALID),       # G % 32
    (1, 4096, 8, 4, 16, INVALID),       # G < 32
    (1, 4096, 8, 4, 384, INVALID),      # K % G
    (0, 4096, 8, 4, 128, INVALID),
    (1, 4096, 0, 4, 128, INVALID),
    (1, 1 << 22, 8, 4, 128, UNSUPPORTED),
])
def test_product_validation(lib, M, K, N, bits, G, expect):
    for fn in (lib.qmm_gemv, lib.qmm_gemm):
        assert fn(FAKE, FAKE, FAKE, None, FAKE, M, K, N, bits, G, None) == expect


def test_gemv_rejects_large_m(lib):
    assert lib.qmm_gemv(FAKE, FAKE, FAKE, None, FAKE, 17, 4096, 8, 4, 128, None) == INVALID


def test_product_null_pointers(lib):
    for fn in (lib.qmm_gemv, lib.qmm_gemm):
        assert fn(None, FAKE, FAKE, None, FAKE, 1, 256, 8, 4, 64, None) == INVALID
        assert fn(FAKE, None, FAKE, None, FAKE, 1, 256, 8, 4, 64, None) == INVALID
        assert fn(FAKE, FAKE, None, None, FAKE, 1, 256, 8, 4, 64, None) == INVALID
        assert fn(FAKE, FAKE, FAKE, None, None, 1, 256, 8, 4, 64, None) == INVALID


def test_w4a8_validation(lib):
    f = lib.qmm_gemm_w4a8
    assert f(None, FAKE, FAKE, FAKE, None, FAKE, None, 16, 4096, 64, 128, None) == INVALID
    assert f(FAKE, None, FAKE, FAKE, None, FAKE, None, 16, 4096, 64, 128, None) == INVALID
    assert f(FAKE, FAKE, FAKE, FAKE, None, FAKE, None, 16, 4096, 64, 100, None) == INVALID
    assert f(FAKE, FAKE, FAKE, FAKE, None, FAKE, None, 16, 4096, 64, 64, None) == UNSUPPORTED
    assert f(FAKE, FAKE, FAKE, FAKE, None, FAKE, None, 16, 4096, 64, 384, None) in (INVALID, UNSUPPORTED)
    assert f(FAKE, FAKE, FAKE, FAKE, None, FAKE, None, 0, 4096, 64, 128, None) == INVALID


def test_wka8_validation(lib):
    """Host-side checks only (every call returns before any HIP call)."""
    f = lib.qmm_gemm_wka8
    for bits in (0, 9, -1):
        assert f(FAKE, FAKE, FAKE, FAKE, None, FAKE, None, 16, 4096, 64, bits, 128, None) == INVALID
    assert f(None, FAKE, FAKE, FAKE, None, FAKE, None, 16, 4096, 64, 8, 128, None) == INVALID
    assert f(FAKE, FAKE, None, FAKE, None, FAKE, None, 16, 4096, 64, 8, 128, None) == INVALID
    assert f(FAKE, FAKE, FAKE, FAKE, None, FAKE, None, 16, 4096, 64, 8, 64, None) == UNSUPPORTED
    assert f(FAKE, FAKE, FAKE, FAKE, None, FAKE, None, 16, 4096, 64, 3, 2048, None) == UNSUPPORTED
    assert f(FAKE, FAKE, FAKE, FAKE, None, FAKE, None, 16, 4000, 64, 8, 128, None) == INVALID


def test_pack_signed_validation(lib):
    f = lib.qmm_pack_signed
    assert f(None, FAKE, 256, 8, 4, None) == INVALID
    assert f(FAKE, None, 256, 8, 4, None) == INVALID
    assert f(FAKE, FAKE, 256, 8, 0, None) == INVALID
    assert f(FAKE, FAKE, 250, 8, 4, None) == INVALID


def test_binding_rejects_unknown_float_format():
    """The binding names an unknown code format before looking at any tensor."""
    import torch
    import bit_weight_quantized_qmm_amd as q
    X = torch.zeros((1, 64), dtype=torch.float16)
    for fmt in (-1, 7):
        with pytest.raises(ValueError, match="unknown float code format"):
            q.gemm_fp(X, X, X, fmt, 32)
    assert (q.FP4_E2M1, q.FP8_E4M3, q.FP6_E3M2, q.FP6_E2M3) == (0, 1, 2, 3)
    assert (q.FP3_E1M1, q.FP5_E2M2, q.FP7_E3M3) == (4, 5, 6)


def test_gemm_fp_validation(lib):
    f = lib.qmm_gemm_fp
    for fmt in (-1, 7, 8):
        assert f(FAKE, FAKE, FAKE, FAKE, 4, 256, 8, fmt, 64, None) == INVALID
    for fmt in (4, 5, 6):   # 3-, 5-, 7-bit formats: the same shape checks
        assert f(FAKE, FAKE, FAKE, FAKE, 4, 256, 8, fmt, 48, None) == INVALID
        assert f(FAKE, FAKE, FAKE, FAKE, 4, 250, 8, fmt, 50, None) == INVALID
        assert f(None, FAKE, FAKE, FAKE, 4, 256, 8, fmt, 64, None) == INVALID
    assert f(None, FAKE, FAKE, FAKE, 4, 256, 8, 0, 64, None) == INVALID
    assert f(FAKE, FAKE, None, FAKE, 4, 256, 8, 1, 64, None) == INVALID
    assert f(FAKE, FAKE, FAKE, FAKE, 4, 256, 8, 0, 48, None) == INVALID


def test_quantize_validation(lib):
    """Host-side checks only (every call returns before any HIP call)."""
    f = lib.qmm_quantize
    assert f(None, FAKE, FAKE, FAKE, 256, 8, 4, 64, None) == INVALID
    assert f(FAKE, None, FAKE, FAKE, 256, 8, 4, 64, None) == INVALID
    assert f(FAKE, FAKE, None, FAKE, 256, 8, 4, 64, None) == INVALID
    assert f(FAKE, FAKE, FAKE, None, 256, 8, 4, 64, None) == INVALID
    assert f(FAKE, FAKE, FAKE, FAKE, 256, 8, 9, 64, None) == INVALID
    assert f(FAKE, FAKE, FAKE, FAKE, 256, 8, 4, 48, None) == INVALID
    assert f(FAKE, FAKE, FAKE, FAKE, 250, 8, 4, 50, None) == INVALID
    assert f(FAKE, FAKE, FAKE, FAKE, 256, 0, 4, 64, None) == INVALID
    assert f(FAKE, FAKE, FAKE, FAKE, 32 * 65536, 1, 4, 32, None) == UNSUPPORTED


def test_status_strings(lib):
    assert lib.qmm_status_string(OK) == b"ok"
    for st in (INVALID, UNSUPPORTED, HIPERR):
        assert lib.qmm_status_string(st) and lib.qmm_status_string(st) != b"ok"


def test_last_hip_error_is_the_error_text(lib):
    """qmm_last_hip_error (the boundary's name for the thread-local error text)
    reports the same message as qmm_last_error."""
    assert lib.qmm_gemv(FAKE, FAKE, FAKE, None, FAKE, 17, 4096, 8, 4, 128, None) == INVALID
    msg = lib.qmm_last_hip_error()
    assert msg and msg == lib.qmm_last_error() and b"qmm_gemv" in msg


def test_probe_validation(lib):
    """The measurement hooks check their arguments before any HIP call."""
    assert lib.qmm_probe_read(None, 1024, FAKE, 4, None) == INVALID
    assert lib.qmm_probe_read(FAKE, 1024, None, 4, None) == INVALID
    assert lib.qmm_probe_read(FAKE, 1000, FAKE, 4, None) == INVALID
    assert lib.qmm_probe_read(FAKE, 1024, FAKE, 0, None) == INVALID
    assert lib.qmm_probe_mfma(None, 10, 4, 0, None) == INVALID
    assert lib.qmm_probe_mfma(FAKE, 0, 4, 0, None) == INVALID
    assert lib.qmm_probe_mfma(FAKE, 10, 4, 2, None) == INVALID
    assert lib.qmm_probe_mfma(FAKE, 10, 70000, 0, None) == INVALID


def test_gemv_lut_validation(lib):
    """The table-lookup entry point: shape checks, then its own limits
    (M == 1, bits == 1, K <= 8192) before any HIP call."""
    f = lib.qmm_gemv_lut
    assert f(FAKE, FAKE, FAKE, None, FAKE, 1, 4016, 8, 1, 32, None) == INVALID
    assert f(None, FAKE, FAKE, None, FAKE, 1, 256, 8, 1, 64, None) == INVALID
    assert f(FAKE, FAKE, FAKE, None, FAKE, 2, 256, 8, 1, 64, None) == UNSUPPORTED
    assert f(FAKE, FAKE, FAKE, None, FAKE, 1, 256, 8, 2, 64, None) == UNSUPPORTED
    assert f(FAKE, FAKE, FAKE, None, FAKE, 1, 8224, 8, 1, 32, None) == UNSUPPORTED


class _Prob(ctypes.Structure):
    _fields_ = [("X", ctypes.c_void_p), ("wq", ctypes.c_void_p), ("s", ctypes.c_void_p), ("z", ctypes.c_void_p),
                ("Y", ctypes.c_void_p), ("N", ctypes.c_int64), ("bits", ctypes.c_int)]


def test_gemv_grouped_validation(lib):
    """Host-side checks of the grouped decode entry point (nothing launches)."""
    f = lib.qmm_gemv_grouped
    f.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p]
    f.restype = ctypes.c_int
    good = _Prob(0x1000, 0x1000, 0x1000, None, 0x1000, 64, 4)
    arr = (_Prob * 17)(*([good] * 17))
    ptr = ctypes.cast(arr, ctypes.c_void_p)
    assert f(None, 1, 256, 64, None) == INVALID
    assert f(ptr, 0, 256, 64, None) == INVALID
    assert f(ptr, 17, 256, 64, None) == INVALID
    assert f(ptr, 2, 4016, 64, None) == INVALID          # K % 32
    assert f(ptr, 2, 256, 48, None) == INVALID           # G % 32
    assert f(ptr, 2, 32768, 128, None) == UNSUPPORTED    # K beyond the decode kernel
    bad = (_Prob * 2)(good, _Prob(0x1000, None, 0x1000, None, 0x1000, 64, 4))
    assert f(ctypes.cast(bad, ctypes.c_void_p), 2, 256, 64, None) == INVALID
    bad = (_Prob * 2)(good, _Prob(0x1000, 0x1000, 0x1000, None, 0x1000, 64, 9))
    assert f(ctypes.cast(bad, ctypes.c_void_p), 2, 256, 64, None) == INVALID
    bad = (_Prob * 2)(good, _Prob(0x1000, 0x1000, 0x1000, None, 0x1000, 0, 4))
    assert f(ctypes.cast(bad, ctypes.c_void_p), 2, 256, 64, None) == INVALID
