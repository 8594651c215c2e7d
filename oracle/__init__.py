"""CPU oracle for the MXFP4 GEMM -- TEST INFRASTRUCTURE ONLY.

Only the test suite, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product path (the HIP library and
its Python binding) never does, and shares no code with it.

The arithmetic lives in ``mxfp4_oracle.c`` (scalar C, built by ``build.py``);
this module only moves numpy arrays across ctypes.  Bit patterns are passed as
numpy ``uint16`` (bf16) and ``uint8`` (fp4x2 and e8m0) arrays.

Sources (kernelindex.com "kernelbot amd-mxfp4-mm" submissions):
  * scale rule -- submission 752099 `_bf16_to_fp4_hw`, submission 754549
    `_quantize_mxfp4`, submission 739530 `hw_quant32` (zero group);
  * element rounding, saturation, sign and nibble order -- submission 694791
    `_mxfp4_quant_tile`;
  * fp32-accumulated block-scaled dot -- submission 752099
    `_quant_gemm_fused_launcher` (`tl.dot_scaled`).
"""
import ctypes
import os

import numpy as np

from . import build as _build

_LIB = None
_u8p = ctypes.POINTER(ctypes.c_uint8)
_u16p = ctypes.POINTER(ctypes.c_uint16)
_f32p = ctypes.POINTER(ctypes.c_float)
_f64p = ctypes.POINTER(ctypes.c_double)
_i64 = ctypes.c_int64


def _lib():
    global _LIB
    if _LIB is None:
        path = os.environ.get("MXFP4_ORACLE_LIB") or _build.LIB  # override: pin-strength test
        if path == _build.LIB and (not os.path.exists(path)
                                   or os.path.getmtime(path) < os.path.getmtime(_build.SRC)):
            _build.build()
        lib = ctypes.CDLL(path)
        lib.oracle_scale_byte.argtypes = [ctypes.c_float]
        lib.oracle_scale_byte.restype = ctypes.c_int
        lib.oracle_e2m1_code.argtypes = [ctypes.c_float, ctypes.c_int]
        lib.oracle_e2m1_code.restype = ctypes.c_int
        lib.oracle_e2m1_codes.argtypes = [_f32p, ctypes.POINTER(ctypes.c_int32), _i64, _u8p]
        lib.oracle_e2m1_codes.restype = ctypes.c_int
        lib.oracle_dequant_value.argtypes = [ctypes.c_int, ctypes.c_int]
        lib.oracle_dequant_value.restype = ctypes.c_double
        lib.oracle_quantize_rows.argtypes = [_u16p, _i64, _i64, _i64, _u8p, _u8p]
        lib.oracle_quantize_rows.restype = ctypes.c_int
        lib.oracle_dequantize.argtypes = [_u8p, _u8p, _i64, _i64, _f64p]
        lib.oracle_dequantize.restype = ctypes.c_int
        lib.oracle_gemm.argtypes = [_f64p, _f64p, _i64, _i64, _i64, _f32p, _f64p]
        lib.oracle_gemm.restype = ctypes.c_int
        lib.oracle_gemm_abs.argtypes = [_f64p, _f64p, _i64, _i64, _i64, _f64p]
        lib.oracle_gemm_abs.restype = ctypes.c_int
        _LIB = lib
    return _LIB


def _ptr(a, t):
    return a.ctypes.data_as(t)


def scale_byte(amax: float) -> int:
    """e8m0 scale byte for a group whose largest magnitude is ``amax``."""
    return _lib().oracle_scale_byte(float(amax))


def e2m1_code(x: float, scale_byte_: int) -> int:
    """4-bit code of value ``x`` (an fp32 number) under scale byte ``scale_byte_``."""
    return _lib().oracle_e2m1_code(float(x), int(scale_byte_))


def e2m1_codes(x: np.ndarray, scale_bytes: np.ndarray) -> np.ndarray:
    """Vector form of ``e2m1_code``: fp32 values and int scale bytes of equal length."""
    xv = np.ascontiguousarray(x, dtype=np.float32).reshape(-1)
    sv = np.ascontiguousarray(np.broadcast_to(scale_bytes, xv.shape), dtype=np.int32)
    out = np.empty(xv.shape, dtype=np.uint8)
    _lib().oracle_e2m1_codes(_ptr(xv, _f32p), sv.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)),
                             xv.size, _ptr(out, _u8p))
    return out


def dequant_value(code: int, scale_byte_: int) -> float:
    return _lib().oracle_dequant_value(int(code), int(scale_byte_))


def quantize(x_bf16: np.ndarray):
    """Quantize a [rows, K] bf16 bit array; returns (fp4x2 [rows, K/2], e8m0 [rows, K/32])."""
    x = np.ascontiguousarray(x_bf16, dtype=np.uint16)
    rows, K = x.shape
    q = np.zeros((rows, K // 2), dtype=np.uint8)
    s = np.zeros((rows, K // 32), dtype=np.uint8)
    rc = _lib().oracle_quantize_rows(_ptr(x, _u16p), rows, K, K, _ptr(q, _u8p), _ptr(s, _u8p))
    if rc != 0:
        raise ValueError("oracle quantize: K must be a multiple of 32 (got %d)" % K)
    return q, s


def dequantize(fp4: np.ndarray, scale: np.ndarray) -> np.ndarray:
    """Dequantize linear fp4x2 [rows, K/2] + e8m0 [rows, K/32] to float64 [rows, K]."""
    q = np.ascontiguousarray(fp4, dtype=np.uint8)
    s = np.ascontiguousarray(scale, dtype=np.uint8)
    rows, half = q.shape
    K = 2 * half
    if s.shape != (rows, K // 32):
        raise ValueError("scale shape %s does not match fp4 shape %s" % (s.shape, q.shape))
    out = np.empty((rows, K), dtype=np.float64)
    rc = _lib().oracle_dequantize(_ptr(q, _u8p), _ptr(s, _u8p), rows, K, _ptr(out, _f64p))
    if rc != 0:
        raise ValueError("oracle dequantize failed")
    return out


def gemm(a_deq: np.ndarray, b_deq: np.ndarray, want64: bool = True):
    """C[m, n] = sum_k a[m, k] * b[n, k]: returns (fp32 running sum, fp64 sum or None)."""
    a = np.ascontiguousarray(a_deq, dtype=np.float64)
    b = np.ascontiguousarray(b_deq, dtype=np.float64)
    M, K = a.shape
    N, K2 = b.shape
    if K != K2:
        raise ValueError("K mismatch")
    c32 = np.empty((M, N), dtype=np.float32)
    c64 = np.empty((M, N), dtype=np.float64) if want64 else None
    rc = _lib().oracle_gemm(_ptr(a, _f64p), _ptr(b, _f64p), M, N, K, _ptr(c32, _f32p),
                            _ptr(c64, _f64p) if want64 else None)
    if rc != 0:
        raise ValueError("oracle gemm failed")
    return c32, c64


def gemm_abs(a_deq: np.ndarray, b_deq: np.ndarray) -> np.ndarray:
    """sum_k |a[m, k] * b[n, k]|, for error bounds."""
    a = np.ascontiguousarray(a_deq, dtype=np.float64)
    b = np.ascontiguousarray(b_deq, dtype=np.float64)
    M, K = a.shape
    N, _ = b.shape
    out = np.empty((M, N), dtype=np.float64)
    _lib().oracle_gemm_abs(_ptr(a, _f64p), _ptr(b, _f64p), M, N, K, _ptr(out, _f64p))
    return out


def reference(a_bf16: np.ndarray, b_bf16: np.ndarray, want64: bool = False):
    """Whole reference pipeline: quantize A and B, dequantize, fp32 dot.

    Returns a dict with the quantized operands, their dequantized values and
    ``c32`` (plus ``c64`` when asked for)."""
    aq, asc = quantize(a_bf16)
    bq, bsc = quantize(b_bf16)
    ad = dequantize(aq, asc)
    bd = dequantize(bq, bsc)
    c32, c64 = gemm(ad, bd, want64=want64)
    return {"aq": aq, "as": asc, "bq": bq, "bs": bsc, "ad": ad, "bd": bd, "c32": c32, "c64": c64}
