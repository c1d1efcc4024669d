"""ctypes wrapper over the plain fp64 C oracle (zq_oracle.c).

TEST INFRASTRUCTURE. Only the test suite, the smoke check and the benchmark's
CPU-baseline leg may import this module. The product library never does.

Arrays are numpy arrays. bfloat16 data travels as uint16 bit patterns tagged
with the dtype name "bf16"; float16 data may be given as numpy float16 or as
uint16 bit patterns tagged "f16".
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "zq_oracle.c")
LIB = os.path.join(HERE, "libzq_oracle.so")

OK, ERR_INVALID_ARG, ERR_UNSUPPORTED, ERR_RANGE = 0, 1, 2, 3
DTYPES = {"i8": 0, "f16": 1, "bf16": 2, "f32": 3}

_lib = None


def build(force: bool = False) -> str:
    """Compile the oracle with gcc (no fp contraction, so sums are plain)."""
    if force or not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SRC):
        tmp = LIB + ".tmp"
        subprocess.check_call(
            ["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math",
             "-shared", "-fPIC", "-o", tmp, SRC, "-lm"])
        os.replace(tmp, LIB)
    return LIB


def lib():
    global _lib
    if _lib is None:
        build()
        L = ctypes.CDLL(LIB)
        vp, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
        L.zqo_f16_to_f64.argtypes = [ctypes.c_uint16]
        L.zqo_f16_to_f64.restype = ctypes.c_double
        L.zqo_bf16_to_f64.argtypes = [ctypes.c_uint16]
        L.zqo_bf16_to_f64.restype = ctypes.c_double
        L.zqo_f64_to_f16.argtypes = [ctypes.c_double]
        L.zqo_f64_to_f16.restype = ctypes.c_uint16
        L.zqo_f64_to_bf16.argtypes = [ctypes.c_double]
        L.zqo_f64_to_bf16.restype = ctypes.c_uint16
        L.zqo_compute_scales.argtypes = [vp, i32, i64, i64, i32, i32, vp]
        L.zqo_quantize.argtypes = [vp, i32, i64, i64, i32, i32, vp, vp]
        L.zqo_pack.argtypes = [vp, i64, i64, i32, vp]
        L.zqo_unpack.argtypes = [vp, i64, i64, i32, vp]
        L.zqo_unpack.restype = None
        L.zqo_dequant.argtypes = [vp, i64, i64, i32, vp, vp]
        L.zqo_dequant.restype = None
        L.zqo_gemm.argtypes = [vp, i32, vp, i32, i64, i64, vp, i32, i64, i64, vp, i64]
        for f in ("zqo_compute_scales", "zqo_quantize", "zqo_pack", "zqo_gemm"):
            getattr(L, f).restype = ctypes.c_int
        L.zqo_compute_scales_zeros.argtypes = [vp, i32, i64, i64, i32, vp, vp]
        L.zqo_quantize_asym.argtypes = [vp, i32, i64, i64, i32, vp, vp, vp]
        L.zqo_pack_u.argtypes = [vp, i64, i64, i32, vp]
        L.zqo_unpack_u.argtypes = [vp, i64, i64, i32, vp]
        L.zqo_unpack_u.restype = None
        L.zqo_dequant_asym.argtypes = [vp, i64, i64, vp, vp, vp]
        L.zqo_dequant_asym.restype = None
        L.zqo_gemm_asym.argtypes = [vp, i32, vp, vp, i64, i64, vp, i32, i64, i64, vp, i64]
        for f in ("zqo_compute_scales_zeros", "zqo_quantize_asym", "zqo_pack_u", "zqo_gemm_asym"):
            getattr(L, f).restype = ctypes.c_int
        _lib = L
    return _lib


class OracleError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__(f"{what}: oracle status {status}")
        self.status = status


def _ptr(a: np.ndarray) -> int:
    return a.ctypes.data


def _typed(a: np.ndarray, dtype: str) -> np.ndarray:
    """Contiguous array with the storage the C side expects for `dtype`."""
    if dtype == "f16":
        a = a.view(np.uint16) if a.dtype == np.float16 else a
        assert a.dtype == np.uint16
    elif dtype == "bf16":
        assert a.dtype == np.uint16, "bf16 data is passed as uint16 bit patterns"
    elif dtype == "f32":
        assert a.dtype == np.float32
    elif dtype == "i8":
        assert a.dtype == np.int8
    return np.ascontiguousarray(a)


def f16_to_f64(bits: int) -> float:
    return lib().zqo_f16_to_f64(int(bits))


def bf16_to_f64(bits: int) -> float:
    return lib().zqo_bf16_to_f64(int(bits))


def f64_to_f16(v: float) -> int:
    return lib().zqo_f64_to_f16(float(v))


def f64_to_bf16(v: float) -> int:
    return lib().zqo_f64_to_bf16(float(v))


def num_scales(group: int, n: int, k: int) -> int:
    return 1 if group == 0 else n * (k // group)


def compute_scales(w: np.ndarray, dtype: str, bits: int, group: int) -> np.ndarray:
    w = _typed(w, dtype)
    n, k = w.shape
    out = np.zeros(num_scales(group, n, k), dtype=np.uint16)
    st = lib().zqo_compute_scales(_ptr(w), DTYPES[dtype], n, k, bits, group, _ptr(out))
    if st:
        raise OracleError(st, "compute_scales")
    return out


def quantize(w: np.ndarray, dtype: str, bits: int, group: int, scales: np.ndarray) -> np.ndarray:
    w = _typed(w, dtype)
    n, k = w.shape
    scales = np.ascontiguousarray(scales, dtype=np.uint16)
    codes = np.zeros((n, k), dtype=np.int8)
    st = lib().zqo_quantize(_ptr(w), DTYPES[dtype], n, k, bits, group, _ptr(scales), _ptr(codes))
    if st:
        raise OracleError(st, "quantize")
    return codes


def pack(codes: np.ndarray, bits: int) -> np.ndarray:
    codes = np.ascontiguousarray(codes, dtype=np.int8)
    n, k = codes.shape
    out = np.zeros((n, k * bits // 8), dtype=np.uint8)
    st = lib().zqo_pack(_ptr(codes), n, k, bits, _ptr(out))
    if st:
        raise OracleError(st, "pack")
    return out


def unpack(packed: np.ndarray, n: int, k: int, bits: int) -> np.ndarray:
    packed = np.ascontiguousarray(packed, dtype=np.uint8)
    assert packed.size == n * k * bits // 8
    out = np.zeros((n, k), dtype=np.int8)
    lib().zqo_unpack(_ptr(packed), n, k, bits, _ptr(out))
    return out


def dequant(codes: np.ndarray, group: int, scales: np.ndarray) -> np.ndarray:
    codes = np.ascontiguousarray(codes, dtype=np.int8)
    n, k = codes.shape
    scales = np.ascontiguousarray(scales, dtype=np.uint16)
    out = np.zeros((n, k), dtype=np.float64)
    lib().zqo_dequant(_ptr(codes), n, k, group, _ptr(scales), _ptr(out))
    return out


def gemm(packed: np.ndarray, bits: int, scales: np.ndarray, group: int, n: int, k: int,
         x: np.ndarray, x_dtype: str) -> np.ndarray:
    """y[m][n] in float64 for x of shape [m][k] (or [k] for one row)."""
    packed = np.ascontiguousarray(packed, dtype=np.uint8)
    scales = np.ascontiguousarray(scales, dtype=np.uint16)
    x = _typed(x, x_dtype)
    one = x.ndim == 1
    x2 = x.reshape(1, -1) if one else x
    m = x2.shape[0]
    assert x2.shape[1] == k
    y = np.zeros((m, n), dtype=np.float64)
    st = lib().zqo_gemm(_ptr(packed), bits, _ptr(scales), group, n, k, _ptr(x2),
                        DTYPES[x_dtype], m, k, _ptr(y), n)
    if st:
        raise OracleError(st, "gemm")
    return y[0] if one else y


def gemm_rows(packed: np.ndarray, bits: int, scales: np.ndarray, group: int, n: int, k: int,
              x: np.ndarray, x_dtype: str, rows: np.ndarray) -> np.ndarray:
    """y[:, rows] only: each selected weight row is passed to the oracle on its own."""
    rows = np.asarray(rows, dtype=np.int64)
    packed = np.ascontiguousarray(packed, dtype=np.uint8).reshape(n, -1)
    scales = np.ascontiguousarray(scales, dtype=np.uint16)
    x2 = x.reshape(1, -1) if x.ndim == 1 else x
    out = np.zeros((x2.shape[0], rows.size), dtype=np.float64)
    for j, r in enumerate(rows):
        sc = scales if group == 0 else scales.reshape(n, -1)[r]
        out[:, j] = gemm(packed[r:r + 1], bits, sc, group, 1, k, x2, x_dtype)[:, 0]
    return out


# ---------------------------------------------------------------------------
# asymmetric variant: unsigned codes, fp16 scale and zero point per 128-group


def compute_scales_zeros(w: np.ndarray, dtype: str, bits: int):
    w = _typed(w, dtype)
    n, k = w.shape
    sc = np.zeros(n * (k // 128), dtype=np.uint16)
    zr = np.zeros(n * (k // 128), dtype=np.uint16)
    st = lib().zqo_compute_scales_zeros(_ptr(w), DTYPES[dtype], n, k, bits, _ptr(sc), _ptr(zr))
    if st:
        raise OracleError(st, "compute_scales_zeros")
    return sc, zr


def quantize_asym(w: np.ndarray, dtype: str, bits: int, scales: np.ndarray, zeros: np.ndarray) -> np.ndarray:
    w = _typed(w, dtype)
    n, k = w.shape
    scales = np.ascontiguousarray(scales, dtype=np.uint16)
    zeros = np.ascontiguousarray(zeros, dtype=np.uint16)
    codes = np.zeros((n, k), dtype=np.uint8)
    st = lib().zqo_quantize_asym(_ptr(w), DTYPES[dtype], n, k, bits, _ptr(scales), _ptr(zeros), _ptr(codes))
    if st:
        raise OracleError(st, "quantize_asym")
    return codes


def pack_u(codes: np.ndarray, bits: int) -> np.ndarray:
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    n, k = codes.shape
    out = np.zeros((n, k * bits // 8), dtype=np.uint8)
    st = lib().zqo_pack_u(_ptr(codes), n, k, bits, _ptr(out))
    if st:
        raise OracleError(st, "pack_u")
    return out


def unpack_u(packed: np.ndarray, n: int, k: int, bits: int) -> np.ndarray:
    packed = np.ascontiguousarray(packed, dtype=np.uint8)
    assert packed.size == n * k * bits // 8
    out = np.zeros((n, k), dtype=np.uint8)
    lib().zqo_unpack_u(_ptr(packed), n, k, bits, _ptr(out))
    return out


def dequant_asym(codes: np.ndarray, scales: np.ndarray, zeros: np.ndarray) -> np.ndarray:
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    n, k = codes.shape
    scales = np.ascontiguousarray(scales, dtype=np.uint16)
    zeros = np.ascontiguousarray(zeros, dtype=np.uint16)
    out = np.zeros((n, k), dtype=np.float64)
    lib().zqo_dequant_asym(_ptr(codes), n, k, _ptr(scales), _ptr(zeros), _ptr(out))
    return out


def gemm_asym(packed: np.ndarray, bits: int, scales: np.ndarray, zeros: np.ndarray, n: int, k: int,
              x: np.ndarray, x_dtype: str) -> np.ndarray:
    """y[m][n] in float64 for x of shape [m][k] (or [k] for one row)."""
    packed = np.ascontiguousarray(packed, dtype=np.uint8)
    scales = np.ascontiguousarray(scales, dtype=np.uint16)
    zeros = np.ascontiguousarray(zeros, dtype=np.uint16)
    x = _typed(x, x_dtype)
    one = x.ndim == 1
    x2 = x.reshape(1, -1) if one else x
    m = x2.shape[0]
    assert x2.shape[1] == k
    y = np.zeros((m, n), dtype=np.float64)
    st = lib().zqo_gemm_asym(_ptr(packed), bits, _ptr(scales), _ptr(zeros), n, k, _ptr(x2),
                             DTYPES[x_dtype], m, k, _ptr(y), n)
    if st:
        raise OracleError(st, "gemm_asym")
    return y[0] if one else y
