"""Thin ctypes binding of libzq.so (C-ABI in include/zq.h).

Argument marshalling only: every step runs in the HIP kernels of libzq. Tensors
must live on a ROCm device; calls enqueue on torch's current stream. There is
no CPU path: if the library is missing, every call raises.
"""
from __future__ import annotations

import atexit
import ctypes
import os
import sys
import weakref
from dataclasses import dataclass

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libzq.so")

OK, ERR_INVALID_ARG, ERR_UNSUPPORTED, ERR_RANGE, ERR_HIP = 0, 1, 2, 3, 4
I8, F16, BF16, F32 = 0, 1, 2, 3
_DT = {torch.int8: I8, torch.float16: F16, torch.bfloat16: BF16, torch.float32: F32}

# every exported symbol of include/zq.h
SYMBOLS = ("zq_packed_bytes", "zq_num_scales", "zq_pack", "zq_pack_noalloc", "zq_pack_asym", "zq_unpack",
           "zq_gemv", "zq_gemm",
           "zq_plan_create", "zq_plan_run", "zq_plan_check", "zq_plan_destroy",
           "zq_status_string", "zq_last_error")


class ZqError(RuntimeError):
    def __init__(self, status: int, call: str, detail: str):
        super().__init__(f"{call}: status {status} ({detail})")
        self.status = status


class _Weight(ctypes.Structure):
    _fields_ = [("bits", ctypes.c_int32), ("group", ctypes.c_int32), ("n", ctypes.c_int64),
                ("k", ctypes.c_int64), ("packed", ctypes.c_void_p), ("scales", ctypes.c_void_p),
                ("zeros", ctypes.c_void_p)]


class _Problem(ctypes.Structure):
    _fields_ = [("w", _Weight), ("x", ctypes.c_void_p), ("x_dtype", ctypes.c_int32),
                ("ldx", ctypes.c_int64), ("y", ctypes.c_void_p), ("y_dtype", ctypes.c_int32),
                ("ldy", ctypes.c_int64), ("phase", ctypes.c_int32)]


_lib = None


def lib() -> ctypes.CDLL:
    """Load libzq.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m weight_quantized_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        vp, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
        wp = ctypes.POINTER(_Weight)
        L.zq_packed_bytes.argtypes = [i32, i64, i64]
        L.zq_packed_bytes.restype = ctypes.c_size_t
        L.zq_num_scales.argtypes = [i32, i64, i64]
        L.zq_num_scales.restype = i64
        L.zq_pack.argtypes = [vp, i32, i64, i64, i32, i32, vp, vp, vp, vp]
        L.zq_pack_noalloc.argtypes = [vp, i32, i64, i64, i32, i32, vp, vp, vp, vp]
        L.zq_pack_asym.argtypes = [vp, i32, i64, i64, i32, vp, vp, vp, vp, vp, vp]
        L.zq_unpack.argtypes = [wp, vp, i32, vp]
        L.zq_gemv.argtypes = [wp, vp, i32, vp, i32, vp]
        L.zq_gemm.argtypes = [wp, vp, i32, i64, i64, vp, i32, i64, vp]
        for f in ("zq_pack", "zq_pack_noalloc", "zq_pack_asym", "zq_unpack", "zq_gemv", "zq_gemm"):
            getattr(L, f).restype = i32
        L.zq_plan_create.argtypes = [ctypes.POINTER(_Problem), i32, i64, ctypes.POINTER(vp)]
        L.zq_plan_run.argtypes = [vp, vp]
        L.zq_plan_check.argtypes = [vp]
        L.zq_plan_destroy.argtypes = [vp]
        for f in ("zq_plan_create", "zq_plan_run", "zq_plan_check", "zq_plan_destroy"):
            getattr(L, f).restype = i32
        L.zq_status_string.argtypes = [i32]
        L.zq_status_string.restype = ctypes.c_char_p
        L.zq_last_error.argtypes = []
        L.zq_last_error.restype = ctypes.c_char_p
        _lib = L
    return _lib


def _check(status: int, call: str) -> None:
    if status != OK:
        raise ZqError(status, call, lib().zq_last_error().decode())


def _stream(t: torch.Tensor) -> int:
    return torch.cuda.current_stream(t.device).cuda_stream


def _ptr(t: torch.Tensor | None) -> int | None:
    return None if t is None else t.data_ptr()


def packed_bytes(bits: int, n: int, k: int) -> int:
    return lib().zq_packed_bytes(bits, n, k)


def num_scales(group: int, n: int, k: int) -> int:
    return lib().zq_num_scales(group, n, k)


@dataclass
class ZqWeight:
    """A packed weight matrix in device memory: codes [n][k*bits/8] uint8 and
    fp16 scales; with `zeros` (fp16 [n][k/128]) the codes are unsigned and the
    weights asymmetric (w = q * s + z)."""
    bits: int
    group: int
    n: int
    k: int
    packed: torch.Tensor
    scales: torch.Tensor
    zeros: torch.Tensor | None = None

    def desc(self) -> _Weight:
        return _Weight(self.bits, self.group, self.n, self.k, _ptr(self.packed), _ptr(self.scales),
                       _ptr(self.zeros))

    @property
    def nbytes(self) -> int:
        return self.packed.numel() + 2 * self.scales.numel() + (0 if self.zeros is None else 2 * self.zeros.numel())


def pack(w: torch.Tensor, bits: int, group: int, scales: torch.Tensor | None = None) -> ZqWeight:
    """Quantize (float w) or bit-pack (int8 codes) an [n][k] device tensor. Synchronous."""
    n, k = w.shape
    w = w.contiguous()
    nb = packed_bytes(bits, n, k)
    ns = num_scales(group, n, k)
    packed = torch.empty(max(nb, 0), dtype=torch.uint8, device=w.device)
    out_scales = torch.empty(max(ns, 1), dtype=torch.float16, device=w.device)
    sin = None if scales is None else scales.contiguous()
    _check(lib().zq_pack(_ptr(w), _DT.get(w.dtype, -1), n, k, bits, group, _ptr(sin), _ptr(packed),
                         _ptr(out_scales), _stream(w)), "zq_pack")
    return ZqWeight(bits, group, n, k, packed, out_scales)


def pack_into(w: torch.Tensor, bits: int, group: int, packed: torch.Tensor, scales_out: torch.Tensor | None,
              scales: torch.Tensor | None = None, noalloc: bool = False) -> None:
    """zq_pack (or, with noalloc, zq_pack_noalloc) into caller-given outputs:
    packed (uint8, >= packed_bytes) and scales_out (fp16, >= num_scales, or
    None with int8 codes or given scales). Synchronous."""
    n, k = w.shape
    if not w.is_contiguous():
        raise ValueError("w must be contiguous")
    if packed.numel() < packed_bytes(bits, n, k) or (scales_out is not None and
                                                     scales_out.numel() < num_scales(group, n, k)):
        raise ValueError("output buffers too small")
    fn = lib().zq_pack_noalloc if noalloc else lib().zq_pack
    _check(fn(_ptr(w), _DT.get(w.dtype, -1), n, k, bits, group, _ptr(scales), _ptr(packed), _ptr(scales_out),
              _stream(w)), "zq_pack_noalloc" if noalloc else "zq_pack")


def pack_asym(w: torch.Tensor, bits: int, scales: torch.Tensor | None = None,
              zeros: torch.Tensor | None = None) -> ZqWeight:
    """Asymmetric quantize (float w) or bit-pack (int8 unsigned codes) an [n][k]
    device tensor, with fp16 scale and zero point per 128-group. Synchronous."""
    n, k = w.shape
    w = w.contiguous()
    packed = torch.empty(max(packed_bytes(bits, n, k), 0), dtype=torch.uint8, device=w.device)
    ng = max(n * (k // 128), 1)
    out_s = torch.empty(ng, dtype=torch.float16, device=w.device)
    out_z = torch.empty(ng, dtype=torch.float16, device=w.device)
    sin = None if scales is None else scales.contiguous()
    zin = None if zeros is None else zeros.contiguous()
    _check(lib().zq_pack_asym(_ptr(w), _DT.get(w.dtype, -1), n, k, bits, _ptr(sin), _ptr(zin), _ptr(packed),
                              _ptr(out_s), _ptr(out_z), _stream(w)), "zq_pack_asym")
    return ZqWeight(bits, 128, n, k, packed, out_s, out_z)


def unpack(W: ZqWeight, dtype: torch.dtype = torch.int8) -> torch.Tensor:
    out = torch.empty((W.n, W.k), dtype=dtype, device=W.packed.device)
    d = W.desc()
    _check(lib().zq_unpack(ctypes.byref(d), _ptr(out), _DT.get(dtype, -1), _stream(out)), "zq_unpack")
    return out


def gemv(W: ZqWeight, x: torch.Tensor, out: torch.Tensor | None = None,
         out_dtype: torch.dtype = torch.float32) -> torch.Tensor:
    """y[n] = sum_k x[k] * w_deq[n][k] for one activation row x [k]."""
    if x.numel() < W.k or not x.is_contiguous():
        raise ValueError(f"x must hold {W.k} contiguous elements")
    if out is None:
        out = torch.empty(W.n, dtype=out_dtype, device=x.device)
    if out.numel() < W.n or not out.is_contiguous():
        raise ValueError(f"out must hold {W.n} contiguous elements")
    d = W.desc()
    _check(lib().zq_gemv(ctypes.byref(d), _ptr(x), _DT.get(x.dtype, -1), _ptr(out),
                         _DT.get(out.dtype, -1), _stream(x)), "zq_gemv")
    return out


def gemm(W: ZqWeight, X: torch.Tensor, out: torch.Tensor | None = None,
         out_dtype: torch.dtype = torch.float32) -> torch.Tensor:
    """Y[m][n] = sum_k X[m][k] * w_deq[n][k]; X may have a row stride >= k."""
    m = X.shape[0]
    if X.dim() != 2 or X.stride(1) != 1 or X.shape[1] < W.k:
        raise ValueError(f"X must be [m, >= {W.k}] with contiguous rows")
    if out is None:
        out = torch.empty((m, W.n), dtype=out_dtype, device=X.device)
    if out.dim() != 2 or out.stride(1) != 1 or out.shape[0] != m or out.shape[1] < W.n:
        raise ValueError(f"out must be [{m}, >= {W.n}] with contiguous rows")
    d = W.desc()
    _check(lib().zq_gemm(ctypes.byref(d), _ptr(X), _DT.get(X.dtype, -1), m, X.stride(0), _ptr(out),
                         _DT.get(out.dtype, -1), out.stride(0), _stream(X)), "zq_gemm")
    return out


def gemm_raw(W: ZqWeight, x_ptr: int, x_dtype: int, m: int, ldx: int, y_ptr: int, y_dtype: int,
             ldy: int, stream: int) -> None:
    """zq_gemm on raw device pointers (benchmark loops: no tensor bookkeeping)."""
    d = W.desc()
    _check(lib().zq_gemm(ctypes.byref(d), x_ptr, x_dtype, m, ldx, y_ptr, y_dtype, ldy, stream),
           "zq_gemm")


# Plans still open when the interpreter exits are closed by an atexit hook,
# which runs before torch's own exit handlers (registered earlier, run later)
# tear down the device: no HIP call is left for object finalisation.
_live_plans: "weakref.WeakSet[Plan]" = weakref.WeakSet()


def _close_live_plans() -> None:
    for p in list(_live_plans):
        try:
            p.close()
        except Exception:
            pass


atexit.register(_close_live_plans)


class Plan:
    """Many products in one resident launch (zq_plan_*). `problems` is a list of
    (ZqWeight, X [m, k], Y [m, n], phase); phases must not decrease. Every X
    and Y has the same m rows (the C-ABI cannot see tensor sizes)."""

    def __init__(self, problems):
        self._h = None
        self._keep = problems  # the plan reads these buffers at every run
        m = problems[0][1].shape[0] if problems[0][1].dim() == 2 else 1
        arr = (_Problem * len(problems))()
        for i, (W, X, Y, phase) in enumerate(problems):
            X2 = X if X.dim() == 2 else X.view(1, -1)
            Y2 = Y if Y.dim() == 2 else Y.view(1, -1)
            if X2.shape[0] != m or Y2.shape[0] != m:
                raise ValueError(f"problem {i}: X and Y need {m} rows (got {X2.shape[0]} and {Y2.shape[0]})")
            if X2.shape[1] < W.k or Y2.shape[1] < W.n or X2.stride(1) != 1 or Y2.stride(1) != 1:
                raise ValueError(f"problem {i}: X must be [m, >= {W.k}] and Y [m, >= {W.n}], rows contiguous")
            arr[i] = _Problem(W.desc(), _ptr(X2), _DT.get(X2.dtype, -1), X2.stride(0), _ptr(Y2),
                              _DT.get(Y2.dtype, -1), Y2.stride(0), phase)
        h = ctypes.c_void_p()
        _check(lib().zq_plan_create(arr, len(problems), m, ctypes.byref(h)), "zq_plan_create")
        self._h = h
        self.device = problems[0][1].device
        _live_plans.add(self)

    def run(self) -> None:
        _check(lib().zq_plan_run(self._h, torch.cuda.current_stream(self.device).cuda_stream), "zq_plan_run")

    def check(self) -> None:
        _check(lib().zq_plan_check(self._h), "zq_plan_check")

    def close(self) -> None:
        if self._h:
            _check(lib().zq_plan_destroy(self._h), "zq_plan_destroy")
            self._h = None

    def __enter__(self) -> "Plan":
        return self

    def __exit__(self, *exc) -> None:
        self.close()

    def __del__(self):
        # no HIP call while the interpreter shuts down: live plans were closed
        # by the atexit hook, and anything left is freed with the process
        if sys.is_finalizing():
            return
        try:
            self.close()
        except Exception:
            pass
