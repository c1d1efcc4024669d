"""The C-ABI library loads, exports every symbol its header declares, and
rejects invalid arguments before any HIP call (so these run without a GPU)."""
import ctypes
import os
import re

import pytest

from weight_quantized_amd import zq

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "zq.h")


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(zq.LIB_PATH):
        from weight_quantized_amd import build
        build.build()
    return zq.lib()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(zq_\w+)\s*\(", text)))


def test_header_declares_the_binding_symbols():
    assert declared_functions() == sorted(zq.SYMBOLS)


def test_library_exports_every_declared_symbol(L):
    for name in declared_functions():
        assert hasattr(L, name), name


def test_size_queries(L):
    assert L.zq_packed_bytes(4, 3584, 3584) == 3584 * 1792
    assert L.zq_packed_bytes(2, 512, 3584) == 512 * 896
    assert L.zq_packed_bytes(8, 7, 128) == 7 * 128
    assert L.zq_packed_bytes(3, 7, 128) == 0
    assert L.zq_num_scales(0, 100, 256) == 1
    assert L.zq_num_scales(128, 100, 256) == 200
    assert L.zq_num_scales(64, 100, 256) == -1


def test_status_strings(L):
    for s in range(5):
        assert L.zq_status_string(s)
    assert L.zq_status_string(99) == b"unknown status"


def W(bits=4, group=128, n=16, k=256, packed=0x1000, scales=0x2000):
    return zq._Weight(bits, group, n, k, packed, scales)


def gemm(L, w, x=0x3000, xdt=zq.F16, m=1, ldx=None, y=0x4000, ydt=zq.F32, ldy=None):
    ldx = w.k if ldx is None else ldx
    ldy = w.n if ldy is None else ldy
    return L.zq_gemm(ctypes.byref(w), x, xdt, m, ldx, y, ydt, ldy, None)


# Every case below must be refused by validation, before any HIP call: the
# pointers are bogus host addresses that would fault if anything touched them.
BAD_GEMM = [
    (dict(w=W(bits=3)), zq.ERR_UNSUPPORTED, "bits"),
    (dict(w=W(bits=16)), zq.ERR_UNSUPPORTED, "bits"),
    (dict(w=W(group=64)), zq.ERR_UNSUPPORTED, "group"),
    (dict(w=W(k=200)), zq.ERR_UNSUPPORTED, "multiple of group"),
    (dict(w=W(bits=2, group=0, k=6)), zq.ERR_UNSUPPORTED, "codes per byte"),
    (dict(w=W(n=-1)), zq.ERR_INVALID_ARG, "negative"),
    (dict(w=W(packed=0)), zq.ERR_INVALID_ARG, "null packed"),
    (dict(w=W(scales=0)), zq.ERR_INVALID_ARG, "null packed or scales"),
    (dict(w=W(), xdt=zq.F32), zq.ERR_INVALID_ARG, "x_dtype"),
    (dict(w=W(), xdt=zq.I8), zq.ERR_INVALID_ARG, "x_dtype"),
    (dict(w=W(), ydt=zq.I8), zq.ERR_INVALID_ARG, "y_dtype"),
    (dict(w=W(), m=-2), zq.ERR_INVALID_ARG, "negative m"),
    (dict(w=W(), m=2, ldx=100), zq.ERR_INVALID_ARG, "ldx"),
    (dict(w=W(), ldy=3), zq.ERR_INVALID_ARG, "ldy"),
    (dict(w=W(), x=0), zq.ERR_INVALID_ARG, "null X"),
    (dict(w=W(), y=0), zq.ERR_INVALID_ARG, "null X or Y"),
]


@pytest.mark.parametrize("kw,status,detail", BAD_GEMM)
def test_gemm_validation_without_device(L, kw, status, detail):
    assert gemm(L, **kw) == status
    assert detail in L.zq_last_error().decode()


def test_null_descriptor(L):
    assert L.zq_gemm(None, 0x3000, zq.F16, 1, 256, 0x4000, zq.F32, 16, None) == zq.ERR_INVALID_ARG
    assert L.zq_gemv(None, 0x3000, zq.F16, 0x4000, zq.F32, None) == zq.ERR_INVALID_ARG
    assert L.zq_unpack(None, 0x3000, zq.I8, None) == zq.ERR_INVALID_ARG


def test_empty_problems_are_accepted_without_device(L):
    assert gemm(L, W(), m=0) == zq.OK          # nothing to do: no HIP call
    assert gemm(L, W(n=0)) == zq.OK
    assert L.zq_last_error() == b""


def test_gemv_and_unpack_validation(L):
    w = W(bits=3)
    assert L.zq_gemv(ctypes.byref(w), 0x3000, zq.F16, 0x4000, zq.F32, None) == zq.ERR_UNSUPPORTED
    w = W()
    assert L.zq_gemv(ctypes.byref(w), 0x3000, zq.F32, 0x4000, zq.F32, None) == zq.ERR_INVALID_ARG
    assert L.zq_unpack(ctypes.byref(w), 0x3000, 9, None) == zq.ERR_INVALID_ARG
    assert L.zq_unpack(ctypes.byref(w), 0, zq.F32, None) == zq.ERR_INVALID_ARG


@pytest.mark.parametrize("args,status", [
    ((0x1000, zq.F32, 4, 256, 3, 128, None, 0x2000, 0x3000), zq.ERR_UNSUPPORTED),
    ((0x1000, zq.F32, 4, 256, 4, 32, None, 0x2000, 0x3000), zq.ERR_UNSUPPORTED),
    ((0x1000, zq.F32, 4, 100, 4, 128, None, 0x2000, 0x3000), zq.ERR_UNSUPPORTED),
    ((0x1000, 7, 4, 256, 4, 128, None, 0x2000, 0x3000), zq.ERR_INVALID_ARG),
    ((0, zq.F32, 4, 256, 4, 128, None, 0x2000, 0x3000), zq.ERR_INVALID_ARG),
    ((0x1000, zq.F32, 4, 256, 4, 128, None, 0, 0x3000), zq.ERR_INVALID_ARG),
    ((0x1000, zq.F32, 4, 256, 4, 128, None, 0x2000, None), zq.ERR_INVALID_ARG),
    ((0x1000, zq.F32, -4, 256, 4, 128, None, 0x2000, 0x3000), zq.ERR_INVALID_ARG),
])
def test_pack_validation_without_device(L, args, status):
    assert L.zq_pack(*args, None) == status


@pytest.mark.parametrize("args,status", [
    ((0x1000, zq.F32, 4, 256, 8, None, None, 0x2000, 0x3000, 0x4000), zq.ERR_UNSUPPORTED),   # INT8
    ((0x1000, zq.F32, 4, 200, 4, None, None, 0x2000, 0x3000, 0x4000), zq.ERR_UNSUPPORTED),   # k % 128
    ((0x1000, 7, 4, 256, 4, None, None, 0x2000, 0x3000, 0x4000), zq.ERR_INVALID_ARG),        # dtype
    ((0, zq.F32, 4, 256, 4, None, None, 0x2000, 0x3000, 0x4000), zq.ERR_INVALID_ARG),        # null w
    ((0x1000, zq.F32, 4, 256, 4, 0x5000, None, 0x2000, 0x3000, 0x4000), zq.ERR_INVALID_ARG),  # half given
    ((0x1000, zq.F32, 4, 256, 4, None, None, 0x2000, 0x3000, None), zq.ERR_INVALID_ARG),     # no zeros out
    ((0x1000, zq.I8, 4, 256, 4, None, None, 0x2000, None, None), zq.ERR_INVALID_ARG),        # codes, no s/z
])
def test_pack_asym_validation_without_device(L, args, status):
    assert L.zq_pack_asym(*args, None) == status


def test_asymmetric_weight_validation(L):
    for bits, group in ((8, 128), (4, 0)):
        w = W(bits=bits, group=group)
        w.zeros = 0x7000
        assert L.zq_unpack(ctypes.byref(w), 0x3000, zq.F32, None) == zq.ERR_UNSUPPORTED
        assert gemm(L, w) == zq.ERR_UNSUPPORTED


def problems(entries):
    """zq_problem array from (weight, m-independent fields, phase) entries,
    with bogus 256-byte aligned host addresses (never touched)"""
    arr = (zq._Problem * len(entries))()
    for i, (w, xdt, phase) in enumerate(entries):
        arr[i] = zq._Problem(w, 0x100000 + 0x1000 * i, xdt, w.k, 0x200000 + 0x1000 * i, zq.F32, w.n, phase)
    return arr


PLAN_CASES = [
    # m, entries, status, detail
    (0, [(dict(), zq.F16, 0)], zq.ERR_UNSUPPORTED, "m >= 1"),
    # prefill plans (m > 64, symmetric codes): one phase, one x dtype
    (128, [(dict(group=0), zq.BF16, 0), (dict(group=0), zq.BF16, 1)], zq.ERR_UNSUPPORTED, "one phase"),
    (128, [(dict(group=0), zq.BF16, 0), (dict(group=0), zq.F16, 0)], zq.ERR_UNSUPPORTED, "one activation type"),
    (128, [(dict(group=0, k=200), zq.BF16, 0)], zq.ERR_UNSUPPORTED, "multiple of 64"),
    # mid-batch plans with several phases (32 < m <= 64): INT4 with k a
    # multiple of 512 only (one phase would take the prefill tiles)
    (48, [(dict(bits=8), zq.F16, 0), (dict(bits=8), zq.F16, 1)], zq.ERR_UNSUPPORTED, "INT4"),
    (60, [(dict(bits=4, k=384), zq.BF16, 0), (dict(bits=4, k=384), zq.BF16, 1)], zq.ERR_UNSUPPORTED,
     "multiple of 512"),
    (40, [(dict(bits=2), zq.BF16, 0), (dict(bits=2), zq.BF16, 1)], zq.ERR_UNSUPPORTED, "INT4"),
]


@pytest.mark.parametrize("m,entries,status,detail", PLAN_CASES)
def test_plan_validation_without_device(L, m, entries, status, detail):
    arr = problems([(W(**kw, n=64) if "k" in kw else W(**kw, n=64, k=512), xdt, ph) for kw, xdt, ph in entries])
    h = ctypes.c_void_p()
    assert L.zq_plan_create(arr, len(entries), m, ctypes.byref(h)) == status
    assert detail in L.zq_last_error().decode()
    assert not h.value
