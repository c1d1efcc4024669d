"""Pins of the fp64 CPU oracle against things other than itself.

Each test pins one oracle function to library conversions (numpy / torch),
exhaustive round trips, closed forms, exact rational brute force, or the
hand-worked examples in tests/golden/hand_examples.txt. A plausible slip in
the oracle (a dropped term, a wrong sign or index, a swapped nibble, a
transposed operand, a wrong rounding) fails at least one of them.
"""
import itertools
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import oracle as O
from weight_quantized_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_examples.txt")


# --------------------------------------------------------------------------
# fp16 / bf16 conversions: library routines as the pin


def test_f16_decode_all_patterns_match_numpy():
    pats = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = pats.view(np.float16).astype(np.float64)
    got = np.array([O.f16_to_f64(int(p)) for p in pats])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))


def _f16_probe_values():
    finite = np.arange(0, 0x7C00, dtype=np.uint32).astype(np.uint16).view(np.float16).astype(np.float64)
    lo, hi = finite[:-1], finite[1:]
    mid = (lo + hi) / 2                       # exact ties
    g = synth.rng(7)
    vals = [finite, mid, np.nextafter(mid, 0), np.nextafter(mid, np.inf),
            np.exp(g.uniform(-40, 12, 20000)), [65504.0, 65519.99, 65520.0, 65536.0, 1e10, 2.0 ** -25,
                                                 2.0 ** -26, 3 * 2.0 ** -26, 1e-30, 0.0]]
    v = np.concatenate([np.asarray(a, dtype=np.float64) for a in vals])
    return np.concatenate([v, -v])


def test_f16_encode_matches_numpy_rne():
    v = _f16_probe_values()
    ref = v.astype(np.float16).view(np.uint16)
    got = np.array([O.f64_to_f16(float(a)) for a in v], dtype=np.uint16)
    bad = np.nonzero(got != ref)[0]
    assert bad.size == 0, [(v[i], hex(got[i]), hex(ref[i])) for i in bad[:5]]


def test_bf16_decode_all_patterns_match_torch():
    pats = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = torch.from_numpy(pats.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    got = np.array([O.bf16_to_f64(int(p)) for p in pats])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])


def test_bf16_encode_matches_torch_rne_on_float32_inputs():
    finite = torch.from_numpy(np.arange(0, 0x7F80, dtype=np.int32).astype(np.int16)).view(torch.bfloat16)
    f = finite.to(torch.float32).numpy().astype(np.float64)
    mid = (f[:-1] + f[1:]) / 2                # ties; exact in float32 (9 significant bits)
    g = synth.rng(8)
    rnd = g.standard_normal(20000).astype(np.float32).astype(np.float64) * np.exp(g.uniform(-60, 60, 20000))
    v = np.concatenate([f, mid, rnd]).astype(np.float32)
    v = v[np.isfinite(v)]
    v = np.concatenate([v, -v])
    ref = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = np.array([O.f64_to_bf16(float(a)) for a in v], dtype=np.uint16)
    bad = np.nonzero(got != ref)[0]
    assert bad.size == 0, [(v[i], hex(got[i]), hex(ref[i])) for i in bad[:5]]


def test_scale_closed_form_fp16_of_0_02():
    assert O.f64_to_f16(0.02) == 0x251F
    assert O.f16_to_f64(0x251F) == 0.0200042724609375


# --------------------------------------------------------------------------
# packing: exhaustive round trips and hand examples


@pytest.mark.parametrize("bits", [2, 4, 8])
def test_every_byte_round_trips_unpack_then_pack(bits):
    per = 8 // bits
    allbytes = np.arange(256, dtype=np.uint8).reshape(256, 1)
    codes = O.unpack(allbytes, 256, per, bits)
    lo, hi = -(1 << (bits - 1)), (1 << (bits - 1)) - 1
    assert codes.min() >= lo and codes.max() <= hi
    assert np.array_equal(O.pack(codes, bits), allbytes)


@pytest.mark.parametrize("bits", [2, 4, 8])
def test_every_code_tuple_round_trips_pack_then_unpack(bits):
    per = 8 // bits
    rng_ = range(-(1 << (bits - 1)), 1 << (bits - 1))
    tuples = np.array(list(itertools.product(rng_, repeat=per)), dtype=np.int8)
    assert tuples.shape[0] == 256
    packed = O.pack(tuples, bits)
    assert np.array_equal(np.sort(packed.ravel()), np.arange(256, dtype=np.uint8))
    assert np.array_equal(O.unpack(packed, 256, per, bits), tuples)


def _golden(kind):
    out = []
    with open(GOLDEN) as fh:
        for line in fh:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            head, *rest = line.split()
            if head != kind:
                continue
            out.append(dict(tok.split("=", 1) for tok in rest))
    return out


def _ints(s):
    return [int(t) for t in s.split(",")]


def _floats(s):
    return [float(t) for t in s.split(",")]


def test_golden_pack_examples():
    cases = _golden("pack")
    assert len(cases) == 8
    for c in cases:
        bits = int(c["bits"])
        codes = np.array([_ints(c["codes"])], dtype=np.int8)
        want = np.array([[int(b, 16) for b in c["bytes"].split(",")]], dtype=np.uint8)
        assert np.array_equal(O.pack(codes, bits), want), c
        assert np.array_equal(O.unpack(want, 1, codes.shape[1], bits), codes), c


def test_golden_gemv_examples():
    cases = _golden("gemv")
    assert len(cases) == 3
    for c in cases:
        bits, n, k = int(c["bits"]), int(c["n"]), int(c["k"])
        codes = np.array(_ints(c["codes"]), dtype=np.int8).reshape(n, k)
        scales = np.array([int(c["scales"], 16)], dtype=np.uint16)
        x = np.array(_floats(c["x"]), dtype=np.float16)
        y = O.gemm(O.pack(codes, bits), bits, scales, 0, n, k, x, "f16")
        assert np.array_equal(y, np.array(_floats(c["y"]))), (c, y)


def test_golden_group_example():
    (c,) = _golden("gemv_groups")
    k = int(c["k"])
    codes = np.concatenate([np.full(128, int(c["code0"])), np.full(128, int(c["code1"]))]).astype(np.int8)
    scales = np.array([int(s, 16) for s in c["scales"].split(",")], dtype=np.uint16)
    x = np.full(k, float(c["x"]), dtype=np.float16)
    y = O.gemm(O.pack(codes.reshape(1, k), 4), 4, scales, 128, 1, k, x, "f16")
    assert y[0] == float(c["y"])


def test_golden_f16_example():
    (c,) = _golden("f16")
    assert O.f64_to_f16(float(c["value"])) == int(c["bits"], 16)
    assert O.f16_to_f64(int(c["bits"], 16)) == float(c["exact"])


# --------------------------------------------------------------------------
# quantizer: invariants that the definition fixes


def _weights(dtype, n, k, seed, scale_spread=True):
    g = synth.rng(seed)
    w = g.standard_normal((n, k)).astype(np.float32)
    if scale_spread:  # rows of very different magnitude, some exact zeros
        w *= np.exp(g.uniform(-6, 6, (n, 1))).astype(np.float32)
        w[0, :] = 0.0
    if dtype == "f32":
        return w
    if dtype == "f16":
        return np.clip(w, -60000, 60000).astype(np.float16)
    return synth.f32_to_bf16_bits(w)


def _as_f64(w, dtype):
    if dtype == "bf16":
        return torch.from_numpy(w.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    return w.astype(np.float64)


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("bits", [2, 4, 8])
@pytest.mark.parametrize("group", [0, 128])
def test_quantize_error_at_most_half_scale_and_no_clip(dtype, bits, group):
    n, k = 6, 256
    w = _weights(dtype, n, k, seed=bits * 10 + group)
    s = O.compute_scales(w, dtype, bits, group)
    q = O.quantize(w, dtype, bits, group, s)
    qmax = (1 << (bits - 1)) - 1
    assert q.min() >= -qmax and q.max() <= qmax          # symmetric grid: -2^(b-1) never produced
    wf = _as_f64(w, dtype)
    sf = np.array([O.f16_to_f64(int(b)) for b in s])
    sidx = np.zeros((n, k), dtype=np.int64) if group == 0 else (
        np.arange(n)[:, None] * (k // group) + np.arange(k)[None, :] // group)
    S = sf[sidx]
    for i, j in itertools.product(range(n), range(0, k, 3)):
        err = abs(Fraction(float(wf[i, j])) - int(q[i, j]) * Fraction(float(S[i, j])))
        assert err <= Fraction(float(S[i, j])) / 2, (i, j)
    # scale rule: s16 * qmax >= absmax, and one fp16 step down would clip
    units = [wf.ravel()] if group == 0 else [wf[i, g * 128:(g + 1) * 128] for i in range(n) for g in range(k // 128)]
    for u, sb in zip(units, s):
        a = float(np.max(np.abs(u)))
        if a == 0:
            assert sb == 0
            continue
        assert O.f16_to_f64(int(sb)) * qmax >= a
        rne = O.f64_to_f16(a / qmax)
        assert int(sb) in (rne, rne + 1)
        if int(sb) == rne + 1:
            assert O.f16_to_f64(rne) * qmax < a


@pytest.mark.parametrize("bits", [2, 4, 8])
def test_quantize_is_idempotent_on_dequantized_weights(bits):
    n, k = 5, 384
    w = _weights("f32", n, k, seed=bits)
    s = O.compute_scales(w, "f32", bits, 128)
    q = O.quantize(w, "f32", bits, 128, s)
    wdeq = O.dequant(q, 128, s).astype(np.float32)  # q*s is exact in float32 (<= 19 bits)
    assert np.array_equal(wdeq.astype(np.float64), O.dequant(q, 128, s))
    assert np.array_equal(O.quantize(wdeq, "f32", bits, 128, s), q)


def test_quantize_ties_round_half_to_even_and_caller_scale_clips():
    one = np.array([0x3C00], dtype=np.uint16)  # 1.0
    w = np.array([[2.5, 3.5, -2.5, -3.5, 0.5, -0.5, 1.5, 100.0, -100.0, 6.5, -7.5, 0.0]], dtype=np.float32)
    q = O.quantize(w, "f32", 4, 0, one)
    assert q.tolist() == [[2, 4, -2, -4, 0, 0, 2, 7, -8, 6, -8, 0]]


def test_quantize_zero_unit_gives_zero_scale_and_codes():
    w = np.zeros((2, 128), dtype=np.float32)
    w[1, 5] = 3.0
    s = O.compute_scales(w, "f32", 4, 128)
    assert s[0] == 0 and s[1] != 0
    q = O.quantize(w, "f32", 4, 128, s)
    assert not q[0].any() and q[1, 5] == 7


def test_range_and_shape_errors():
    w = np.ones((1, 128), dtype=np.float32)
    w[0, 3] = np.inf
    with pytest.raises(O.OracleError) as e:
        O.compute_scales(w, "f32", 4, 128)
    assert e.value.status == O.ERR_RANGE
    big = np.full((1, 128), 7 * 65504 * 1.5, dtype=np.float32)   # scale would exceed fp16
    with pytest.raises(O.OracleError) as e:
        O.compute_scales(big, "f32", 4, 128)
    assert e.value.status == O.ERR_RANGE
    with pytest.raises(O.OracleError) as e:
        O.pack(np.array([[8, 0]], dtype=np.int8), 4)
    assert e.value.status == O.ERR_RANGE
    with pytest.raises(O.OracleError) as e:
        O.compute_scales(np.ones((1, 64), dtype=np.float32), "f32", 4, 128)
    assert e.value.status == O.ERR_UNSUPPORTED
    with pytest.raises(O.OracleError) as e:
        O.compute_scales(np.ones((1, 128), dtype=np.float32), "f32", 3, 0)
    assert e.value.status == O.ERR_UNSUPPORTED
    with pytest.raises(O.OracleError) as e:
        O.compute_scales(np.ones((1, 128), dtype=np.float32), "f32", 4, 64)
    assert e.value.status == O.ERR_UNSUPPORTED


# --------------------------------------------------------------------------
# dequant and the linear layer


def test_dequant_is_exact_product():
    g = synth.rng(3)
    q = synth.codes_uniform(g, 4, 256, 4)
    s = synth.scales_abs_normal(g, 8)
    d = O.dequant(q, 128, s)
    for i, j in itertools.product(range(4), range(256)):
        assert Fraction(float(d[i, j])) == int(q[i, j]) * Fraction(O.f16_to_f64(int(s[i * 2 + j // 128])))


@pytest.mark.parametrize("bits,group", [(4, 0), (4, 128), (2, 128), (8, 0)])
def test_one_hot_recovers_one_dequantized_column(bits, group):
    n, k = 7, 256
    g = synth.rng(bits + group)
    q = synth.codes_uniform(g, n, k, bits)
    s = synth.scales_abs_normal(g, O.num_scales(group, n, k))
    p = O.pack(q, bits)
    wdeq = O.dequant(q, group, s)
    X = np.eye(k, dtype=np.float16)           # every one-hot vector at once
    y = O.gemm(p, bits, s, group, n, k, X, "f16")
    assert np.array_equal(y, wdeq.T)          # y[m=k][n] = q[n][k] * s exactly


def _brute(q, sf, group, x):
    """exact rational y[m][n] = sum_k x[m][k] * q[n][k] * s(n,k)"""
    n, k = q.shape
    out = []
    for xm in x:
        row = []
        for i in range(n):
            acc = Fraction(0)
            for j in range(k):
                s = sf[0] if group == 0 else sf[i * (k // group) + j // group]
                acc += Fraction(float(xm[j])) * int(q[i, j]) * Fraction(s)
            row.append(acc)
        out.append(row)
    return out


@pytest.mark.parametrize("n,k", [(4, 8), (8, 16), (16, 32), (4, 256)])
@pytest.mark.parametrize("bits", [2, 4, 8])
def test_tiny_gemm_matches_exact_brute_force(n, k, bits):
    group = 128 if k % 128 == 0 else 0
    g = synth.rng(n * k + bits)
    q = synth.codes_uniform(g, n, k, bits)
    s = synth.scales_abs_normal(g, O.num_scales(group, n, k))
    x = synth.normal(g, (3, k), "f16")
    y = O.gemm(O.pack(q, bits), bits, s, group, n, k, x, "f16")
    sf = [O.f16_to_f64(int(b)) for b in s]
    exact = _brute(q, sf, group, x)
    for mi in range(3):
        for i in range(n):
            bound = sum(abs(Fraction(float(x[mi, j])) * int(q[i, j])) for j in range(k)) * Fraction(max(sf))
            assert abs(Fraction(float(y[mi, i])) - exact[mi][i]) <= bound * Fraction(2) ** -48


@pytest.mark.parametrize("xdt", ["f16", "bf16", "f32"])
def test_gemm_matches_textbook_dense_matmul(xdt):
    n, k, m = 33, 384, 5
    g = synth.rng(11)
    q = synth.codes_uniform(g, n, k, 4)
    s = synth.scales_abs_normal(g, n * k // 128)
    x = synth.normal(g, (m, k), xdt)
    y = O.gemm(O.pack(q, 4), 4, s, 128, n, k, x, xdt)
    X = _as_f64(x, xdt)
    W = O.dequant(q, 128, s)
    ref = X @ W.T                               # library matmul of the dequantized matrix
    bound = np.abs(X) @ np.abs(W).T
    assert np.all(np.abs(y - ref) <= 1e-13 * bound + 1e-300)
    # and not the transposed or unscaled product
    assert not np.allclose(y, X @ (q.astype(np.float64)).T)


def test_same_codes_under_every_bit_width_give_identical_outputs():
    n, k = 9, 256
    g = synth.rng(5)
    q = g.integers(-2, 2, size=(n, k), dtype=np.int8)   # representable in 2, 4 and 8 bits
    s = synth.scales_abs_normal(g, n * 2)
    x = synth.normal(g, (2, k), "bf16")
    ys = [O.gemm(O.pack(q, b), b, s, 128, n, k, x, "bf16") for b in (2, 4, 8)]
    assert np.array_equal(ys[0], ys[1]) and np.array_equal(ys[1], ys[2])


def test_per_tensor_equals_group_when_all_group_scales_equal():
    n, k = 6, 512
    g = synth.rng(9)
    q = synth.codes_uniform(g, n, k, 4)
    s1 = synth.scales_abs_normal(g, 1)
    sg = np.full(n * k // 128, s1[0], dtype=np.uint16)
    x = synth.normal(g, (2, k), "f16")
    p = O.pack(q, 4)
    assert np.array_equal(O.gemm(p, 4, s1, 0, n, k, x, "f16"), O.gemm(p, 4, sg, 128, n, k, x, "f16"))


def test_gemm_rows_matches_full_gemm():
    n, k = 20, 256
    g = synth.rng(12)
    q = synth.codes_uniform(g, n, k, 4)
    s = synth.scales_abs_normal(g, n * 2)
    x = synth.normal(g, (3, k), "f16")
    p = O.pack(q, 4)
    full = O.gemm(p, 4, s, 128, n, k, x, "f16")
    rows = np.array([0, 7, 19])
    assert np.array_equal(O.gemm_rows(p, 4, s, 128, n, k, x, "f16", rows), full[:, rows])


# ---------------------------------------------------------------------------
# asymmetric variant (unsigned codes, fp16 scale and zero per 128-group), the
# quantizer of the ZSE wiki's section on the .zse model format


def test_asym_closed_form_integer_grid():
    """weights 0..15 in every group: scale (15 - 0) / 15 = 1, zero 0, codes = weights"""
    w = np.tile(np.arange(16, dtype=np.float32), 16).reshape(2, 128)
    s, z = O.compute_scales_zeros(w, "f32", 4)
    assert np.all(s == 0x3C00) and np.all(z == 0)
    q = O.quantize_asym(w, "f32", 4, s, z)
    assert np.array_equal(q, w.astype(np.uint8))
    assert np.array_equal(O.dequant_asym(q, s, z), w.astype(np.float64))


def test_asym_worked_scale_and_zero_bits():
    """min -1, max 2: scale 3/15 = 0.2 -> fp16 0x3266 (0.199951171875), zero -1 -> 0xBC00"""
    w = (-1.0 + 3.0 * np.arange(128) / 127).astype(np.float32).reshape(1, 128)
    w[0, 0], w[0, -1] = -1.0, 2.0
    s, z = O.compute_scales_zeros(w, "f32", 4)
    assert s[0] == 0x3266 and O.f16_to_f64(int(s[0])) == 0.199951171875
    assert z[0] == 0xBC00
    # INT2: scale 3/3 = 1
    s2, z2 = O.compute_scales_zeros(w, "f32", 2)
    assert s2[0] == 0x3C00 and z2[0] == 0xBC00


@pytest.mark.parametrize("bits", [2, 4])
def test_asym_codes_are_nearest_grid_points(bits):
    """brute force: each code minimises |w - (z + q s)| over q in [0, 2^b - 1]; ties to even q"""
    g = synth.rng(71 + bits)
    w = (g.standard_normal((6, 256)) * np.array([[1], [0.01], [100], [3], [1e-3], [7]])).astype(np.float32)
    s, z = O.compute_scales_zeros(w, "f32", bits)
    q = O.quantize_asym(w, "f32", bits, s, z)
    qmax = (1 << bits) - 1
    grid = np.arange(qmax + 1, dtype=np.float64)
    for r in range(w.shape[0]):
        for c in range(w.shape[1]):
            si = r * 2 + c // 128
            sv, zv = O.f16_to_f64(int(s[si])), O.f16_to_f64(int(z[si]))
            d = np.abs(float(w[r, c]) - (zv + grid * sv))
            best = np.flatnonzero(d == d.min())
            expect = best[0] if len(best) == 1 else [b for b in best if b % 2 == 0][0]
            assert q[r, c] == expect, (r, c)


def test_asym_error_bound_and_constant_group():
    g = synth.rng(5)
    w = g.standard_normal((8, 384)).astype(np.float32)
    w[3, 128:256] = 0.7  # a constant group: scale 0, codes 0, w_deq = fp16(0.7)
    s, z = O.compute_scales_zeros(w, "f32", 4)
    q = O.quantize_asym(w, "f32", 4, s, z)
    wd = O.dequant_asym(q, s, z)
    sv = np.array([O.f16_to_f64(int(v)) for v in s]).reshape(8, 3).repeat(128, axis=1)
    assert s[3 * 3 + 1] == 0 and np.all(q[3, 128:256] == 0)
    assert np.all(wd[3, 128:256] == O.f16_to_f64(O.f64_to_f16(0.7)))
    mask = sv > 0
    assert np.all(np.abs(w.astype(np.float64) - wd)[mask] <= sv[mask] / 2 * (1 + 1e-9))


def test_asym_pack_u_round_trip_and_hand_examples():
    for bits in (2, 4):
        per = 8 // bits
        b = np.arange(256, dtype=np.uint8).reshape(1, 256)
        q = O.unpack_u(b, 1, 256 * per, bits)
        assert q.max() == (1 << bits) - 1
        assert np.array_equal(O.pack_u(q, bits), b)
    assert O.pack_u(np.array([[1, 15]], dtype=np.uint8), 4)[0, 0] == 0xF1
    assert O.pack_u(np.array([[1, 2, 0, 3]], dtype=np.uint8), 2)[0, 0] == 0xC9
    with pytest.raises(O.OracleError):
        O.pack_u(np.array([[16, 0]], dtype=np.uint8), 4)


@pytest.mark.parametrize("bits", [2, 4])
@pytest.mark.parametrize("xdt", ["f16", "bf16"])
def test_asym_gemm_equals_dense_matmul(bits, xdt):
    g = synth.rng(90 + bits)
    n, k, m = 9, 384, 3
    w = g.standard_normal((n, k)).astype(np.float32)
    s, z = O.compute_scales_zeros(w, "f32", bits)
    q = O.quantize_asym(w, "f32", bits, s, z)
    p = O.pack_u(q, bits)
    x = synth.normal(g, (m, k), xdt)
    x64 = torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).double().numpy() if xdt == "bf16" \
        else x.astype(np.float64)
    ref = x64 @ O.dequant_asym(O.unpack_u(p, n, k, bits), s, z).T
    np.testing.assert_allclose(O.gemm_asym(p, bits, s, z, n, k, x, xdt), ref, rtol=1e-12, atol=1e-12)


def test_asym_gemm_reduces_to_symmetric_plus_zero_term():
    """q s + z = (q - 8) s + (z + 8 s): the asymmetric product is the pinned
    symmetric one on shifted codes plus one term per group; exact on integers"""
    g = synth.rng(33)
    n, k, m, bits = 7, 256, 4, 4
    q = g.integers(0, 16, size=(n, k)).astype(np.uint8)
    s = np.where(g.random(n * 2) < 0.5, 0x3800, 0x3C00).astype(np.uint16)   # 0.5 or 1
    z = np.array([O.f64_to_f16(v) for v in g.integers(-6, 6, n * 2)], dtype=np.uint16)
    x = g.integers(-4, 5, size=(m, k)).astype(np.float16)
    y = O.gemm_asym(O.pack_u(q, bits), bits, s, z, n, k, x, "f16")
    ys = O.gemm(O.pack(q.astype(np.int16) - 8, bits), bits, s, 128, n, k, x, "f16")
    sv = np.array([O.f16_to_f64(int(v)) for v in s]).reshape(n, 2)
    zv = np.array([O.f16_to_f64(int(v)) for v in z]).reshape(n, 2)
    xg = x.astype(np.float64).reshape(m, 2, 128).sum(2)          # [m][group]
    assert np.array_equal(y, ys + xg @ (zv + 8 * sv).T)


def test_asym_range_errors():
    w = np.zeros((1, 128), dtype=np.float32)
    w[0, 5] = np.inf
    with pytest.raises(O.OracleError):
        O.compute_scales_zeros(w, "f32", 4)
    w = np.zeros((1, 128), dtype=np.float32)
    w[0, 0], w[0, 1] = -6e5, 6e5  # zero beyond fp16
    with pytest.raises(O.OracleError):
        O.compute_scales_zeros(w, "f32", 4)
    with pytest.raises(O.OracleError):
        O.compute_scales_zeros(np.zeros((1, 100), np.float32), "f32", 4)
