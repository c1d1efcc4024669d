"""Asymmetric weights (unsigned codes, fp16 scale and zero point per 128-group,
the .zse format's quantizer) through the C-ABI, against the fp64 oracle:
packing and unpacking bit-exact, products within the tolerance, integer cases
bit-exact, plans mixing symmetric and asymmetric products."""
import numpy as np
import pytest
import torch

from oracle import oracle as O
from weight_quantized_amd import synth

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
zq = None


@pytest.fixture(scope="module", autouse=True)
def _lib():
    global zq
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from weight_quantized_amd import zq as _zq
    _zq.lib()
    zq = _zq


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def host_u16(t):
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def x_dev(x, xdt):
    if xdt == "bf16":
        return torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).to(DEV)
    return torch.from_numpy(x).to(DEV)


def x64(x, xdt):
    if xdt == "bf16":
        return torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    return x.astype(np.float64)


def asym_weight(bits, n, k, seed):
    """random unsigned codes, scales |N|*0.01+1e-3, zeros N*0.01 (fp16)"""
    g = synth.rng(seed)
    q = g.integers(0, 1 << bits, size=(n, k)).astype(np.uint8)
    s = synth.scales_abs_normal(g, n * (k // 128))
    z = np.array([O.f64_to_f16(v) for v in g.standard_normal(n * (k // 128)) * 0.01], dtype=np.uint16)
    p = O.pack_u(q, bits)
    W = zq.ZqWeight(bits, 128, n, k, dev(p.reshape(-1)), dev(s.view(np.float16)), dev(z.view(np.float16)))
    return q, s, z, p, W


def check(y, yref, x, xdt, wdeq):
    xn = np.sqrt((x64(x, xdt) ** 2).sum(1))[:, None]
    tol = 2e-3 * xn * np.abs(wdeq).max(1)[None, :] + 1e-3 * np.abs(yref)
    bad = np.argwhere(np.abs(y - yref) > tol)
    assert bad.size == 0, f"{len(bad)} outputs out of tolerance, first {bad[:3].tolist()}"


@pytest.mark.parametrize("wdt", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("bits", [2, 4])
def test_pack_asym_float_weights_bit_exact(wdt, bits):
    g = synth.rng(bits * 10 + len(wdt))
    n, k = 70, 512
    w = (g.standard_normal((n, k)) * np.linspace(0.01, 3, n)[:, None] + 0.3).astype(np.float32)
    w[5, 128:256] = 0.25  # a constant group: scale 0
    if wdt == "f32":
        wt, wh = torch.from_numpy(w), w
    elif wdt == "f16":
        wh = w.astype(np.float16)
        wt = torch.from_numpy(wh)
    else:
        wh = synth.f32_to_bf16_bits(w)
        wt = torch.from_numpy(wh.view(np.int16)).view(torch.bfloat16)
    W = zq.pack_asym(wt.to(DEV), bits)
    torch.cuda.synchronize()
    s, z = O.compute_scales_zeros(wh, wdt, bits)
    q = O.quantize_asym(wh, wdt, bits, s, z)
    assert np.array_equal(host_u16(W.scales), s)
    assert np.array_equal(host_u16(W.zeros), z)
    assert np.array_equal(W.packed.cpu().numpy().reshape(n, -1), O.pack_u(q, bits))


@pytest.mark.parametrize("bits", [2, 4])
def test_pack_asym_codes_and_unpack_bit_exact(bits):
    q, s, z, p, W = asym_weight(bits, 33, 384, seed=7 + bits)
    codes = dev(q.astype(np.int8))
    W2 = zq.pack_asym(codes, bits, scales=W.scales, zeros=W.zeros)
    torch.cuda.synchronize()
    assert np.array_equal(W2.packed.cpu().numpy().reshape(33, -1), p)
    assert np.array_equal(zq.unpack(W, torch.int8).cpu().numpy().astype(np.uint8), q)
    ref = O.dequant_asym(q, s, z)
    assert np.array_equal(zq.unpack(W, torch.float32).cpu().numpy(), ref.astype(np.float32))
    h = zq.unpack(W, torch.float16)
    assert np.array_equal(host_u16(h), np.vectorize(O.f64_to_f16)(ref).astype(np.uint16))
    b = zq.unpack(W, torch.bfloat16)
    assert np.array_equal(host_u16(b), np.vectorize(O.f64_to_bf16)(ref).astype(np.uint16))
    bad = q.astype(np.int8).copy()
    bad[3, 7] = 1 << bits
    with pytest.raises(zq.ZqError) as e:
        zq.pack_asym(dev(bad), bits, scales=W.scales, zeros=W.zeros)
    assert e.value.status == zq.ERR_RANGE


@pytest.mark.parametrize("xdt", ["f16", "bf16"])
@pytest.mark.parametrize("bits", [2, 4])
@pytest.mark.parametrize("m", [1, 2, 3, 4, 5, 16])
def test_gemm_asym_matches_oracle(xdt, bits, m):
    # k = 512 / 3584 take the stream kernel for m <= 4; k = 384 (rows of 192
    # or 96 bytes) and m > 4 take the general kernel
    for n, k in [(300, 512), (70, 384), (257, 3584)]:
        seed = 1000 * bits + 100 * m + k % 97 + (xdt == "bf16")
        q, s, z, p, W = asym_weight(bits, n, k, seed)
        x = synth.normal(synth.rng(seed + 1), (m, k), xdt)
        Y = zq.gemm(W, x_dev(x, xdt))
        torch.cuda.synchronize()
        yref = O.gemm_asym(p, bits, s, z, n, k, x, xdt)
        check(Y.double().cpu().numpy(), yref, x, xdt, O.dequant_asym(q, s, z))


@pytest.mark.parametrize("xdt", ["f16", "bf16"])
@pytest.mark.parametrize("m", [1, 3, 8, 20, 40])
def test_gemm_asym_integer_inputs_bit_exact(xdt, m):
    n, k, bits = 90, 3584, 4
    g = synth.rng(500 + m)
    q = g.integers(0, 16, size=(n, k)).astype(np.uint8)
    s = np.where(g.random(n * k // 128) < 0.5, 0x3800, 0x3C00).astype(np.uint16)
    z = np.array([O.f64_to_f16(v) for v in g.integers(-8, 8, n * k // 128)], dtype=np.uint16)
    p = O.pack_u(q, bits)
    W = zq.ZqWeight(bits, 128, n, k, dev(p.reshape(-1)), dev(s.view(np.float16)), dev(z.view(np.float16)))
    v = g.integers(-4, 5, size=(m, k)).astype(np.float32)
    x = v.astype(np.float16) if xdt == "f16" else synth.f32_to_bf16_bits(v)
    Y = zq.gemm(W, x_dev(x, xdt))
    torch.cuda.synchronize()
    assert np.array_equal(Y.double().cpu().numpy(), O.gemm_asym(p, bits, s, z, n, k, x, xdt))


@pytest.mark.parametrize("m", [1, 2])
def test_plan_mixing_symmetric_and_asymmetric(m):
    probs, refs = [], []
    for i, (kind, bits, n, k, ph) in enumerate([("a", 4, 512, 1024, 0), ("s", 4, 300, 1024, 0),
                                                  ("a", 2, 640, 2048, 1), ("a", 4, 3584, 3584, 2)]):
        if kind == "a":
            q, s, z, p, W = asym_weight(bits, n, k, 60 + i)
        else:
            g = synth.rng(60 + i)
            q = synth.codes_uniform(g, n, k, bits)
            s = synth.scales_abs_normal(g, n * k // 128)
            z, p = None, O.pack(q, bits)
            W = zq.ZqWeight(bits, 128, n, k, dev(p.reshape(-1)), dev(s.view(np.float16)))
        x = synth.normal(synth.rng(70 + i), (m, k), "f16")
        Y = torch.full((m, n), float("nan"), device=DEV)
        probs.append((W, x_dev(x, "f16"), Y, ph))
        refs.append((kind, q, s, z, p, x, bits, n, k))
    plan = zq.Plan(probs)
    for _ in range(2):
        plan.run()
        torch.cuda.synchronize()
    plan.check()
    for (W, X, Y, _), (kind, q, s, z, p, x, bits, n, k) in zip(probs, refs):
        if kind == "a":
            yref, wdeq = O.gemm_asym(p, bits, s, z, n, k, x, "f16"), O.dequant_asym(q, s, z)
            if m == 1 or bits != 4:  # single calls of INT4 at m >= 2 take the MFMA kernel
                assert torch.equal(zq.gemm(W, X), Y)
        else:
            yref, wdeq = O.gemm(p, bits, s, 128, n, k, x, "f16"), O.dequant(q, 128, s)
        check(Y.double().cpu().numpy(), yref, x, "f16", wdeq)


@pytest.mark.parametrize("xdt", ["f16", "bf16"])
@pytest.mark.parametrize("m", [2, 8, 16, 17, 32, 33, 48, 100])
def test_gemm_asym_batched_mfma_matches_oracle(xdt, m):
    # INT4 with k a multiple of 512 at m >= 2: the MFMA batched-decode kernel
    # (in 32-row chunks past 32), zero points included per group
    for n, k in [(300, 512), (257, 1536)]:
        seed = 3000 + 10 * m + k % 89 + (xdt == "bf16")
        q, s, z, p, W = asym_weight(4, n, k, seed)
        x = synth.normal(synth.rng(seed + 1), (m, k), xdt)
        Y = zq.gemm(W, x_dev(x, xdt))
        torch.cuda.synchronize()
        check(Y.double().cpu().numpy(), O.gemm_asym(p, 4, s, z, n, k, x, xdt), x, xdt, O.dequant_asym(q, s, z))


@pytest.mark.parametrize("m", [8, 24, 40])
def test_plan_asym_batched_matches_oracle_and_single_calls(m):
    # an MFMA plan mixing asymmetric and symmetric INT4 products
    probs, refs = [], []
    for i, (kind, n, k) in enumerate([("a", 512, 1024), ("s", 300, 1024), ("a", 1000, 1536)]):
        if kind == "a":
            q, s, z, p, W = asym_weight(4, n, k, 90 + i)
        else:
            g = synth.rng(90 + i)
            q = synth.codes_uniform(g, n, k, 4)
            s = synth.scales_abs_normal(g, n * k // 128)
            z, p = None, O.pack(q, 4)
            W = zq.ZqWeight(4, 128, n, k, dev(p.reshape(-1)), dev(s.view(np.float16)))
        x = synth.normal(synth.rng(95 + i), (m, k), "bf16")
        Y = torch.full((m, n), float("nan"), device=DEV)
        probs.append((W, x_dev(x, "bf16"), Y, 0))
        refs.append((kind, q, s, z, p, x, n, k))
    plan = zq.Plan(probs)
    for _ in range(2):
        plan.run()
        torch.cuda.synchronize()
    plan.check()
    for (W, X, Y, _), (kind, q, s, z, p, x, n, k) in zip(probs, refs):
        if kind == "a":
            yref, wdeq = O.gemm_asym(p, 4, s, z, n, k, x, "bf16"), O.dequant_asym(q, s, z)
        else:
            yref, wdeq = O.gemm(p, 4, s, 128, n, k, x, "bf16"), O.dequant(q, 128, s)
        check(Y.double().cpu().numpy(), yref, x, "bf16", wdeq)
        if m <= 32:
            assert torch.equal(zq.gemm(W, X), Y)  # same kernel, same per-row arithmetic
