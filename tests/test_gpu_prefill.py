"""The prefill MFMA kernel (m > 64, one scale per tensor, k a multiple of 64)
against the fp64 oracle: ragged tiles, every code width, both activation
types, and bit-exact integer cases."""
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


def weight(bits, n, k, seed, codes=None, scale=None):
    g = synth.rng(seed)
    q = synth.codes_uniform(g, n, k, bits) if codes is None else codes
    s = synth.scales_abs_normal(g, 1) if scale is None else np.array([scale], dtype=np.uint16)
    p = O.pack(q, bits)
    W = zq.ZqWeight(bits, 0, n, k, torch.from_numpy(p.reshape(-1)).to(DEV),
                    torch.from_numpy(s.view(np.float16)).to(DEV))
    return q, s, p, W


def x_dev(x, xdt):
    if xdt == "bf16":
        return torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).to(DEV)
    return torch.from_numpy(x).to(DEV)


def x64(x, xdt):
    if xdt == "bf16":
        return torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    return x.astype(np.float64)


@pytest.mark.parametrize("xdt", ["f16", "bf16"])
@pytest.mark.parametrize("bits", [2, 4, 8])
@pytest.mark.parametrize("m,n,k", [(65, 100, 64), (256, 256, 192), (300, 600, 1024), (520, 260, 512)])
def test_prefill_matches_oracle(xdt, bits, m, n, k):
    seed = 13 * m + 7 * n + k + bits + (xdt == "bf16")
    q, s, p, W = weight(bits, n, k, seed)
    x = synth.normal(synth.rng(seed + 1), (m, k), xdt)
    Y = zq.gemm(W, x_dev(x, xdt))
    torch.cuda.synchronize()
    yref = O.gemm(p, bits, s, 0, n, k, x, xdt)
    xn = np.sqrt((x64(x, xdt) ** 2).sum(1))[:, None]
    tol = 2e-3 * xn * np.abs(O.dequant(q, 0, s)).max(1)[None, :] + 1e-3 * np.abs(yref)
    err = np.abs(Y.double().cpu().numpy() - yref)
    assert np.all(err <= tol), f"{np.argwhere(err > tol)[:3]}"


@pytest.mark.parametrize("xdt", ["f16", "bf16"])
@pytest.mark.parametrize("bits", [2, 4, 8])
def test_prefill_integer_inputs_bit_exact(xdt, bits):
    m, n, k = 300, 270, 1024
    g = synth.rng(40 + bits)
    q, s, p, W = weight(bits, n, k, 0, codes=synth.codes_uniform(g, n, k, bits), scale=0x3800)
    v = g.integers(-4, 5, size=(m, k)).astype(np.float32)
    x = v.astype(np.float16) if xdt == "f16" else synth.f32_to_bf16_bits(v)
    Y = zq.gemm(W, x_dev(x, xdt))
    torch.cuda.synchronize()
    assert np.array_equal(Y.double().cpu().numpy(), O.gemm(p, bits, s, 0, n, k, x, xdt))


def test_prefill_strided_rows_and_low_precision_out():
    m, n, k, ldx = 130, 300, 256, 320
    q, s, p, W = weight(4, n, k, 5)
    xf = synth.normal(synth.rng(6), (m, ldx), "bf16")
    X = x_dev(xf, "bf16")[:, :k]
    Y32 = zq.gemm(W, X)
    Yb = zq.gemm(W, X, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    x = np.ascontiguousarray(xf[:, :k])
    yref = O.gemm(p, 4, s, 0, n, k, x, "bf16")
    xn = np.sqrt((x64(x, "bf16") ** 2).sum(1))[:, None]
    tol = 2e-3 * xn * np.abs(O.dequant(q, 0, s)).max(1)[None, :] + 1e-3 * np.abs(yref)
    assert np.all(np.abs(Y32.double().cpu().numpy() - yref) <= tol)
    assert torch.equal(Yb, Y32.to(torch.bfloat16))


# ---------------------------------------------------------------------------
# prefill plans: the tiles of many products in one persistent launch per bit
# width, taken from a device counter


def plan_problems(m, shapes, xdt, seed):
    probs, refs = [], []
    for i, (bits, n, k) in enumerate(shapes):
        q, s, p, W = weight(bits, n, k, seed + 10 * i)
        x = synth.normal(synth.rng(seed + 10 * i + 1), (m, k), xdt)
        Y = torch.full((m, n), float("nan"), device=DEV)
        probs.append((W, x_dev(x, xdt), Y, 0))
        refs.append((q, s, p, x, bits, n, k))
    return probs, refs


@pytest.mark.parametrize("xdt", ["f16", "bf16"])
def test_prefill_plan_matches_single_calls_and_oracle(xdt):
    # mixed bit widths and k, ragged m and n tiles; three runs (the counters
    # must come back to zero after each)
    m = 300
    shapes = [(4, 600, 1024), (2, 256, 192), (8, 100, 512), (4, 513, 64), (2, 70, 1024), (8, 260, 256)]
    probs, refs = plan_problems(m, shapes, xdt, seed=700 + (xdt == "bf16"))
    plan = zq.Plan(probs)
    for _ in range(3):
        for _, _, Y, _ in probs:
            Y.fill_(float("nan"))
        plan.run()
        torch.cuda.synchronize()
        plan.check()
        for (W, X, Y, _), (q, s, p, x, bits, n, k) in zip(probs, refs):
            # the same tile code as the single-launch kernel: identical outputs
            assert torch.equal(zq.gemm(W, X), Y)
    for (W, X, Y, _), (q, s, p, x, bits, n, k) in zip(probs, refs):
        yref = O.gemm(p, bits, s, 0, n, k, x, xdt)
        xn = np.sqrt((x64(x, xdt) ** 2).sum(1))[:, None]
        tol = 2e-3 * xn * np.abs(O.dequant(q, 0, s)).max(1)[None, :] + 1e-3 * np.abs(yref)
        assert np.all(np.abs(Y.double().cpu().numpy() - yref) <= tol), f"bits={bits} n={n} k={k}"


def test_prefill_plan_more_tiles_than_workgroups_integer_exact():
    # INT4: 128 + 160 tiles, more than the 256 workgroups, so some take two;
    # integer activations and scale 1.0 make every output exact
    m = 512
    probs, refs = [], []
    g = synth.rng(901)
    for i, (bits, n, k) in enumerate([(4, 16384, 128), (4, 20480, 64), (8, 6144, 128), (2, 10240, 192)]):
        q = synth.codes_uniform(g, n, k, bits)
        _, s, p, W = weight(bits, n, k, 0, codes=q, scale=0x3C00)
        v = g.integers(-4, 5, size=(m, k)).astype(np.float32)
        x = synth.f32_to_bf16_bits(v)
        Y = torch.full((m, n), float("nan"), device=DEV)
        probs.append((W, x_dev(x, "bf16"), Y, 0))
        refs.append((p, s, x, bits, n, k))
    plan = zq.Plan(probs)
    for _ in range(2):
        plan.run()
        torch.cuda.synchronize()
    plan.check()
    for (W, X, Y, _), (p, s, x, bits, n, k) in zip(probs, refs):
        assert np.array_equal(Y.double().cpu().numpy(), O.gemm(p, bits, s, 0, n, k, x, "bf16")), f"bits={bits}"


def test_prefill_plan_validation():
    _, _, _, W = weight(4, 64, 256, seed=3)
    X = torch.zeros((128, 256), dtype=torch.bfloat16, device=DEV)
    Xh = torch.zeros((128, 256), dtype=torch.float16, device=DEV)
    Y = torch.empty((128, 64), device=DEV)
    with pytest.raises(zq.ZqError) as e:  # two phases
        zq.Plan([(W, X, Y, 0), (W, X, torch.empty((128, 64), device=DEV), 1)])
    assert e.value.status == zq.ERR_UNSUPPORTED
    with pytest.raises(zq.ZqError) as e:  # two activation types
        zq.Plan([(W, X, Y, 0), (W, Xh, torch.empty((128, 64), device=DEV), 0)])
    assert e.value.status == zq.ERR_UNSUPPORTED
    Wg = zq.ZqWeight(4, 128, 64, 256, W.packed, torch.ones(64 * 2, dtype=torch.float16, device=DEV))
    with pytest.raises(zq.ZqError) as e:  # group scales
        zq.Plan([(Wg, X, Y, 0)])
    assert e.value.status == zq.ERR_UNSUPPORTED
    X48 = torch.zeros((48, 256), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(zq.ZqError) as e:  # 32 < m <= 64
        zq.Plan([(W, X48, torch.empty((48, 64), device=DEV), 0)])
    assert e.value.status == zq.ERR_UNSUPPORTED
