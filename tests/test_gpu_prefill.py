"""The prefill MFMA kernel (m > 64, symmetric codes; one scale per tensor with
k a multiple of 64, or one per row and 128 k) against the fp64 oracle:
ragged tiles, every code width, both activation types, zero and negative
group scales, and bit-exact integer cases."""
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


def weight(bits, n, k, seed, codes=None, scale=None, group=0):
    """codes (uniform unless given) and fp16 scale patterns: |N(0,1)| * 0.01 +
    1e-3, or the given pattern(s)"""
    g = synth.rng(seed)
    q = synth.codes_uniform(g, n, k, bits) if codes is None else codes
    ns = 1 if group == 0 else n * (k // group)
    if scale is None:
        s = synth.scales_abs_normal(g, ns)
    else:
        s = np.broadcast_to(np.asarray(scale, dtype=np.uint16), (ns,)).copy()
    p = O.pack(q, bits)
    W = zq.ZqWeight(bits, group, n, k, torch.from_numpy(p.reshape(-1)).to(DEV),
                    torch.from_numpy(s.view(np.float16)).to(DEV))
    return q, s, p, W


def check(Y, yref, x, xdt, q, group, s, what=""):
    xn = np.sqrt((x64(x, xdt) ** 2).sum(1))[:, None]
    tol = 2e-3 * xn * np.abs(O.dequant(q, group, s)).max(1)[None, :] + 1e-3 * np.abs(yref)
    err = np.abs(Y - yref)
    assert np.all(err <= tol), f"{what}: {int((err > tol).sum())} out of tolerance, first {np.argwhere(err > tol)[:3]}"


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
    check(Y.double().cpu().numpy(), O.gemm(p, bits, s, 0, n, k, x, xdt), x, xdt, q, 0, s)


# group scales: m = 65..520 with ragged row and column tiles (128 x 256)
@pytest.mark.parametrize("xdt", ["f16", "bf16"])
@pytest.mark.parametrize("bits", [2, 4, 8])
@pytest.mark.parametrize("m,n,k", [(65, 100, 128), (128, 256, 256), (200, 600, 1024), (257, 300, 3584),
                                   (520, 260, 512)])
def test_prefill_group_matches_oracle(xdt, bits, m, n, k):
    seed = 17 * m + 5 * n + k + bits + (xdt == "bf16")
    q, s, p, W = weight(bits, n, k, seed, group=128)
    x = synth.normal(synth.rng(seed + 1), (m, k), xdt)
    Y = zq.gemm(W, x_dev(x, xdt))
    torch.cuda.synchronize()
    check(Y.double().cpu().numpy(), O.gemm(p, bits, s, 128, n, k, x, xdt), x, xdt, q, 128, s)


@pytest.mark.parametrize("xdt", ["f16", "bf16"])
@pytest.mark.parametrize("bits", [2, 4, 8])
def test_prefill_group_zero_and_negative_scales(xdt, bits):
    # whole groups with scale 0 (they add nothing; the accumulators keep the
    # previous group's units) and negative scales, also at a row's first and
    # last group
    m, n, k = 150, 300, 1280
    g = synth.rng(60 + bits)
    s = synth.scales_abs_normal(g, n * k // 128).reshape(n, k // 128)
    s[g.random(s.shape) < 0.15] = 0
    s[:, 0][g.random(n) < 0.3] = 0
    s[:, -1][g.random(n) < 0.3] = 0
    s[:7] = 0  # rows with no nonzero scale
    neg = g.random(s.shape) < 0.2
    s[neg] |= 0x8000
    q, s, p, W = weight(bits, n, k, 61 + bits, scale=s.reshape(-1), group=128)
    x = synth.normal(synth.rng(62 + bits), (m, k), xdt)
    Y = zq.gemm(W, x_dev(x, xdt))
    torch.cuda.synchronize()
    Yn = Y.double().cpu().numpy()
    check(Yn, O.gemm(p, bits, s, 128, n, k, x, xdt), x, xdt, q, 128, s)
    assert np.all(Yn[:, :7] == 0)


@pytest.mark.parametrize("xdt", ["f16", "bf16"])
@pytest.mark.parametrize("bits", [2, 4, 8])
@pytest.mark.parametrize("group", [0, 128])
def test_prefill_integer_inputs_bit_exact(xdt, bits, group):
    # integer activations; scale 0.5 per tensor, or 0.5 / 1 / 0 per group:
    # every partial sum is exact in fp32, and so is every change of units
    m, n, k = 300, 270, 1024
    g = synth.rng(40 + bits + group)
    scale = 0x3800 if group == 0 else g.choice(np.array([0x3800, 0x3C00, 0x0000], dtype=np.uint16),
                                                size=n * k // 128, p=[0.45, 0.45, 0.1])
    q, s, p, W = weight(bits, n, k, 0, codes=synth.codes_uniform(g, n, k, bits), scale=scale, group=group)
    v = g.integers(-4, 5, size=(m, k)).astype(np.float32)
    x = v.astype(np.float16) if xdt == "f16" else synth.f32_to_bf16_bits(v)
    Y = zq.gemm(W, x_dev(x, xdt))
    torch.cuda.synchronize()
    assert np.array_equal(Y.double().cpu().numpy(), O.gemm(p, bits, s, group, n, k, x, xdt))


def test_prefill_strided_rows_and_low_precision_out():
    m, n, k, ldx = 130, 300, 256, 320
    q, s, p, W = weight(4, n, k, 5)
    xf = synth.normal(synth.rng(6), (m, ldx), "bf16")
    X = x_dev(xf, "bf16")[:, :k]
    Y32 = zq.gemm(W, X)
    Yb = zq.gemm(W, X, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    x = np.ascontiguousarray(xf[:, :k])
    check(Y32.double().cpu().numpy(), O.gemm(p, 4, s, 0, n, k, x, "bf16"), x, "bf16", q, 0, s)
    assert torch.equal(Yb, Y32.to(torch.bfloat16))


# ---------------------------------------------------------------------------
# prefill plans: the tiles of many products in one persistent launch per bit
# width, taken from a device counter


def plan_problems(m, shapes, xdt, seed):
    probs, refs = [], []
    for i, (bits, n, k, group) in enumerate(shapes):
        q, s, p, W = weight(bits, n, k, seed + 10 * i, group=group)
        x = synth.normal(synth.rng(seed + 10 * i + 1), (m, k), xdt)
        Y = torch.full((m, n), float("nan"), device=DEV)
        probs.append((W, x_dev(x, xdt), Y, 0))
        refs.append((q, s, p, x, bits, n, k, group))
    return probs, refs


@pytest.mark.parametrize("xdt", ["f16", "bf16"])
def test_prefill_plan_matches_single_calls_and_oracle(xdt):
    # mixed bit widths, k and scale kinds (a queue each), ragged m and n
    # tiles; three runs (the counters must come back to zero after each)
    m = 300
    shapes = [(4, 600, 1024, 0), (2, 256, 192, 0), (8, 100, 512, 0), (4, 513, 64, 0), (2, 70, 1024, 0),
              (8, 260, 256, 0), (4, 700, 1024, 128), (2, 300, 256, 128), (8, 130, 384, 128), (4, 60, 128, 128)]
    probs, refs = plan_problems(m, shapes, xdt, seed=700 + (xdt == "bf16"))
    plan = zq.Plan(probs)
    for _ in range(3):
        for _, _, Y, _ in probs:
            Y.fill_(float("nan"))
        plan.run()
        torch.cuda.synchronize()
        plan.check()
        for (W, X, Y, _), _r in zip(probs, refs):
            # the same tile code as the single-launch kernel: identical outputs
            assert torch.equal(zq.gemm(W, X), Y)
    for (W, X, Y, _), (q, s, p, x, bits, n, k, group) in zip(probs, refs):
        check(Y.double().cpu().numpy(), O.gemm(p, bits, s, group, n, k, x, xdt), x, xdt, q, group, s,
              what=f"bits={bits} n={n} k={k} group={group}")


def test_prefill_plan_more_tiles_than_workgroups_integer_exact():
    # INT4: 256 + 320 tiles, more than the 512 workgroups, so some take two;
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
    _, _, _, W8 = weight(8, 64, 192, seed=4)
    X192 = torch.zeros((128, 200), dtype=torch.bfloat16, device=DEV)[:, 3:195]
    with pytest.raises(zq.ZqError) as e:  # activations not 16-byte aligned
        zq.Plan([(W8, X192, Y, 0)])
    assert e.value.status == zq.ERR_UNSUPPORTED
    # 16 < m <= 64 in one phase: the prefill tiles too (64 rows high here)
    X48 = torch.randn((48, 256), device=DEV).to(torch.bfloat16)
    Y48 = torch.full((48, 64), float("nan"), device=DEV)
    plan = zq.Plan([(W, X48, Y48, 0)])
    plan.run()
    torch.cuda.synchronize()
    plan.check()
    assert torch.equal(Y48, zq.gemm(W, X48))
