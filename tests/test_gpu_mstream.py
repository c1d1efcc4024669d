"""The MFMA batched-decode kernel (INT4, 5..32 activation rows, k a multiple
of 512), through zq_gemm and through plans, against the fp64 oracle."""
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


def weight(bits, group, n, k, seed, codes=None, scales=None):
    g = synth.rng(seed)
    q = synth.codes_uniform(g, n, k, bits) if codes is None else codes
    s = synth.scales_abs_normal(g, O.num_scales(group, n, k)) if scales is None else scales
    p = O.pack(q, bits)
    W = zq.ZqWeight(bits, group, n, k, torch.from_numpy(p.reshape(-1)).to(DEV),
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


def check(y, yref, x, xdt, q, group, s, what=""):
    xn = np.sqrt((x64(x, xdt) ** 2).sum(1))[:, None]
    tol = 2e-3 * xn * np.abs(O.dequant(q, group, s)).max(1)[None, :] + 1e-3 * np.abs(yref)
    err = np.abs(y - yref)
    bad = np.argwhere(err > tol)
    assert bad.size == 0, f"{what}: {len(bad)} bad, first {bad[:3].tolist()}"


@pytest.mark.parametrize("xdt", ["f16", "bf16"])
@pytest.mark.parametrize("group", [0, 128])
@pytest.mark.parametrize("m", [2, 3, 4, 5, 8, 13, 16, 17, 24, 32])
def test_mstream_gemm_matches_oracle(xdt, group, m):
    # ragged tiles (300 = 18 x 16 + 12), several 256-row blocks, 1 and 3 chunks
    for n, k in [(16, 512), (300, 1536), (1000, 512)]:
        seed = 7919 * m + 31 * n + k + group + (xdt == "bf16")
        q, s, p, W = weight(4, group, n, k, seed)
        x = synth.normal(synth.rng(seed + 1), (m, k), xdt)
        Y = zq.gemm(W, x_dev(x, xdt))
        torch.cuda.synchronize()
        yref = O.gemm(p, 4, s, group, n, k, x, xdt)
        check(Y.double().cpu().numpy(), yref, x, xdt, q, group, s, f"m={m} n={n} k={k}")


@pytest.mark.parametrize("xdt", ["f16", "bf16"])
@pytest.mark.parametrize("m", [5, 8, 32])
def test_mstream_integer_inputs_bit_exact(xdt, m):
    n, k = 530, 3584
    g = synth.rng(100 + m)
    q = synth.codes_uniform(g, n, k, 4)
    s = np.where(g.random(n * k // 128) < 0.5, 0x3800, 0x3C00).astype(np.uint16)
    q, s, p, W = weight(4, 128, n, k, 0, codes=q, scales=s)
    v = g.integers(-4, 5, size=(m, k)).astype(np.float32)
    x = v.astype(np.float16) if xdt == "f16" else synth.f32_to_bf16_bits(v)
    Y = zq.gemm(W, x_dev(x, xdt))
    torch.cuda.synchronize()
    assert np.array_equal(Y.double().cpu().numpy(), O.gemm(p, 4, s, 128, n, k, x, xdt))


def test_mstream_long_k_and_low_precision_out():
    m, n, k = 32, 96, 18944
    q, s, p, W = weight(4, 128, n, k, 9)
    x = synth.normal(synth.rng(10), (m, k), "bf16")
    yref = O.gemm(p, 4, s, 128, n, k, x, "bf16")
    Y = zq.gemm(W, x_dev(x, "bf16"))
    Yh = zq.gemm(W, x_dev(x, "bf16"), out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    check(Y.double().cpu().numpy(), yref, x, "bf16", q, 128, s, "f32 out")
    assert torch.equal(Yh, Y.to(torch.bfloat16))  # same sums, rounded once


@pytest.mark.parametrize("m", [2, 8, 16, 17, 32])
def test_mstream_plan_matches_oracle_and_single_calls(m):
    spec = [(128, 512, 1024, "f16", 0), (0, 300, 1024, "f16", 0), (128, 4096, 512, "bf16", 1),
            (0, 640, 2048, "bf16", 1), (128, 3584, 3584, "f16", 2)]
    probs, refs = [], []
    for i, (group, n, k, xdt, ph) in enumerate(spec):
        q, s, p, W = weight(4, group, n, k, seed=500 + i)
        x = synth.normal(synth.rng(600 + i), (m, k), xdt)
        Y = torch.full((m, n), float("nan"), device=DEV)
        probs.append((W, x_dev(x, xdt), Y, ph))
        refs.append((q, s, p, x, xdt, group, n, k))
    plan = zq.Plan(probs)
    for _ in range(3):
        for _, _, Y, _ in probs:
            Y.fill_(float("nan"))
        plan.run()
        torch.cuda.synchronize()
    plan.check()
    for (W, X, Y, _), (q, s, p, x, xdt, group, n, k) in zip(probs, refs):
        assert torch.equal(zq.gemm(W, X), Y)  # same kernel, same per-row arithmetic
        check(Y.double().cpu().numpy(), O.gemm(p, 4, s, group, n, k, x, xdt), x, xdt, q, group, s)


@pytest.mark.parametrize("m", [8, 17, 32])
def test_mstream_plan_long_ranges(m):
    """Workgroup ranges of several hundred rows: 512-row blocks with both
    256-row halves live, a partial second half, blocks that end at a product
    boundary, one and two 512-k chunks. Every 5th row and the rows around each
    workgroup's range and each 256-row half are checked against the oracle."""
    ncu = torch.cuda.get_device_properties(0).multi_processor_count
    spec = [(128, 41000, 512, 0), (128, 69000, 512, 1), (0, 150000, 1024, 2)]  # (group, n, k, seed)
    probs, refs = [], []
    for group, n, k, sd in spec:
        q, s, p, W = weight(4, group, n, k, seed=700 + sd)
        x = synth.normal(synth.rng(800 + sd), (m, k), "bf16")
        Y = torch.full((m, n), float("nan"), device=DEV)
        probs.append((W, x_dev(x, "bf16"), Y, 0))
        refs.append((q, s, p, x, group, n, k))
    plan = zq.Plan(probs)
    plan.run()
    torch.cuda.synchronize()
    plan.check()
    # segments: (group 0, k 1024) then (group 128, k 512) = products 0 and 1
    seams = {0: set(), 1: set(), 2: set()}
    for members in ([2], [0, 1]):
        N = sum(spec[i][1] for i in members)
        for w in range(ncu):
            r0, r1 = w * N // ncu, (w + 1) * N // ncu
            for r in list(range(r0, r1, 256)) + [r1 - 1]:
                for rr in (r - 1, r, r + 1, r + 255, r + 256):
                    off = 0
                    for i in members:
                        if off <= rr < off + spec[i][1] and r0 <= rr < r1:
                            seams[i].add(rr - off)
                        off += spec[i][1]
    for i, ((W, X, Y, _), (q, s, p, x, group, n, k)) in enumerate(zip(probs, refs)):
        rows = np.array(sorted(set(range(0, n, 5)) | seams[i] | {n - 1}), dtype=np.int64)
        pr = p.reshape(n, -1)[rows]
        sr = s if group == 0 else s.reshape(n, -1)[rows]
        yref = O.gemm(pr, 4, sr, group, len(rows), k, x, "bf16")
        got = Y[:, torch.from_numpy(rows).to(DEV)].double().cpu().numpy()
        check(got, yref, x, "bf16", q[rows], group, sr, f"m={m} product {i}")


def test_mstream_plan_phase_chain():
    """phase 0: Y1 = W1 X0 (fp16 out, exact integers); phase 1: Y2 = W2 Y1."""
    m, k1, n1, n2 = 16, 1024, 2048, 700
    g = synth.rng(77)
    q1 = g.integers(-1, 2, size=(n1, k1), dtype=np.int8)
    q2 = synth.codes_uniform(g, n2, n1, 4)
    _, s1, p1, W1 = weight(4, 128, n1, k1, 0, codes=q1, scales=np.full(n1 * k1 // 128, 0x3C00, np.uint16))
    _, s2, p2, W2 = weight(4, 128, n2, n1, 0, codes=q2, scales=np.full(n2 * n1 // 128, 0x3C00, np.uint16))
    x0 = g.integers(-1, 2, size=(m, k1)).astype(np.float16)
    X0 = torch.from_numpy(x0).to(DEV)
    Y1 = torch.empty((m, n1), dtype=torch.float16, device=DEV)
    Y2 = torch.empty((m, n2), dtype=torch.float32, device=DEV)
    plan = zq.Plan([(W1, X0, Y1, 0), (W2, Y1, Y2, 1)])
    y1 = O.gemm(p1, 4, s1, 128, n1, k1, x0, "f16")
    y2 = O.gemm(p2, 4, s2, 128, n2, n1, y1.astype(np.float16), "f16")
    for _ in range(4):
        Y1.fill_(float("nan"))
        Y2.fill_(0)
        plan.run()
        torch.cuda.synchronize()
        assert np.array_equal(Y1.double().cpu().numpy(), y1)
        assert np.array_equal(Y2.double().cpu().numpy(), y2)
    plan.check()


def test_mstream_plan_rejects_other_formats():
    _, _, _, W = weight(8, 128, 64, 512, seed=1)
    X = torch.zeros((8, 512), dtype=torch.float16, device=DEV)
    with pytest.raises(zq.ZqError) as e:
        zq.Plan([(W, X, torch.empty((8, 64), device=DEV), 0)])
    assert e.value.status == zq.ERR_UNSUPPORTED
    _, _, _, W4 = weight(4, 128, 64, 384, seed=2)
    X = torch.zeros((8, 384), dtype=torch.float16, device=DEV)
    with pytest.raises(zq.ZqError):
        zq.Plan([(W4, X, torch.empty((8, 64), device=DEV), 0)])
    X33 = torch.zeros((33, 512), dtype=torch.float16, device=DEV)
    with pytest.raises(zq.ZqError):  # two phases past 32 rows: the batched-decode chunks, INT4 k % 512 only
        zq.Plan([(W4, X33, torch.empty((33, 64), device=DEV), 0), (W4, X33, torch.empty((33, 64), device=DEV), 1)])


# ---------------------------------------------------------------------------
# mid-batch m (32 < m): symmetric codes take the prefill tiles (32, 64 or 128
# rows high), single calls and one-phase plans; plans with several phases (and
# asymmetric codes) run in 32-row chunks on the batched-decode kernel


def chunks(m):
    out, r0 = [], 0
    while r0 < m:
        mc = 31 if m - r0 == 33 else min(32, m - r0)
        out.append((r0, mc))
        r0 += mc
    return out


@pytest.mark.parametrize("xdt", ["f16", "bf16"])
@pytest.mark.parametrize("group", [0, 128])
@pytest.mark.parametrize("m", [33, 48, 64, 65, 100])
def test_midbatch_matches_oracle(xdt, group, m):
    n, k = 300, 1024
    seed = 40 * m + group + (xdt == "bf16")
    q, s, p, W = weight(4, group, n, k, seed)
    x = synth.normal(synth.rng(seed + 1), (m, k), xdt)
    X = x_dev(x, xdt)
    Y = zq.gemm(W, X)
    torch.cuda.synchronize()
    check(Y.double().cpu().numpy(), O.gemm(p, 4, s, group, n, k, x, xdt), x, xdt, q, group, s, what=f"m={m}")


@pytest.mark.parametrize("m", [33, 64, 100])
def test_midbatch_plan_matches_oracle_and_single_calls(m):
    probs, refs = [], []
    for i, (group, n, k) in enumerate([(128, 512, 1024), (0, 300, 512), (128, 1000, 1536)]):
        q, s, p, W = weight(4, group, n, k, seed=800 + 10 * m + i)
        x = synth.normal(synth.rng(850 + 10 * m + i), (m, k), "bf16")
        Y = torch.full((m, n), float("nan"), device=DEV)
        probs.append((W, x_dev(x, "bf16"), Y, 0))
        refs.append((q, s, p, x, group, n, k))
    plan = zq.Plan(probs)
    for _ in range(2):
        plan.run()
        torch.cuda.synchronize()
    plan.check()
    for (W, X, Y, _), (q, s, p, x, group, n, k) in zip(probs, refs):
        check(Y.double().cpu().numpy(), O.gemm(p, 4, s, group, n, k, x, "bf16"), x, "bf16", q, group, s,
              what=f"n={n}")
        assert torch.equal(Y, zq.gemm(W, X))  # a prefill plan: the single calls' tiles


def test_midbatch_plan_rejects_other_formats():
    # several phases past 32 rows: 32-row chunks, INT4 only
    _, _, _, W8 = weight(8, 128, 64, 512, seed=3)
    X = torch.zeros((48, 512), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(zq.ZqError) as e:
        zq.Plan([(W8, X, torch.empty((48, 64), device=DEV), 0), (W8, X, torch.empty((48, 64), device=DEV), 1)])
    assert e.value.status == zq.ERR_UNSUPPORTED
