"""Plans (many products in one resident launch) against the oracle and against
single zq_gemm calls; phase order checked with a real output -> input chain."""
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


@pytest.mark.parametrize("m", [1, 2, 4])
def test_plan_matches_oracle_and_single_calls(m):
    # mixed formats inside one phase are split into segments without a barrier
    # a miniature decoder layer stack with mixed formats: (bits, group, n, k, xdt, phase)
    spec = [(4, 128, 512, 1024, "f16", 0), (4, 128, 256, 1024, "f16", 0), (8, 0, 300, 2048, "f16", 1),
            (2, 128, 640, 1024, "bf16", 2), (4, 0, 1000, 512, "bf16", 2), (8, 128, 96, 4096, "bf16", 3),
            (4, 128, 3584, 3584, "f16", 4)]
    probs, refs = [], []
    for i, (bits, group, n, k, xdt, ph) in enumerate(spec):
        q, s, p, W = weight(bits, group, n, k, seed=100 + i)
        x = synth.normal(synth.rng(200 + i), (m, k), xdt)
        Y = torch.full((m, n), float("nan"), device=DEV)
        probs.append((W, x_dev(x, xdt), Y, ph))
        refs.append((q, s, p, x, xdt, group, bits, n, k))
    plan = zq.Plan(probs)
    for rep in range(3):
        for _, _, Y, _ in probs:
            Y.fill_(float("nan"))
        plan.run()
        torch.cuda.synchronize()
        plan.check()
        if rep == 0:
            first = [Y.clone() for _, _, Y, _ in probs]
        for (W, X, Y, _), (q, s, p, x, xdt, group, bits, n, k), f in zip(probs, refs, first):
            assert torch.equal(Y, f)                         # identical across runs
    for (W, X, Y, _), (q, s, p, x, xdt, group, bits, n, k) in zip(probs, refs):
        single = zq.gemm(W, X)
        torch.cuda.synchronize()
        # this plan mixes code widths, so it runs on the vector-ALU kernel;
        # a single call takes that kernel too for m = 1 and for INT2/INT8,
        # while single INT4 calls with m >= 2 run on the MFMA kernel (its own
        # summation order, checked against the oracle below)
        if m == 1 or bits != 4:
            assert torch.equal(single, Y)                    # same kernel, same split
        yref = O.gemm(p, bits, s, group, n, k, x, xdt)
        xn = np.sqrt((x64(x, xdt) ** 2).sum(1))[:, None]
        tol = 2e-3 * xn * np.abs(O.dequant(q, group, s)).max(1)[None, :] + 1e-3 * np.abs(yref)
        assert np.all(np.abs(Y.double().cpu().numpy() - yref) <= tol)


def test_plan_phase_order_with_output_feeding_input():
    """phase 0: y1 = W1 x0 (fp16 out, exact integers); phase 1: y2 = W2 y1.
    y1 is NaN before every run: phase 1 must read the values phase 0 stored."""
    k1, n1, n2 = 1024, 2048, 700
    g = synth.rng(5)
    q1 = g.integers(-1, 2, size=(n1, k1), dtype=np.int8)
    q2 = synth.codes_uniform(g, n2, n1, 4)
    one = np.full(n1 * k1 // 128, 0x3C00, dtype=np.uint16)
    _, s1, p1, W1 = weight(4, 128, n1, k1, 0, codes=q1, scales=one)
    _, s2, p2, W2 = weight(4, 128, n2, n1, 0, codes=q2, scales=np.full(n2 * n1 // 128, 0x3C00, dtype=np.uint16))
    x0 = g.integers(-1, 2, size=(1, k1)).astype(np.float16)
    X0 = torch.from_numpy(x0).to(DEV)
    Y1 = torch.empty((1, n1), dtype=torch.float16, device=DEV)
    Y2 = torch.empty((1, n2), dtype=torch.float32, device=DEV)
    plan = zq.Plan([(W1, X0, Y1, 0), (W2, Y1, Y2, 1)])
    y1_ref = O.gemm(p1, 4, s1, 128, n1, k1, x0, "f16")           # |y1| <= 1024: exact in fp16
    y2_ref = O.gemm(p2, 4, s2, 128, n2, n1, y1_ref.astype(np.float16), "f16")
    for _ in range(5):
        Y1.fill_(float("nan"))
        Y2.fill_(0)
        plan.run()
        torch.cuda.synchronize()
        assert np.array_equal(Y1.double().cpu().numpy(), y1_ref)
        assert np.array_equal(Y2.double().cpu().numpy(), y2_ref)
    plan.check()


def test_plan_many_phases_on_one_stream_with_other_work():
    probs = []
    for i in range(24):
        _, _, _, W = weight(4, 128, 512, 512, seed=i)
        X = torch.randn(1, 512, device=DEV).half()
        probs.append((W, X, torch.empty((1, 512), device=DEV), i))
    plan = zq.Plan(probs)
    outs = []
    for _ in range(4):
        plan.run()
        torch.cuda.synchronize()
        outs.append(torch.cat([Y for _, _, Y, _ in probs]).clone())
        probs[0][2].fill_(1.0)   # unrelated work between runs
    assert all(torch.equal(outs[0], o) for o in outs[1:])
    plan.check()


def test_plan_validation():
    _, _, _, Wbad = weight(4, 0, 64, 320, seed=1)        # k = 320: not whole 128-groups
    X = torch.zeros((1, 320), dtype=torch.float16, device=DEV)
    with pytest.raises(zq.ZqError) as e:
        zq.Plan([(Wbad, X, torch.empty((1, 64), device=DEV), 0)])
    assert e.value.status == zq.ERR_UNSUPPORTED
    _, _, _, W = weight(4, 128, 64, 512, seed=2)
    X = torch.zeros((1, 512), dtype=torch.float16, device=DEV)
    with pytest.raises(zq.ZqError) as e:
        zq.Plan([(W, X, torch.empty((1, 64), device=DEV), 1), (W, X, torch.empty((1, 64), device=DEV), 0)])
    assert e.value.status == zq.ERR_INVALID_ARG
    # 32 < m <= 64 with two phases takes INT4 only (32-row chunks of the
    # batched-decode kernel; one phase would go to the prefill tiles)
    _, _, _, W8 = weight(8, 128, 64, 512, seed=3)
    X33 = torch.zeros((33, 512), dtype=torch.float16, device=DEV)
    with pytest.raises(zq.ZqError) as e:
        zq.Plan([(W8, X33, torch.empty((33, 64), device=DEV), 0), (W8, X33, torch.empty((33, 64), device=DEV), 1)])
    assert e.value.status == zq.ERR_UNSUPPORTED


@pytest.mark.parametrize("xdt", ["f16", "bf16"])
def test_plan_m4_long_k(xdt):
    """m = 4 rows of k = 18944 (the 7B down projection's K): the staged
    activations take most of the LDS; two phases so the counter is reused."""
    m, k = 4, 18944
    probs, refs = [], []
    for i, n in enumerate([640, 384]):
        q, s, p, W = weight(4, 128, n, k, seed=300 + i)
        x = synth.normal(synth.rng(400 + i), (m, k), xdt)
        Y = torch.full((m, n), float("nan"), device=DEV)
        probs.append((W, x_dev(x, xdt), Y, i))
        refs.append((q, s, p, x, n))
    plan = zq.Plan(probs)
    for _ in range(2):
        plan.run()
        torch.cuda.synchronize()
    plan.check()
    for (W, X, Y, _), (q, s, p, x, n) in zip(probs, refs):
        yref = O.gemm(p, 4, s, 128, n, k, x, xdt)
        xn = np.sqrt((x64(x, xdt) ** 2).sum(1))[:, None]
        tol = 2e-3 * xn * np.abs(O.dequant(q, 128, s)).max(1)[None, :] + 1e-3 * np.abs(yref)
        assert np.all(np.abs(Y.double().cpu().numpy() - yref) <= tol)
        assert torch.equal(zq.gemm(W, X), Y)


def _check_chain(plan, y0, x0h, W0ref, later, xdt, runs=3):
    """run `plan` `runs` times with y0 (phase 0's output, the later phase's
    input) NaN-filled before each run; check phase 0 against the oracle and
    each later product against the oracle on the y0 values actually stored"""
    q0, s0, p0, g0, b0, n0, k0 = W0ref
    for _ in range(runs):
        y0.fill_(float("nan"))
        for _, _, Y, _ in later:
            Y.fill_(float("nan"))
        plan.run()
        torch.cuda.synchronize()
        plan.check()
        y0_host = y0.cpu()
        assert not torch.isnan(y0_host).any()
        y0ref = O.gemm(p0, b0, s0, g0, n0, k0, x0h, xdt)
        y0bits = y0_host.view(torch.int16).numpy().view(np.uint16) if xdt == "bf16" else y0_host.numpy()
        y0_64 = x64(y0bits, xdt)
        xn = np.sqrt((x64(x0h, xdt) ** 2).sum(1))[:, None]
        tol0 = 2e-3 * xn * np.abs(O.dequant(q0, g0, s0)).max(1)[None, :] + 1e-3 * np.abs(y0ref)
        tol0 = tol0 + 0.5 * np.abs(y0ref) * (2.0 ** -7 if xdt == "bf16" else 2.0 ** -10)
        assert np.all(np.abs(y0_64 - y0ref) <= tol0)
        xn1 = np.sqrt((y0_64 ** 2).sum(1))[:, None]
        for W, _, Y, (q, s, p, bits, group, n, k) in later:
            y = Y.double().cpu().numpy()
            assert not np.isnan(y).any(), "a later segment read the earlier phase's output before it was stored"
            yref = O.gemm(p, bits, s, group, n, k, y0bits, xdt)
            tol = 2e-3 * xn1 * np.abs(O.dequant(q, group, s)).max(1)[None, :] + 1e-3 * np.abs(yref)
            assert np.all(np.abs(y - yref) <= tol)


def _chain_plan(m, xdt, first, later_specs, seed):
    """phase 0: y0 = W0 x0 (y0 in the activation dtype); phase 1: the products
    of later_specs (bits, group, n) all read y0"""
    b0, g0, n0, k0 = first
    q0, s0, p0, W0 = weight(b0, g0, n0, k0, seed=seed)
    x0h = synth.normal(synth.rng(seed + 1), (m, k0), xdt)
    tdt = torch.bfloat16 if xdt == "bf16" else torch.float16
    y0 = torch.empty((m, n0), dtype=tdt, device=DEV)
    probs = [(W0, x_dev(x0h, xdt), y0, 0)]
    later = []
    for i, (bits, group, n) in enumerate(later_specs):
        q, s, p, W = weight(bits, group, n, n0, seed=seed + 10 + i)
        Y = torch.empty((m, n), dtype=torch.float32, device=DEV)
        probs.append((W, y0, Y, 1))
        later.append((W, y0, Y, (q, s, p, bits, group, n, n0)))
    return zq.Plan(probs), y0, x0h, (q0, s0, p0, g0, b0, n0, k0), later


def test_phase_wait_when_first_segment_has_fewer_workgroups():
    """vector-ALU plan, m = 1. Phase 0 (16 workgroups) writes y0; phase 1 is an
    INT2 segment spread over 1 workgroup, then an INT4 segment over 256: the
    workgroups with no INT2 rows must still wait before they read y0."""
    plan, y0, x0h, ref0, later = _chain_plan(1, "f16", (4, 128, 1024, 256), [(2, 128, 16), (4, 128, 8192)], 700)
    _check_chain(plan, y0, x0h, ref0, later, "f16")


def test_phase_wait_across_lds_split_segments():
    """vector-ALU plan, m = 4. Phase 1 holds 40 one-row INT2 products and one
    of 2048 rows, all of k = 128: a workgroup's range would stage more
    activation buffers than LDS holds, so the phase is cut into segments of
    10, 10, 10 and 11 products without waits between them; only the last one
    spreads over more than one workgroup."""
    specs = [(2, 128, 1)] * 40 + [(2, 128, 2048)]
    plan, y0, x0h, ref0, later = _chain_plan(4, "f16", (4, 128, 128, 256), specs, 800)
    _check_chain(plan, y0, x0h, ref0, later, "f16")


def test_mstream_phase_wait_when_first_segment_has_few_rows():
    """MFMA batched-decode plan, m = 8: phase 1 is a per-tensor INT4 segment of
    16 rows (rows on 16 of 256 workgroups), then a group-scaled one of 8192."""
    plan, y0, x0h, ref0, later = _chain_plan(8, "bf16", (4, 128, 1024, 18944), [(4, 0, 16), (4, 128, 8192)], 900)
    _check_chain(plan, y0, x0h, ref0, later, "bf16")
