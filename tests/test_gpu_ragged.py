"""Rows that end in a partial step of the M <= 4 decode kernel, through the
C-ABI, against the fp64 oracle.

The decode kernel walks a weight row in steps of 16 chunks (256 bytes). Rows
whose chunk count is not a multiple of 16 (K = 896 and 4736 in INT4: the
o and down projections of one rank's share of Qwen2.5-7B under 4-way tensor
parallelism) end in a partial step. Cases: every bit width, per-tensor and
per-group scales, symmetric and asymmetric codes, M = 1..4, fp16 and bf16
activations, rows of a single partial step, and plans that mix partial and
whole steps. Plans with M <= 4 and these shapes run on the decode kernel
(the MFMA batched kernel needs K % 512 == 0), so they pin it down.
"""
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


def x_dev(x, xdt):
    if xdt == "bf16":
        return torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).to(DEV)
    return torch.from_numpy(x).to(DEV)


def x64(x, xdt):
    if xdt == "bf16":
        return torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    return x.astype(np.float64)


def check(y, yref, x, xdt, wdeq, what=""):
    xn = np.sqrt((x64(x, xdt) ** 2).sum(1))[:, None]
    tol = 2e-3 * xn * np.abs(wdeq).max(1)[None, :] + 1e-3 * np.abs(yref)
    bad = np.argwhere(~(np.abs(y - yref) <= tol))
    assert bad.size == 0, f"{what}: {len(bad)} outputs out of tolerance, first {bad[:3].tolist()}"


def sym_weight(bits, group, n, k, seed):
    g = synth.rng(seed)
    q = synth.codes_uniform(g, n, k, bits)
    s = synth.scales_abs_normal(g, O.num_scales(group, n, k))
    p = O.pack(q, bits)
    W = zq.ZqWeight(bits, group, n, k, dev(p.reshape(-1)), dev(s.view(np.float16)))
    ref = lambda x, xdt: O.gemm(p, bits, s, group, n, k, x, xdt)  # noqa: E731
    return W, ref, O.dequant(q, group, s)


def asym_weight(bits, n, k, seed):
    g = synth.rng(seed)
    q = g.integers(0, 1 << bits, size=(n, k)).astype(np.uint8)
    s = synth.scales_abs_normal(g, n * (k // 128))
    z = np.array([O.f64_to_f16(v) for v in g.standard_normal(n * (k // 128)) * 0.01], dtype=np.uint16)
    p = O.pack_u(q, bits)
    W = zq.ZqWeight(bits, 128, n, k, dev(p.reshape(-1)), dev(s.view(np.float16)), dev(z.view(np.float16)))
    ref = lambda x, xdt: O.gemm_asym(p, bits, s, z, n, k, x, xdt)  # noqa: E731
    return W, ref, O.dequant_asym(q, s, z)


# (n, k) per bit width: chunks per row C = k * bits / 128; C % 16 != 0 in all,
# C < 16 (a single partial step) in some
RAGGED = {
    2: [(300, 896), (37, 4736), (130, 1152)],   # C = 14, 74, 18
    4: [(300, 896), (37, 4736), (70, 128)],     # C = 28, 148, 4
    8: [(300, 896), (37, 4736), (70, 384)],     # C = 56, 296, 24
}


@pytest.mark.parametrize("xdt", ["f16", "bf16"])
@pytest.mark.parametrize("bits", [2, 4, 8])
@pytest.mark.parametrize("group", [0, 128])
@pytest.mark.parametrize("m", [1, 2, 3, 4])
def test_partial_last_step_matches_oracle(xdt, bits, group, m):
    for n, k in RAGGED[bits]:
        seed = 7919 * bits + 131 * m + 17 * group + k % 1009 + (xdt == "bf16")
        W, ref, wdeq = sym_weight(bits, group, n, k, seed)
        x = synth.normal(synth.rng(seed + 1), (m, k), xdt)
        Y = zq.gemm(W, x_dev(x, xdt))
        torch.cuda.synchronize()
        check(Y.double().cpu().numpy(), ref(x, xdt), x, xdt, wdeq, what=f"n={n} k={k}")


@pytest.mark.parametrize("xdt", ["f16", "bf16"])
@pytest.mark.parametrize("bits", [2, 4])
@pytest.mark.parametrize("m", [1, 4])
def test_partial_last_step_asymmetric(xdt, bits, m):
    for n, k in RAGGED[bits]:
        seed = 4409 * bits + 53 * m + k % 997 + (xdt == "bf16")
        W, ref, wdeq = asym_weight(bits, n, k, seed)
        x = synth.normal(synth.rng(seed + 1), (m, k), xdt)
        Y = zq.gemm(W, x_dev(x, xdt))
        torch.cuda.synchronize()
        check(Y.double().cpu().numpy(), ref(x, xdt), x, xdt, wdeq, what=f"n={n} k={k}")


@pytest.mark.parametrize("xdt", ["f16", "bf16"])
@pytest.mark.parametrize("bits", [2, 4, 8])
@pytest.mark.parametrize("m", [1, 3])
def test_partial_last_step_integer_inputs_bit_exact(xdt, bits, m):
    # integer activations, scales 0.5 / 1: every fp32 partial sum is exact, and
    # so is the zero padding of the partial step
    n, k = 90, 4736
    g = synth.rng(300 + 10 * bits + m)
    q = synth.codes_uniform(g, n, k, bits)
    s = np.where(g.random(n * k // 128) < 0.5, 0x3800, 0x3C00).astype(np.uint16)
    p = O.pack(q, bits)
    W = zq.ZqWeight(bits, 128, n, k, dev(p.reshape(-1)), dev(s.view(np.float16)))
    v = g.integers(-4, 5, size=(m, k)).astype(np.float32)
    x = v.astype(np.float16) if xdt == "f16" else synth.f32_to_bf16_bits(v)
    Y = zq.gemm(W, x_dev(x, xdt))
    torch.cuda.synchronize()
    assert np.array_equal(Y.double().cpu().numpy(), O.gemm(p, bits, s, 128, n, k, x, xdt))


def test_activation_storage_past_k_is_never_read():
    # activations past k are never read: a row of x whose storage continues
    # with NaN (ldx > k) gives finite outputs equal to the unpadded ones
    n, k, m = 64, 896, 2
    W, ref, wdeq = sym_weight(4, 128, n, k, 5)
    x = synth.normal(synth.rng(6), (m, k), "f16")
    xs = np.full((m, k + 128), np.nan, dtype=np.float16)
    xs[:, :k] = x
    X = dev(xs)[:, :k]
    Y = zq.gemm(W, X)
    torch.cuda.synchronize()
    y = Y.double().cpu().numpy()
    assert np.isfinite(y).all()
    check(y, ref(x, "f16"), x, "f16", wdeq)


@pytest.mark.parametrize("m", [1, 2, 4])
def test_plan_tp4_shard_shapes(m):
    # one decoder layer of the 7B shard under 4-way tensor parallelism, two
    # layers' worth of products, in the four chained phases and independent
    shapes = synth.QWEN25_7B_TP4
    phase = {"q": 0, "k": 0, "v": 0, "o": 1, "gate": 2, "up": 2, "down": 3}
    for order in ("independent", "chained"):
        probs, refs = [], []
        for layer in range(2):
            for i, (name, n, k) in enumerate(shapes):
                seed = 100 * layer + i + 10 * m
                if name == "down" and layer == 1:
                    W, ref, wdeq = asym_weight(4, n, k, seed)  # one asymmetric product in the mix
                else:
                    W, ref, wdeq = sym_weight(4, 128, n, k, seed)
                x = synth.normal(synth.rng(seed + 7), (m, k), "f16")
                Y = torch.full((m, n), float("nan"), device=DEV)
                ph = 4 * layer + phase[name] if order == "chained" else 0
                probs.append((W, x_dev(x, "f16"), Y, ph))
                refs.append((ref, x, wdeq, name))
        plan = zq.Plan(probs)
        for _ in range(2):
            plan.run()
            torch.cuda.synchronize()
        plan.check()
        for (W, X, Y, _), (ref, x, wdeq, name) in zip(probs, refs):
            check(Y.double().cpu().numpy(), ref(x, "f16"), x, "f16", wdeq, what=f"{order} {name}")


@pytest.mark.parametrize("m", [1, 4])
def test_plan_mixing_partial_and_whole_steps(m):
    # products with whole steps (k = 3584, 512), partial ones, and one of a
    # single partial step, in one plan
    probs, refs = [], []
    for i, (n, k) in enumerate([(512, 3584), (300, 896), (1000, 512), (2000, 4736), (77, 128), (3584, 896)]):
        W, ref, wdeq = sym_weight(4, 128, n, k, 900 + i)
        x = synth.normal(synth.rng(950 + i), (m, k), "bf16")
        Y = torch.full((m, n), float("nan"), device=DEV)
        probs.append((W, x_dev(x, "bf16"), Y, 0))
        refs.append((ref, x, wdeq))
    plan = zq.Plan(probs)
    plan.run()
    torch.cuda.synchronize()
    plan.check()
    for (W, X, Y, _), (ref, x, wdeq) in zip(probs, refs):
        check(Y.double().cpu().numpy(), ref(x, "bf16"), x, "bf16", wdeq, what=f"n={W.n} k={W.k}")
