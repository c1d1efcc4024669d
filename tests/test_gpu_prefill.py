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
