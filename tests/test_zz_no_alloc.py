"""zq_pack_noalloc (the allocation-free variant of zq_pack, whose flag words
live in a static device array inside the library) against zq_pack, through
the C-ABI: packed codes and scales must be identical bit for bit, on two
calls in a row with the second one smaller, and the static words must be
cleared between calls (a large tensor absmax, or an error, in one call must
not leak into the next)."""
import numpy as np
import pytest
import torch

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


def _weights(n, k, dtype, seed, scale=1.0):
    g = synth.rng(seed)
    w = torch.from_numpy(g.standard_normal((n, k), dtype=np.float32) * np.float32(scale))
    return w.to(dtype).to(DEV)


def _both(w, bits, group, scales=None):
    """zq_pack and zq_pack_noalloc on the same input, into fresh buffers"""
    n, k = w.shape
    outs = []
    for noalloc in (False, True):
        packed = torch.full((zq.packed_bytes(bits, n, k),), 0xA5, dtype=torch.uint8, device=DEV)
        sc = None if scales is not None and w.dtype == torch.int8 else \
            torch.full((max(zq.num_scales(group, n, k), 1),), float("nan"), dtype=torch.float16, device=DEV)
        zq.pack_into(w, bits, group, packed, sc, scales=scales, noalloc=noalloc)
        outs.append((packed.cpu(), None if sc is None else sc.view(torch.int16).cpu()))
    return outs


@pytest.mark.parametrize("dtype,bits,group,big,small", [
    (torch.float32, 4, 0, (300, 1024), (40, 256)),
    (torch.bfloat16, 2, 128, (512, 2048), (64, 128)),
    (torch.float16, 8, 128, (96, 4096), (8, 512)),
    (torch.float32, 8, 0, (1000, 640), (3, 128)),
])
def test_noalloc_pack_matches_pack_on_two_calls(dtype, bits, group, big, small):
    # the first call's tensor absmax is 100x the second's: a stale absmax
    # word would give the second call the first one's scale
    for i, ((n, k), scale) in enumerate([(big, 100.0), (small, 1.0)]):
        w = _weights(n, k, dtype, seed=10 * bits + i, scale=scale)
        (p0, s0), (p1, s1) = _both(w, bits, group)
        assert torch.equal(p0, p1), f"call {i}: packed codes differ"
        assert torch.equal(s0, s1), f"call {i}: scales differ"


def test_noalloc_pack_integer_codes_and_given_scales():
    for i, (n, k) in enumerate([(256, 1024), (16, 128)]):
        g = synth.rng(70 + i)
        q = torch.from_numpy(synth.codes_uniform(g, n, k, 4)).to(DEV)
        s = torch.from_numpy(synth.scales_abs_normal(g, n * k // 128).view(np.float16)).to(DEV)
        (p0, s0), (p1, s1) = _both(q, 4, 128, scales=s)
        assert torch.equal(p0, p1) and s0 is None and s1 is None


def test_noalloc_pack_error_then_clean_call():
    w = _weights(64, 256, torch.float32, seed=3)
    w[5, 7] = float("inf")
    packed = torch.empty(zq.packed_bytes(4, 64, 256), dtype=torch.uint8, device=DEV)
    sc = torch.empty(zq.num_scales(128, 64, 256), dtype=torch.float16, device=DEV)
    with pytest.raises(zq.ZqError) as e:
        zq.pack_into(w, 4, 128, packed, sc, noalloc=True)
    assert e.value.status == zq.ERR_RANGE
    q = torch.full((32, 128), 9, dtype=torch.int8, device=DEV)  # outside INT4
    with pytest.raises(zq.ZqError) as e:
        zq.pack_into(q, 4, 0, torch.empty(32 * 64, dtype=torch.uint8, device=DEV), None,
                     scales=torch.ones(1, dtype=torch.float16, device=DEV), noalloc=True)
    assert e.value.status == zq.ERR_RANGE
    # the next call starts from cleared words and succeeds
    w2 = _weights(48, 384, torch.float32, seed=4)
    (p0, s0), (p1, s1) = _both(w2, 4, 128)
    assert torch.equal(p0, p1) and torch.equal(s0, s1)
    (p0, s0), (p1, s1) = _both(w2, 4, 0)
    assert torch.equal(p0, p1) and torch.equal(s0, s1)


def test_noalloc_pack_empty_shapes():
    for n, k in [(0, 256), (16, 0)]:
        w = torch.zeros((n, k), dtype=torch.float32, device=DEV)
        packed = torch.empty(max(zq.packed_bytes(4, n, k), 1), dtype=torch.uint8, device=DEV)
        sc = torch.full((1,), float("nan"), dtype=torch.float16, device=DEV)
        zq.pack_into(w, 4, 0, packed, sc, noalloc=True)
        assert sc.view(torch.int16).item() == 0  # absmax of an empty tensor is 0: scale +0
