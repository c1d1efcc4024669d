"""Parity at the benchmark's full sizes, in the launch configurations bench.py
times, on sampled outputs: for every product of the step, a few weight rows
and activation rows are copied back and recomputed by the fp64 oracle.

    Qwen2.5-7B decode stack   (28 layers x 7, M = 1, INT4 g128, fp16 x), plan
    Qwen2.5-7B decode stack with asymmetric INT4 weights, plan
    one rank's share of the 7B decode stack under 4-way tensor parallelism, plan
    Qwen2.5-32B decode stack  (64 layers x 7, M = 1), plan
    7B stack, M = 4, 8, 32 (bf16 x), plan (MFMA batched-decode kernel), and
    M = 128, 512, plan (group-scaled prefill tiles)
    7B prefill stack (per-layer INT2/4/8, per-tensor scale, M = 2048, bf16 x),
    plan (tile queues) and graph over 4 streams
"""
import os
import sys

import numpy as np
import pytest
import torch

from oracle import oracle as O
from weight_quantized_amd import synth

pytestmark = pytest.mark.gpu
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def mods():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    sys.path.insert(0, ROOT)
    import bench
    from weight_quantized_amd import zq
    zq.lib()
    return bench, zq


def run_step(bench, stack, launch, order="independent", streams=4):
    torch = stack.torch
    for _, _, y in stack.launches:
        y.fill_(float("nan"))
    if launch == "plan":
        stack.make_plan(order)
        stack.plan_step()
        torch.cuda.synchronize()
        stack.plan.check()
    else:
        sms = [torch.cuda.Stream() for _ in range(streams)]
        g = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            stack.step(sms)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        with torch.cuda.graph(g):
            stack.step(sms)
        for _, _, y in stack.launches:
            y.fill_(float("nan"))
        g.replay()
        g.replay()  # a second replay must give the same outputs
        torch.cuda.synchronize()


def _ceil(a, b):
    return -(-a // b)


def split_rows(stack, order="independent"):
    """Rows where the work of the plan that bench.py times is split, per
    product index: the first and last row of every workgroup's range and of
    every 256-row block, the rows of quads whose steps are split between two
    waves (vector-ALU decode kernel), and 256-column tile edges (prefill). This
    mirrors the kernels' documented split (segments of one format, rows
    [w*N/G, (w+1)*N/G) of a segment for workgroup w, equal runs of quad-steps
    per wave) so that the sampled check always covers the seams."""
    ncu = torch.cuda.get_device_properties(0).multi_processor_count
    L = stack.launches
    out = {i: set() for i in range(len(L))}
    if stack.m > 64 and all(W.zeros is None for W, _, _ in L):  # prefill tiles
        for i, (W, _, _) in enumerate(L):
            for t in range(0, W.n, 256):
                out[i].update({t, min(t + 255, W.n - 1)})
        return out
    m = min(stack.m, 32)  # 32-row chunks past 32: each chunk splits the rows like an m = 32 plan
    # the plan's product order: bench's order, then a stable sort by format
    per_layer = len(stack.shapes)
    idx = list(range(len(L)))
    if order == "independent":
        idx.sort(key=lambda i: (L[i][0].k, i // per_layer, stack.shapes[i % per_layer][0]))
        phases = {i: 0 for i in idx}
    else:
        ph = {"q": 0, "k": 0, "v": 0, "o": 1, "gate": 2, "up": 2, "down": 3}
        phases = {i: 4 * (i // per_layer) + ph[stack.shapes[i % per_layer][0]] for i in idx}
    fmt = lambda i: (L[i][0].bits, L[i][0].group, L[i][0].zeros is not None, -L[i][0].k)
    idx.sort(key=lambda i: (phases[i], fmt(i)))
    mfma = m >= 2 and all(W.bits == 4 and W.k % 512 == 0 for W, _, _ in L)
    segs = []
    for i in idx:
        if segs and phases[segs[-1][0]] == phases[i] and fmt(segs[-1][0]) == fmt(i):
            segs[-1].append(i)
        else:
            segs.append([i])
    for seg in segs:
        W0 = L[seg[0]][0]
        offs, N = [], 0
        for i in seg:
            offs.append(N)
            N += L[i][0].n

        def mark(r):
            for i, o in zip(seg, offs):
                if o <= r < o + L[i][0].n:
                    out[i].add(r - o)

        if mfma:
            G = ncu
        else:
            C = W0.k // (128 // W0.bits)
            steps = _ceil(N, 4) * _ceil(C, 16)
            G = max(1, min(ncu, _ceil(steps, 16 if m == 1 else 8)))
        for w in range(G):
            r0, r1 = w * N // G, (w + 1) * N // G
            if r1 == r0:
                continue
            for r in range(r0, r1, 256):
                mark(r)
                mark(min(r + 255, r1 - 1))
            mark(r1 - 1)
            if not mfma:
                NW = 16 if m == 1 else 8
                CB = _ceil(W0.k // (128 // W0.bits), 16)
                T = _ceil(r1 - r0, 4) * CB
                for wv in range(1, NW):
                    b = wv * T // NW
                    if b % CB:
                        q = b // CB
                        for rr in range(r0 + 4 * q, min(r0 + 4 * q + 4, r1)):
                            mark(rr)
    return out


def check_sampled(stack, n_rows=6, m_rows=None, seed=0, seams=None):
    """sampled rows of every product against the oracle: row 0, the last row,
    n_rows random rows and, when given, the rows at the work split (seams)"""
    g = np.random.default_rng(seed)
    xdt = stack.xdt
    for idx, (W, x, y) in enumerate(stack.launches):
        extra = sorted(seams[idx]) if seams else []
        rows = np.unique(np.concatenate([[0, W.n - 1], g.integers(0, W.n, n_rows), extra]).astype(np.int64))
        # prefill: activation rows at every 128-row tile edge besides the random ones
        edges = [r for t in range(0, stack.m, 128) for r in (t, min(t + 127, stack.m - 1))]
        ms = np.arange(stack.m) if m_rows is None else np.unique(
            np.concatenate([[0, stack.m - 1], g.integers(0, stack.m, m_rows), edges]).astype(np.int64))
        rowbytes = W.k * W.bits // 8
        p = W.packed.view(W.n, rowbytes)[torch.from_numpy(rows).to(W.packed.device)].cpu().numpy()
        sc = W.scales.view(torch.int16).cpu().numpy().view(np.uint16)
        if W.group:
            sc = sc.reshape(W.n, -1)[rows]
        xs = x[torch.from_numpy(ms).to(x.device)].view(torch.int16).cpu().numpy().view(np.uint16)
        zr = None if W.zeros is None else \
            W.zeros.view(torch.int16).cpu().numpy().view(np.uint16).reshape(W.n, -1)[rows]
        if zr is None:
            yref = O.gemm(p, W.bits, sc, W.group, len(rows), W.k, xs, xdt)
        else:
            yref = O.gemm_asym(p, W.bits, sc, zr, len(rows), W.k, xs, xdt)
        got = y[torch.from_numpy(ms).to(y.device)][:, torch.from_numpy(rows).to(y.device)].double().cpu().numpy()
        if xdt == "bf16":
            x64 = torch.from_numpy(xs.view(np.int16)).view(torch.bfloat16).double().numpy()
        else:
            x64 = xs.view(np.float16).astype(np.float64)
        if zr is None:
            wmax = np.abs(O.dequant(O.unpack(p, len(rows), W.k, W.bits), W.group, sc)).max(1)[None, :]
        else:
            wmax = np.abs(O.dequant_asym(O.unpack_u(p, len(rows), W.k, W.bits), sc, zr)).max(1)[None, :]
        tol = 2e-3 * np.sqrt((x64 ** 2).sum(1))[:, None] * wmax + 1e-3 * np.abs(yref)
        err = np.abs(got - yref)
        assert np.all(err <= tol), f"product {idx} (n={W.n}, k={W.k}, bits={W.bits}): " \
                                   f"{int((err > tol).sum())} sampled outputs out of tolerance"


def test_qwen7b_decode_plan(mods):
    bench, zq = mods
    stack = bench.Stack("qwen7b-decode", None, None, torch, zq, synth)
    run_step(bench, stack, "plan")
    check_sampled(stack, seams=split_rows(stack))
    run_step(bench, stack, "plan", order="chained")
    check_sampled(stack, seed=1, seams=split_rows(stack, "chained"))


def test_qwen7b_decode_asym_plan(mods):
    bench, zq = mods
    stack = bench.Stack("qwen7b-decode-asym", None, None, torch, zq, synth)
    run_step(bench, stack, "plan")
    check_sampled(stack, seams=split_rows(stack))


def test_qwen7b_tp4_shard_decode_plan(mods):
    # o and down rows (K = 896, 4736) end in a partial step of the decode kernel
    bench, zq = mods
    stack = bench.Stack("qwen7b-decode-tp4", None, None, torch, zq, synth)
    run_step(bench, stack, "plan")
    check_sampled(stack, seams=split_rows(stack))
    run_step(bench, stack, "plan", order="chained")
    check_sampled(stack, seed=2, seams=split_rows(stack, "chained"))


def test_qwen32b_decode_plan(mods):
    bench, zq = mods
    stack = bench.Stack("qwen32b-decode", None, None, torch, zq, synth)
    run_step(bench, stack, "plan")
    check_sampled(stack, n_rows=4, seams=split_rows(stack))
    del stack
    torch.cuda.empty_cache()


@pytest.mark.parametrize("m", [4, 8, 32, 128, 512])
def test_qwen7b_batch_plan(mods, m):
    # m = 128, 512: group-scaled prefill tiles, one persistent launch
    bench, zq = mods
    stack = bench.Stack("qwen7b-batch", m, None, torch, zq, synth)
    run_step(bench, stack, "plan")
    # past 64 rows: sampled activation rows too (with every 128-row tile edge)
    check_sampled(stack, n_rows=4, m_rows=6 if m > 64 else None, seams=split_rows(stack))


def test_qwen7b_prefill_plan(mods):
    # the bench's default prefill launch: one persistent launch per bit width
    bench, zq = mods
    stack = bench.Stack("qwen7b-prefill", None, None, torch, zq, synth)
    run_step(bench, stack, "plan")
    run_step(bench, stack, "plan")  # the tile counters are back at zero
    check_sampled(stack, n_rows=3, m_rows=3, seed=5, seams=split_rows(stack))
    del stack
    torch.cuda.empty_cache()


def test_qwen7b_prefill_graph_streams(mods):
    bench, zq = mods
    stack = bench.Stack("qwen7b-prefill", None, None, torch, zq, synth)
    run_step(bench, stack, "graph", streams=4)
    check_sampled(stack, n_rows=3, m_rows=3)
    del stack
    torch.cuda.empty_cache()
