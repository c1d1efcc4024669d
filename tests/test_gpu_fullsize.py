"""Parity at the benchmark's full sizes, in the launch configurations bench.py
times, on sampled outputs: for every product of the step, a few weight rows
and activation rows are copied back and recomputed by the fp64 oracle.

    Qwen2.5-7B decode stack   (28 layers x 7, M = 1, INT4 g128, fp16 x), plan
    Qwen2.5-7B decode stack with asymmetric INT4 weights, plan
    one rank's share of the 7B decode stack under 4-way tensor parallelism, plan
    Qwen2.5-32B decode stack  (64 layers x 7, M = 1), plan
    7B stack, M = 4, 8, 32 and 128 (bf16 x), plan (MFMA batched-decode kernel,
    in 32-row chunks past 32)
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


def check_sampled(stack, n_rows=6, m_rows=None, seed=0):
    g = np.random.default_rng(seed)
    xdt = stack.xdt
    for idx, (W, x, y) in enumerate(stack.launches):
        rows = np.unique(np.concatenate([[0, W.n - 1], g.integers(0, W.n, n_rows)]))
        ms = np.arange(stack.m) if m_rows is None else np.unique(
            np.concatenate([[0, stack.m - 1], g.integers(0, stack.m, m_rows)]))
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
    check_sampled(stack)
    run_step(bench, stack, "plan", order="chained")
    check_sampled(stack, seed=1)


def test_qwen7b_decode_asym_plan(mods):
    bench, zq = mods
    stack = bench.Stack("qwen7b-decode-asym", None, None, torch, zq, synth)
    run_step(bench, stack, "plan")
    check_sampled(stack)


def test_qwen7b_tp4_shard_decode_plan(mods):
    # o and down rows (K = 896, 4736) end in a partial step of the decode kernel
    bench, zq = mods
    stack = bench.Stack("qwen7b-decode-tp4", None, None, torch, zq, synth)
    run_step(bench, stack, "plan")
    check_sampled(stack)
    run_step(bench, stack, "plan", order="chained")
    check_sampled(stack, seed=2)


def test_qwen32b_decode_plan(mods):
    bench, zq = mods
    stack = bench.Stack("qwen32b-decode", None, None, torch, zq, synth)
    run_step(bench, stack, "plan")
    check_sampled(stack, n_rows=4)
    del stack
    torch.cuda.empty_cache()


@pytest.mark.parametrize("m", [4, 8, 32, 128])
def test_qwen7b_batch_plan(mods, m):
    # m = 128: four 32-row chunks, each a plan launch over all 196 products
    bench, zq = mods
    stack = bench.Stack("qwen7b-batch", m, None, torch, zq, synth)
    run_step(bench, stack, "plan")
    check_sampled(stack, n_rows=4)


def test_qwen7b_prefill_plan(mods):
    # the bench's default prefill launch: one persistent launch per bit width
    bench, zq = mods
    stack = bench.Stack("qwen7b-prefill", None, None, torch, zq, synth)
    run_step(bench, stack, "plan")
    run_step(bench, stack, "plan")  # the tile counters are back at zero
    check_sampled(stack, n_rows=3, m_rows=3, seed=5)
    del stack
    torch.cuda.empty_cache()


def test_qwen7b_prefill_graph_streams(mods):
    bench, zq = mods
    stack = bench.Stack("qwen7b-prefill", None, None, torch, zq, synth)
    run_step(bench, stack, "graph", streams=4)
    check_sampled(stack, n_rows=3, m_rows=3)
    del stack
    torch.cuda.empty_cache()
