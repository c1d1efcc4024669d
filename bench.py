#!/usr/bin/env python3
"""Throughput of the weight-only quantized linear layer on one MI355X.

Default workload (one "step" = one decode token through a Qwen2.5-7B-shaped
stack): 28 layers x 7 projections (q, k, v, o, gate, up, down), each its own
INT4 group-128 weight and its own activation row, M = 1, fp16 activations,
fp32 outputs; the 196 products of a step run as one plan (one resident
launch). All inputs are synthetic, seeded and resident in HBM before timing
starts.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config qwen7b-decode]

Prints one JSON line. The default run also times, in the same process, the
other workloads of the pages' benchmark set and adds each as a key of its own
(each with its roofline fraction; --no-extras skips them):
  config1_gemv512        the 512 x 512 INT4 GEMV (latency: us per call)
  config3_batch          the 7B stack's weights at M = 1, 4, 8, 16, 32 bf16 rows
  mid_batch_prefill      the same weights at M = 128, 256, 512 (prefill tiles),
                         beside the stack with one scale per tensor
  config4_qwen32b_decode the Qwen2.5-32B-shaped decode stack, M = 1
  config5_prefill        the mixed INT2/4/8 prefill stack, M = 2048 (TFLOP/s)

Other workloads (--config) print their own line:
  gemv-512             single 512 x 512 INT4 GEMV, per-tensor scale fp16(0.02)
  qwen7b-batch --m M   the 7B stack at M rows of bf16 activations (M <= 32: one
                       plan launch; 32 < M <= 64: 32-row chunks of it; M > 64:
                       prefill tiles)
  qwen7b-batch-tensor --m M   the same shapes, INT4 with one scale per tensor
  qwen32b-decode       64 layers of Qwen2.5-32B projection shapes, M = 1
  qwen7b-decode-asym   the 7B decode stack with asymmetric INT4 weights (unsigned
                       codes, fp16 scale and zero point per 128-group)
  qwen7b-decode-tp4    one rank's shard of the 7B decode stack under 4-way tensor
                       parallelism (q/k/v/gate/up split by rows, o/down by
                       columns: K = 896 and 4736 rows end in a partial step)
  qwen7b-prefill       7B stack, bits per layer from {2,4,8}, per-tensor scales,
                       M = 2048 bf16 tokens (MFMA-bound: TFLOP/s)
  hbm-copy             a plain 1 GiB device-to-device copy (torch), the
                       measured copy ceiling and the byte-counter calibration
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys
import threading
import time

import numpy as np

HBM_PEAK_GBS = 8000.0        # MI355X HBM3E, 8 TB/s
MFMA_BF16_PEAK_TFS = 2500.0  # MI355X dense bf16 MFMA, 2.5 PFLOP/s
METRIC = "weight GB/s and % HBM roofline (M=1 INT4 GEMV); decode tok/s equiv for 7B/32B stacks"
SETTLE_S = 0.3               # untimed streaming before the warmup steps: clocks ramp over ~30 ms

# HBM bytes per launch of the plan kernel from two rocprofv3 --pmc runs
# (FETCH_SIZE, then WRITE_SIZE), each scaled by what that counter reads for a
# 1 GiB device copy (FETCH_SIZE x 2.0, WRITE_SIZE x 1.0); the summary and the
# commands are in profiles/gemv_stream_qwen7b*_m1.md. A figure holds only
# for the kernel sources it was taken with (sha256 of KERNEL_SOURCES, first 16
# hex digits); for any other source the bench reports traffic as null.
KERNEL_SOURCES = ("weight_quantized_amd/csrc/zq_stream_impl.hpp", "weight_quantized_amd/csrc/zq_device.hpp",
                  "weight_quantized_amd/csrc/zq_internal.hpp", "weight_quantized_amd/csrc/zq_stream_m1.hip",
                  "weight_quantized_amd/csrc/zq_stream.hip")
TRAFFIC = {("qwen7b-decode", 1, "plan", "independent"): (3392038503, "b926738c247dca46"),
           ("qwen7b-decode-tp4", 1, "plan", "independent"): (879137178, "b926738c247dca46"),
           ("qwen7b-decode-asym", 1, "plan", "independent"): (3499875328, "b926738c247dca46")}


def kernel_source_hash() -> str:
    import hashlib
    h = hashlib.sha256()
    root = os.path.dirname(os.path.abspath(__file__))
    for f in KERNEL_SOURCES:
        with open(os.path.join(root, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--config", default="qwen7b-decode",
                   choices=["gemv-512", "qwen7b-decode", "qwen7b-batch", "qwen7b-batch-tensor", "qwen32b-decode",
                            "qwen7b-prefill", "qwen7b-decode-asym", "qwen7b-decode-tp4", "hbm-copy"])
    p.add_argument("--m", type=int, default=None, help="activation rows (qwen7b-batch)")
    p.add_argument("--launch", default=None, choices=["plan", "graph", "eager"],
                   help="plan (the default): one resident launch per step (m <= 32), or one "
                        "persistent launch per bit width over a tile queue (prefill); "
                        "graph: the per-projection launches replayed as a HIP graph")
    p.add_argument("--order", default="independent", choices=["chained", "independent"],
                   help="plan phases: independent = every product of the step at once (each has its "
                        "own activations); chained = q,k,v -> o -> gate,up -> down per layer, each "
                        "phase waiting for the previous one, as a decoder's data flow would")
    p.add_argument("--streams", type=int, default=None,
                   help="graph launch: spread the step's independent products over this many streams "
                        "inside the captured graph, so small kernels run side by side (default 4 for "
                        "prefill, 1 otherwise)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-extras", action="store_true",
                   help="default workload only: skip the other workloads' keys")
    p.add_argument("--layers", type=int, default=None, help="override the layer count (profiling)")
    return p.parse_args()


class Stack:
    """Device-resident weights, activations and outputs of one workload."""

    def __init__(self, cfg: str, m: int | None, layers: int | None, torch, zq, synth):
        self.cfg, self.torch, self.zq = cfg, torch, zq
        dev = torch.device("cuda:0")
        if cfg == "gemv-512":
            shapes, L, bits_of, group, xdt, self.m = [("w", 512, 512)], 1, (lambda l: 4), 0, "f16", 1
        elif cfg in ("qwen7b-decode", "qwen7b-decode-asym"):
            shapes, L, bits_of, group, xdt, self.m = synth.QWEN25_7B, 28, (lambda l: 4), 128, "f16", 1
        elif cfg == "qwen7b-decode-tp4":
            shapes, L, bits_of, group, xdt, self.m = synth.QWEN25_7B_TP4, 28, (lambda l: 4), 128, "f16", 1
        elif cfg == "qwen7b-batch":
            shapes, L, bits_of, group, xdt, self.m = synth.QWEN25_7B, 28, (lambda l: 4), 128, "bf16", m or 8
        elif cfg == "qwen7b-batch-tensor":  # the same shapes, INT4 with one scale per tensor
            shapes, L, bits_of, group, xdt, self.m = synth.QWEN25_7B, 28, (lambda l: 4), 0, "bf16", m or 128
        elif cfg == "qwen32b-decode":
            shapes, L, bits_of, group, xdt, self.m = synth.QWEN25_32B, 64, (lambda l: 4), 128, "f16", 1
        else:
            shapes, L, bits_of, group, xdt, self.m = (synth.QWEN25_7B, 28, (lambda l: synth.layer_bits(5, l)),
                                                      0, "bf16", 2048)
        if layers:
            L = layers
        self.layers, self.shapes, self.group, self.xdt = L, shapes, group, xdt
        self.launches = []   # (zq_weight, x tensor, y tensor)
        self.weight_bytes = 0
        self.flops = 0
        seed = 0
        for l in range(L):
            bits = bits_of(l)
            for name, n, k in shapes:
                seed += 1
                packed = synth.device_uniform_bytes(n * k * bits // 8, 1000003 * seed, dev)
                ns = 1 if group == 0 else n * k // 128
                if cfg == "gemv-512":
                    scales = torch.tensor([0.02], dtype=torch.float16, device=dev)
                else:
                    scales = synth.device_scales_abs_normal(ns, 2000003 * seed, dev)
                x = synth.device_normal((self.m, k), xdt, 3000003 * seed, dev)
                y = torch.empty((self.m, n), dtype=torch.float32, device=dev)
                zeros = synth.device_zeros_normal(ns, 4000003 * seed, dev) if cfg.endswith("-asym") else None
                W = zq.ZqWeight(bits, group, n, k, packed, scales, zeros)
                self.launches.append((W, x, y))
                self.weight_bytes += W.nbytes
                self.flops += 2 * self.m * n * k
        torch.cuda.synchronize()
        L_ = zq.lib()
        self._fn = L_.zq_gemm
        self._descs = [W.desc() for W, _, _ in self.launches]
        xt = zq.F16 if xdt == "f16" else zq.BF16
        self._args = [(ctypes.byref(d), x.data_ptr(), xt, self.m, x.stride(0), y.data_ptr(), zq.F32,
                       y.stride(0)) for d, (_, x, y) in zip(self._descs, self.launches)]
        self.plan = None

    def with_rows(self, m: int, xdt: str):
        """the same weights with fresh activations of m rows in xdt (and fp32
        outputs): a Stack sharing this one's weight tensors"""
        torch, zq = self.torch, self.zq
        from weight_quantized_amd import synth
        other = object.__new__(Stack)
        other.__dict__.update({k: v for k, v in self.__dict__.items() if k not in ("launches", "plan")})
        other.m, other.xdt, other.plan = m, xdt, None
        other.launches, other.flops = [], 0
        dev = torch.device("cuda:0")
        for i, (W, _, _) in enumerate(self.launches):
            x = synth.device_normal((m, W.k), xdt, 5000003 * (i + 1) + m, dev)
            y = torch.empty((m, W.n), dtype=torch.float32, device=dev)
            other.launches.append((W, x, y))
            other.flops += 2 * m * W.n * W.k
        torch.cuda.synchronize()
        return other

    def close(self):
        if self.plan is not None:
            self.plan.close()
            self.plan = None

    def make_plan(self, order: str):
        """one resident launch per step. chained: the decoder-layer phases
        q,k,v -> o -> gate,up -> down, each waiting for the previous phase;
        independent: every product of the step in one phase, in an order that
        groups equal K (all q,k,v,o,gate,up of the step, then all down)."""
        phase_of = {"q": 0, "k": 0, "v": 0, "o": 1, "gate": 2, "up": 2, "down": 3, "w": 0}
        per_layer = len(self.shapes)
        items = []
        for i, (W, x, y) in enumerate(self.launches):
            l, name = divmod(i, per_layer)
            items.append((l, name, (W, x, y)))
        if order == "chained":
            probs = [(W, x, y, 4 * l + phase_of[self.shapes[nm][0]]) for l, nm, (W, x, y) in items]
        else:
            items.sort(key=lambda t: (t[2][0].k, t[0], t[1]))
            probs = [(W, x, y, 0) for l, nm, (W, x, y) in items]
        self.plan = self.zq.Plan(probs)

    def plan_step(self):
        self.plan.run()

    def step(self, streams=None):
        """every product of the step; with `streams`, product i goes to stream
        i % len(streams) (forked from and joined back to the current stream)"""
        torch = self.torch
        fn = self._fn
        if not streams:
            s = torch.cuda.current_stream().cuda_stream
            for a in self._args:
                st = fn(*a, s)
                if st:
                    raise RuntimeError(f"zq_gemm failed: {self.zq.lib().zq_last_error().decode()}")
            return
        cur = torch.cuda.current_stream()
        fork = torch.cuda.Event()
        fork.record(cur)
        for sm in streams:
            sm.wait_event(fork)
        # largest products first, dealt round-robin
        order = sorted(range(len(self._args)), key=lambda i: -self.launches[i][0].n * self.launches[i][0].k)
        for pos, i in enumerate(order):
            sm = streams[pos % len(streams)]
            st = fn(*self._args[i], sm.cuda_stream)
            if st:
                raise RuntimeError(f"zq_gemm failed: {self.zq.lib().zq_last_error().decode()}")
        for sm in streams:
            join = torch.cuda.Event()
            join.record(sm)
            cur.wait_event(join)

    def step_timed_launches(self, ev):
        """eager step with an event pair around every launch"""
        s = self.torch.cuda.current_stream().cuda_stream
        fn = self._fn
        for a in self._args:
            e0, e1 = ev()
            e0.record()
            fn(*a, s)
            e1.record()
            yield e0, e1


def _host_threads():
    """(threads to use, nproc): the oracle runs on the CPU share this process
    is given -- OMP_NUM_THREADS when set (a GPU machine gives each GPU's jobs 16
    host threads, whatever nproc shows), else every core of its affinity set"""
    nproc = len(os.sched_getaffinity(0))
    try:
        share = int(os.environ.get("OMP_NUM_THREADS", "0"))
    except ValueError:
        share = 0
    return (min(share, nproc) if share > 0 else nproc), nproc


def _oracle_jobs(stack: Stack, layer: int, threads: int, xrows: int, torch):
    """one layer's products split by rows into `threads` lists of oracle calls"""
    per_layer = len(stack.shapes)
    jobs = []
    for W, x, _ in stack.launches[layer * per_layer:(layer + 1) * per_layer]:
        p = W.packed.cpu().numpy().reshape(W.n, -1)
        sc = W.scales.view(torch.int16).cpu().numpy().view(np.uint16)
        zz = None if W.zeros is None else W.zeros.view(torch.int16).cpu().numpy().view(np.uint16).reshape(W.n, -1)
        xh = x[:xrows].view(torch.int16).cpu().numpy().view(np.uint16)
        bounds = np.linspace(0, W.n, threads + 1).astype(np.int64)
        for t in range(threads):
            r0, r1 = int(bounds[t]), int(bounds[t + 1])
            if r1 > r0:
                s_rows = sc if W.group == 0 else sc.reshape(W.n, -1)[r0:r1]
                z_rows = None if zz is None else zz[r0:r1]
                jobs.append((p[r0:r1], W.bits, s_rows, z_rows, W.group, r1 - r0, W.k, xh, stack.xdt))
    return [jobs[i::threads] for i in range(threads)]


def _run_oracle(per_thread):
    from oracle import oracle as O

    def work(js):
        for (pp, bits, ss, zz, grp, n, k, xh_, xd) in js:
            if zz is None:
                O.gemm(pp, bits, ss, grp, n, k, xh_, xd)
            else:
                O.gemm_asym(pp, bits, ss, zz, n, k, xh_, xd)

    ths = [threading.Thread(target=work, args=(js,)) for js in per_thread]
    t0, c0 = time.perf_counter(), time.process_time()
    for t in ths:
        t.start()
    for t in ths:
        t.join()
    return time.perf_counter() - t0, time.process_time() - c0


def cpu_baseline(stack: Stack, torch, synth, budget_s: float = 12.0):
    """The fp64 oracle, as it stands, on the host over a bounded sample of the
    same stack: one thread on the first layer, then the thread share on as
    many layers as about `budget_s` CPU-seconds take. The oracle releases the
    GIL (a C library through ctypes), so threads run in parallel."""
    threads, nproc = _host_threads()
    per_layer = len(stack.shapes)
    xrows = min(stack.m, 16)  # prefill: 16 token rows (the work is linear in m)
    layer_bytes = [sum(W.nbytes for W, _, _ in stack.launches[l * per_layer:(l + 1) * per_layer])
                   for l in range(stack.layers)]
    layer_flops = [sum(2 * xrows * W.n * W.k for W, _, _ in stack.launches[l * per_layer:(l + 1) * per_layer])
                   for l in range(stack.layers)]
    prefill = stack.cfg == "qwen7b-prefill"

    def rate(layers, wall):
        return (sum(layer_flops[:layers]) / wall / 1e12) if prefill else (sum(layer_bytes[:layers]) / wall / 1e9)

    wall1, cpu1 = _run_oracle(_oracle_jobs(stack, 0, 1, xrows, torch))
    walls, cpus, used = [], 0.0, 0
    for l in range(stack.layers):
        w, c = _run_oracle(_oracle_jobs(stack, l, threads, xrows, torch))
        walls.append(w)
        cpus += c
        used += 1
        if cpus >= budget_s:
            break
    v_all, v_1 = rate(used, sum(walls)), rate(1, wall1)
    cpu_model = ""
    try:
        with open("/proc/cpuinfo") as fh:
            cpu_model = next((ln.split(":", 1)[1].strip() for ln in fh if ln.startswith("model name")), "")
    except OSError:
        pass
    unit = "TFLOP/s" if prefill else "GB/s"
    return {"value": round(v_all, 4), "unit": unit, "cores": threads, "kind": "oracle",
            "nproc": nproc, "os_cpu_count": os.cpu_count(), "cpu_model": cpu_model,
            "threads_1": {"value": round(v_1, 4), "unit": unit, "threads": 1,
                          "sample": f"layer 0 (all {per_layer} projections, m={xrows} of {stack.m}), "
                                    f"{wall1:.2f} s wall"},
            "threads_all": {"value": round(v_all, 4), "unit": unit, "threads": threads,
                            "sample": f"first {used} of {stack.layers} layers, {cpus:.1f} CPU-s over "
                                      f"{sum(walls):.2f} s wall"},
            "sample": f"first {used} of {stack.layers} layers (all {per_layer} projections, m={xrows} of "
                      f"{stack.m}) on {threads} threads (the host thread share; nproc {nproc}), "
                      f"{cpus:.1f} CPU-s over {sum(walls):.2f} s wall"}


def copy_bench(a, torch):
    """dst.copy_(src) of 1 GiB: read 1 GiB + write 1 GiB per step."""
    nbytes = 1 << 30
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda:0").random_(0, 256)
    dst = torch.empty_like(src)
    for _ in range(a.warmup):
        dst.copy_(src)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(a.steps):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / a.steps
    gbs = 2 * nbytes / (ms * 1e-3) / 1e9
    print(json.dumps({"metric": "device copy GB/s (read + write)", "value": round(gbs, 1), "unit": "GB/s",
                      "n_gpus": 1, "steps": a.steps, "warmup": a.warmup, "ms_per_step": round(ms, 5),
                      "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "u8",
                      "data": "synthetic", "config": {"workload": "1 GiB device-to-device copy",
                                                      "bytes_read": nbytes, "bytes_written": nbytes}}),
          flush=True)


def measure(run, steps: int, warmup: int, torch, settle_s: float = SETTLE_S) -> dict:
    """untimed settle and warmup, then exactly `steps` runs between two device
    synchronisations; an event before every run gives per-step times"""
    t_settle = time.perf_counter()
    while time.perf_counter() - t_settle < settle_s:
        run()
        torch.cuda.synchronize()
    for _ in range(warmup):
        run()
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    w0 = time.perf_counter()
    for i in range(steps):
        ev[i].record()
        run()
    ev[steps].record()
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - w0) * 1e3 / steps
    per = np.array([ev[i].elapsed_time(ev[i + 1]) for i in range(steps)])
    # a plan run is one resident launch (decode) or one launch per bit width
    # (prefill): the per-step intervals of the timed region are its durations
    return {"ms": ev[0].elapsed_time(ev[steps]) / steps, "ms_median": float(np.median(per)),
            "ms_mean_of_steps": float(per.mean()), "wall_ms": wall_ms}


def decode_figures(stack: Stack, t: dict, kern_ms: float) -> dict:
    """a decode workload's step time in the four forms (GB/s, us per layer,
    tok/s equivalent, fraction of the HBM roofline)"""
    gbs = stack.weight_bytes / (t["ms"] * 1e-3) / 1e9
    kern_gbs = stack.weight_bytes / (kern_ms * 1e-3) / 1e9
    return {"value": round(gbs, 1), "unit": "GB/s", "hbm_frac": round(gbs / HBM_PEAK_GBS, 4),
            "ms_per_step": round(t["ms"], 5), "ms_per_step_median": round(t["ms_median"], 5),
            "us_per_layer": round(t["ms"] * 1e3 / stack.layers, 3),
            "tok_s_equiv": round(stack.m / (t["ms"] * 1e-3), 1),
            "tflop_s": round(stack.flops / (t["ms"] * 1e-3) / 1e12, 2),
            "roofline": {"bound": "hbm", "achieved": round(kern_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": round(kern_gbs / HBM_PEAK_GBS, 4)},
            "weight_bytes_per_step": stack.weight_bytes, "layers": stack.layers, "m": stack.m,
            "avg_kernel_us": round(kern_ms * 1e3, 3)}


def prefill_figures(stack: Stack, t: dict, kern_ms: float) -> dict:
    tfs = stack.flops / (t["ms"] * 1e-3) / 1e12
    kern_tfs = stack.flops / (kern_ms * 1e-3) / 1e12
    return {"value": round(tfs, 2), "unit": "TFLOP/s", "mfma_frac": round(tfs / MFMA_BF16_PEAK_TFS, 4),
            "ms_per_step": round(t["ms"], 5), "ms_per_step_median": round(t["ms_median"], 5),
            "us_per_layer": round(t["ms"] * 1e3 / stack.layers, 2),
            "tok_s_equiv": round(stack.m / (t["ms"] * 1e-3), 1),
            "roofline": {"bound": "mfma", "achieved": round(kern_tfs, 2), "peak": MFMA_BF16_PEAK_TFS,
                         "unit": "TFLOP/s", "frac": round(kern_tfs / MFMA_BF16_PEAK_TFS, 4)},
            "flops_per_step": stack.flops, "layers": stack.layers, "m": stack.m,
            "bits_per_layer": [stack.launches[l * len(stack.shapes)][0].bits for l in range(stack.layers)],
            "avg_plan_run_us": round(kern_ms * 1e3, 1)}


def extras(a, base: Stack, torch, zq, synth) -> dict:
    """the other workloads, each timed as a plan (steps scaled to about a
    second of GPU time each), with their roofline fractions"""
    out = {}
    # config 1: the 512 x 512 GEMV, latency-bound (131 KB fit in L2)
    st = Stack("gemv-512", None, None, torch, zq, synth)
    st.make_plan("independent")
    t = measure(st.plan_step, 2000, 50, torch, settle_s=0.05)
    kern = t["ms_mean_of_steps"]
    f = decode_figures(st, t, kern)
    # back-to-back calls: the interval between launches, not the kernel's own
    # duration (about 7 us by trace), is the figure
    out["config1_gemv512"] = {"us_per_call": round(t["ms"] * 1e3, 3),
                              "us_per_call_median": round(t["ms_median"] * 1e3, 3),
                              "value": f["value"], "unit": "GB/s",
                              "roofline": {"bound": "latency", "note": "131,074 weight bytes fit in L2; "
                                           "µs per call is the figure", "hbm_frac": f["hbm_frac"]},
                              "workload": "512x512 INT4, per-tensor fp16(0.02), M=1, fp16 x, plan launches "
                                          "back to back"}
    st.close()
    del st
    # config 3: config 2's weights under continuous batching, bf16 rows
    batch = {}
    for m in (1, 4, 8, 16, 32):
        st = base.with_rows(m, "bf16")
        st.make_plan("independent")
        t = measure(st.plan_step, 40, 3, torch, settle_s=0.05)
        f = decode_figures(st, t, t["ms_mean_of_steps"])
        batch[f"m{m}"] = {k: f[k] for k in ("value", "unit", "hbm_frac", "us_per_layer", "tok_s_equiv", "tflop_s",
                                            "ms_per_step", "ms_per_step_median", "roofline")}
        st.close()
        del st
    out["config3_batch"] = {"workload": "Qwen2.5-7B-shaped stack (config 2's weights), INT4 group-128, bf16 x, "
                                        "one plan per M", "by_m": batch}
    torch.cuda.empty_cache()
    # past 64 rows (prefill tiles): config 2's group-128 weights beside the
    # same stack with one scale per tensor
    mid = {}
    pt = Stack("qwen7b-batch-tensor", 128, None, torch, zq, synth)
    for m in (128, 256, 512):
        row = {}
        for kind, src in (("group128", base), ("per_tensor", pt)):
            st = src.with_rows(m, "bf16")
            st.make_plan("independent")
            t = measure(st.plan_step, 20, 3, torch, settle_s=0.05)
            f = prefill_figures(st, t, t["ms_mean_of_steps"])
            row[kind] = {k: f[k] for k in ("value", "unit", "mfma_frac", "us_per_layer", "ms_per_step_median")}
            st.close()
            del st
        row["group_over_tensor_time"] = round(row["group128"]["us_per_layer"] / row["per_tensor"]["us_per_layer"], 4)
        mid[f"m{m}"] = row
    pt.close()
    del pt
    out["mid_batch_prefill"] = {"workload": "Qwen2.5-7B-shaped stack, INT4, bf16 x, one prefill plan per M: "
                                            "group-128 scales (config 2's weights) and one scale per tensor",
                                "by_m": mid}
    torch.cuda.empty_cache()
    # config 4: the 32B stack (16.09 GB of weights)
    st = Stack("qwen32b-decode", None, None, torch, zq, synth)
    st.make_plan("independent")
    t = measure(st.plan_step, 100, 5, torch)
    f = decode_figures(st, t, t["ms_mean_of_steps"])
    f["workload"] = "Qwen2.5-32B-shaped decode stack: 64 layers x 7 projections, M=1, INT4 group-128, fp16 x"
    out["config4_qwen32b_decode"] = f
    st.close()
    del st
    torch.cuda.empty_cache()
    # config 5: mixed-precision prefill, M = 2048
    st = Stack("qwen7b-prefill", None, None, torch, zq, synth)
    st.make_plan("independent")
    t = measure(st.plan_step, 10, 2, torch)
    f = prefill_figures(st, t, t["ms_mean_of_steps"])
    f["workload"] = ("Qwen2.5-7B-shaped prefill stack, per-layer INT2/INT4/INT8 (seeded), per-tensor scale, "
                     "M=2048, bf16 x, one prefill plan")
    out["config5_prefill"] = f
    st.close()
    del st
    torch.cuda.empty_cache()
    return out


def main():
    a = parse()
    if a.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {a.gpus} is not supported", file=sys.stderr)
        sys.exit(2)
    import torch
    from weight_quantized_amd import synth, zq
    zq.lib()
    if a.config == "hbm-copy":
        copy_bench(a, torch)
        return
    if a.config == "qwen7b-prefill" and a.steps == 50:
        a.steps = 10
    stack = Stack(a.config, a.m, a.layers, torch, zq, synth)

    if a.launch is None:
        a.launch = "plan"  # m <= 32: the decode kernels; m > 64: the prefill tile queue
    # ---- timed region
    graph = None
    if a.launch == "plan":
        stack.make_plan(a.order)
        run = stack.plan_step
    elif a.launch == "graph":
        if a.streams is None:
            a.streams = 4 if a.config == "qwen7b-prefill" else 1
        streams = [torch.cuda.Stream() for _ in range(a.streams)] if a.streams > 1 else None
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            stack.step(streams)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            stack.step(streams)
        run = graph.replay
    else:
        run = stack.step
    t = measure(run, a.steps, a.warmup, torch)
    ms = t["ms"]

    # ---- per-launch kernel durations (event pairs on the launch stream)
    if a.launch == "plan":
        avg_launch_ms = t["ms_mean_of_steps"]  # the plan's resident launch, one per step
        launches = 1
        stack.plan.check()
    else:
        torch.cuda.synchronize()
        pairs = []
        mk = lambda: (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
        for _ in range(max(1, min(a.steps, 20))):
            pairs.extend(stack.step_timed_launches(mk))
        torch.cuda.synchronize()
        avg_launch_ms = float(np.mean([p0.elapsed_time(p1) for p0, p1 in pairs]))
        launches = len(stack.launches)

    out = {"metric": METRIC, "n_gpus": 1, "steps": a.steps, "warmup": a.warmup,
           "ms_per_step": round(ms, 5), "ms_per_step_median": round(t["ms_median"], 5),
           "higher_is_better": True, "scaling": "weak",
           "vs_baseline": None, "dtype": "f16" if stack.xdt == "f16" else "bf16", "data": "synthetic"}
    per_layer_us = ms * 1e3 / stack.layers
    if a.config == "qwen7b-prefill":
        tfs = stack.flops / (ms * 1e-3) / 1e12
        kern_tfs = (stack.flops / launches) / (avg_launch_ms * 1e-3) / 1e12
        out.update({"metric": "prefill TFLOP/s and % bf16 MFMA roofline (mixed INT2/4/8 stack, M=2048)",
                    "value": round(tfs, 2), "unit": "TFLOP/s",
                    "mfma_frac": round(tfs / MFMA_BF16_PEAK_TFS, 4),
                    "us_per_layer": round(per_layer_us, 2),
                    "roofline": {"bound": "mfma", "achieved": round(kern_tfs, 2), "peak": MFMA_BF16_PEAK_TFS,
                                 "unit": "TFLOP/s", "frac": round(kern_tfs / MFMA_BF16_PEAK_TFS, 4),
                                 "traffic": None}})
    else:
        gbs = stack.weight_bytes / (ms * 1e-3) / 1e9
        kern_gbs = (stack.weight_bytes / launches) / (avg_launch_ms * 1e-3) / 1e9
        tr = TRAFFIC.get((a.config, stack.m, a.launch, a.order if a.launch == "plan" else "stream"))
        traffic = tr[0] if tr and a.layers is None and tr[1] == kernel_source_hash() else None
        out.update({"value": round(gbs, 1), "unit": "GB/s", "hbm_frac": round(gbs / HBM_PEAK_GBS, 4),
                    "us_per_layer": round(per_layer_us, 3),
                    "tok_s_equiv": round(stack.m / (ms * 1e-3), 1),
                    "tflop_s": round(stack.flops / (ms * 1e-3) / 1e12, 2),
                    "roofline": {"bound": "hbm", "achieved": round(kern_gbs, 1), "peak": HBM_PEAK_GBS,
                                 "unit": "GB/s", "frac": round(kern_gbs / HBM_PEAK_GBS, 4),
                                 "traffic": traffic},
                    "roofline_bytes_per_launch": stack.weight_bytes // launches})
    out["config"] = {"workload": {
        "gemv-512": "single 512x512 INT4 GEMV, per-tensor fp16 scale 0.02, M=1, fp16 x",
        "qwen7b-decode": "Qwen2.5-7B-shaped decode stack: 28 layers x 7 projections, M=1, INT4 group-128, fp16 x",
        "qwen7b-decode-asym": "Qwen2.5-7B-shaped decode stack: 28 layers x 7 projections, M=1, asymmetric INT4 "
                              "(fp16 scale and zero point per 128-group), fp16 x",
        "qwen7b-decode-tp4": "one rank's 4-way tensor-parallel shard of the Qwen2.5-7B decode stack: 28 layers "
                             "x 7 projections, M=1, INT4 group-128, fp16 x",
        "qwen7b-batch": f"Qwen2.5-7B-shaped stack, M={stack.m}, INT4 group-128, bf16 x",
        "qwen7b-batch-tensor": f"Qwen2.5-7B-shaped stack, M={stack.m}, INT4 one scale per tensor, bf16 x",
        "qwen32b-decode": "Qwen2.5-32B-shaped decode stack: 64 layers x 7 projections, M=1, INT4 group-128, fp16 x",
        "qwen7b-prefill": "Qwen2.5-7B-shaped prefill stack, per-layer INT2/INT4/INT8, per-tensor scale, M=2048, bf16 x",
    }[a.config], "layers": stack.layers, "m": stack.m,
        "weight_bytes_per_step": stack.weight_bytes, "launch": a.launch, "order": a.order if a.launch == "plan" else "stream",
        "launches_per_step": 1 if a.launch == "plan" else len(stack.launches),
        # kernels one plan run enqueues: one per bit width and scale kind
        # (prefill tile queues), one per 32-row chunk (32 < m <= 64 on the
        # batched-decode kernel)
        "kernels_per_plan_run": (len({(W.bits, W.group) for W, _, _ in stack.launches}) if stack.m > 64
                                 else -(-stack.m // 32) if stack.m > 32 else 1) if a.launch == "plan" else None,
        "wall_ms_per_step": round(t["wall_ms"], 5), "avg_kernel_us": round(avg_launch_ms * 1e3, 3),
        "streams": a.streams if a.launch == "graph" else 1,
        "settle_s": SETTLE_S}
    if not a.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(stack, torch, synth)
    if a.config == "qwen7b-decode" and a.launch == "plan" and a.layers is None and not a.no_extras:
        out.update(extras(a, stack, torch, zq, synth))
    stack.close()
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
