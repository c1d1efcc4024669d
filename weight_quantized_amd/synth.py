"""Seeded synthetic inputs shared by the tests, the oracle checks and the bench.

This module holds no step of the quantized linear layer: it only draws
random codes, scales and activations with the laws of the workloads, and the
projection shapes of the Qwen2.5-7B / 32B decode layers that the ZSE pages
benchmark (ZSE wiki, section "Производительность: заявленные цифры"; no trained
weights are used anywhere).

Laws (one per workload):
  - codes: uniform over the full signed range of b bits, [-2^(b-1), 2^(b-1)-1];
  - group or tensor scales: |N(0,1)| * 0.01 + 1e-3 drawn in float32, then
    rounded to float16 by numpy (round to nearest even);
  - activations: N(0,1) drawn in float32, then rounded to float16 (numpy) or
    bfloat16 (torch, round to nearest even).
For whole-stack sizes the packed bytes are drawn on the device as independent
uniform bytes: every b-bit field of a uniform byte is itself uniform over its
2^b values and independent of the other fields, so this is the same code law.
"""
from __future__ import annotations

import numpy as np

# (name, N = output features, K = input features), nn.Linear storage [N][K].
QWEN25_7B = [
    ("q", 3584, 3584), ("k", 512, 3584), ("v", 512, 3584), ("o", 3584, 3584),
    ("gate", 18944, 3584), ("up", 18944, 3584), ("down", 3584, 18944),
]
QWEN25_7B_LAYERS = 28
# one rank's share of the 7B projections under 4-way tensor parallelism:
# q, k, v, gate, up split by output rows, o and down by input columns
QWEN25_7B_TP4 = [
    ("q", 896, 3584), ("k", 128, 3584), ("v", 128, 3584), ("o", 3584, 896),
    ("gate", 4736, 3584), ("up", 4736, 3584), ("down", 3584, 4736),
]
QWEN25_32B = [
    ("q", 5120, 5120), ("k", 1024, 5120), ("v", 1024, 5120), ("o", 5120, 5120),
    ("gate", 27648, 5120), ("up", 27648, 5120), ("down", 5120, 27648),
]
QWEN25_32B_LAYERS = 64


def rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def codes_uniform(g: np.random.Generator, n: int, k: int, bits: int) -> np.ndarray:
    lo, hi = -(1 << (bits - 1)), (1 << (bits - 1))
    return g.integers(lo, hi, size=(n, k), dtype=np.int8)


def scales_abs_normal(g: np.random.Generator, count: int) -> np.ndarray:
    """float16 bit patterns of |N(0,1)| * 0.01 + 1e-3."""
    v = np.abs(g.standard_normal(count, dtype=np.float32)) * np.float32(0.01) + np.float32(1e-3)
    return v.astype(np.float16).view(np.uint16)


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def normal(g: np.random.Generator, shape, dtype: str) -> np.ndarray:
    """N(0,1) activations: np.float16 for "f16", uint16 bf16 bits for "bf16", np.float32 for "f32"."""
    v = g.standard_normal(shape, dtype=np.float32)
    if dtype == "f16":
        return v.astype(np.float16)
    if dtype == "bf16":
        return f32_to_bf16_bits(v)
    if dtype == "f32":
        return v
    raise ValueError(dtype)


def layer_bits(seed: int, layer: int) -> int:
    """Bit width of one layer of the mixed-precision stack, uniform over {2, 4, 8}."""
    return int(rng(seed * 1000 + layer).choice(np.array([2, 4, 8])))


def device_uniform_bytes(nbytes: int, seed: int, device):
    """Independent uniform bytes drawn on `device` with a seeded torch generator."""
    import torch
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    return torch.randint(0, 256, (nbytes,), dtype=torch.uint8, device=device, generator=gen)


def device_normal(shape, dtype: str, seed: int, device):
    """N(0,1) drawn on `device` in float32 with a seeded torch generator, then rounded."""
    import torch
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    v = torch.randn(shape, dtype=torch.float32, device=device, generator=gen)
    return v.to({"f16": torch.float16, "bf16": torch.bfloat16, "f32": torch.float32}[dtype])


def device_scales_abs_normal(count: int, seed: int, device):
    """float16 |N(0,1)| * 0.01 + 1e-3 drawn on `device`."""
    import torch
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    v = torch.randn(count, dtype=torch.float32, device=device, generator=gen)
    return (v.abs() * 0.01 + 1e-3).to(torch.float16)


def device_zeros_normal(count: int, seed: int, device):
    """float16 N(0,1) * 0.01 zero points (asymmetric weights) drawn on `device`."""
    import torch
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    v = torch.randn(count, generator=gen, device=device, dtype=torch.float32) * 0.01
    return v.to(torch.float16)
