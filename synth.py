"""Seeded synthetic inputs shared by the tests, the bench and the smoke check.

This module holds none of the method's arithmetic: it only draws random numbers
and rounds them to bf16 (or fp16, for the fp16 compute type) with torch's own
float32 -> bfloat16 / float16 conversion (round to nearest even), so that the
CPU oracle and the HIP path receive identical bits.

Recipe (every tensor): numpy ``default_rng(PCG64)`` seeded with
``1000 * config + tensor_index``, drawn in float64, cast to float32, then to bf16.
Weights are N(0, sigma) (sigma = 0.02, or 0.015 with a 0.1 % Bernoulli outlier
mask scaled by 20 before rounding); activations and upstream gradients N(0, 1);
LoRA A and B N(0, 0.01).  The second argument of N(mu, sigma) is the standard
deviation.

Tensors too large to stage on the host (the 32-layer decode sweep) are drawn on
the device with a seeded ``torch.Generator`` instead (``device_normal_bf16``).
"""
from __future__ import annotations

import numpy as np
import torch

__all__ = [
    "rng", "normal_bf16", "normal_f16", "normal_16", "bf16_bits_to_f32", "device_normal_bf16",
    "tensor_seed",
]


def tensor_seed(config: int, index: int) -> int:
    """Seed of tensor ``index`` of workload ``config``."""
    return 1000 * int(config) + int(index)


def rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def _f32_to_bf16_bits_torch(a32: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(a32, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()


def normal_bf16(shape, sigma: float, seed: int, outlier_rate: float = 0.0,
                outlier_scale: float = 1.0) -> np.ndarray:
    """bf16 bit patterns (uint16) of N(0, sigma) draws, optionally with a
    Bernoulli(outlier_rate) mask whose entries are multiplied by outlier_scale."""
    g = rng(seed)
    x = g.standard_normal(size=shape) * sigma
    if outlier_rate > 0.0:
        mask = g.random(size=shape) < outlier_rate
        x = np.where(mask, x * outlier_scale, x)
    return _f32_to_bf16_bits_torch(x.astype(np.float32))


def normal_f16(shape, sigma: float, seed: int, outlier_rate: float = 0.0,
               outlier_scale: float = 1.0) -> np.ndarray:
    """fp16 bit patterns (uint16) of the same draws as ``normal_bf16``."""
    g = rng(seed)
    x = g.standard_normal(size=shape) * sigma
    if outlier_rate > 0.0:
        mask = g.random(size=shape) < outlier_rate
        x = np.where(mask, x * outlier_scale, x)
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.float16).view(torch.int16).numpy().view(np.uint16).copy()


def normal_16(dtype: str, *args, **kw) -> np.ndarray:
    """``normal_bf16`` (dtype "bf16") or ``normal_f16`` (dtype "f16")."""
    return normal_f16(*args, **kw) if dtype == "f16" else normal_bf16(*args, **kw)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to float32 (a bit shift)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def device_normal_bf16(shape, sigma: float, seed: int, device="cuda",
                       outlier_rate: float = 0.0, outlier_scale: float = 1.0,
                       dtype=torch.bfloat16):
    """Device-side draw for tensors too large to stage on the host (rounded
    to ``dtype``: bfloat16, or float16 for the fp16 compute type)."""
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    x = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    x.mul_(sigma)
    if outlier_rate > 0.0:
        m = torch.rand(shape, generator=g, device=device) < outlier_rate
        x = torch.where(m, x * outlier_scale, x)
    return x.to(dtype)
