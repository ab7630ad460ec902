"""Oracle: affine integer quantization (scale + zero-point).

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

[kwkr §2.1]: a float range [r_min, r_max] is mapped onto integers
[q_min, q_max];  q = round(r / scale) + zero_point,  r_dq = scale (q - zero_point),
scale = (r_max - r_min) / (q_max - q_min);  the zero-point is the integer that
float 0 maps to, so 0 is represented exactly.

Readings where the page is loose:
* the zero-point is rint_even(-r_min * q_max / (r_max - r_min)), evaluated in
  float64 from the range (the page's "round(-(-2.0)/0.015686)" with the scale
  already rounded to fp32 would give 127.49999 -> 127, not the 128 it prints);
* q is clamped to [q_min, q_max] (the page is silent; 2.0 would otherwise map
  to 256 in the INT8 example);
* rounding is half-to-even throughout.
"""
from __future__ import annotations

import numpy as np


def params(r_min: float, r_max: float, q_min: int = 0, q_max: int = 255):
    """-> (scale fp32, zero_point int)."""
    span = float(r_max) - float(r_min)
    scale = np.float32(span / float(q_max - q_min))
    zp = int(np.rint(q_min - float(r_min) * (q_max - q_min) / span))
    return scale, zp


def quantize(r, scale, zp: int, q_min: int = 0, q_max: int = 255) -> np.ndarray:
    r = np.asarray(r, dtype=np.float32)
    q = np.rint(np.divide(r, np.float32(scale), dtype=np.float32)).astype(np.int64) + zp
    return np.clip(q, q_min, q_max)


def dequantize(q, scale, zp: int) -> np.ndarray:
    return (np.float32(scale) * (np.asarray(q, dtype=np.int64) - zp).astype(np.float32)
            ).astype(np.float32)
