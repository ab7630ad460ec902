"""Oracle: folding the trained adapter into the base weight, then requantizing.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

[lqnn §3.3]: after training, the low-rank branch is merged into W by first
dequantizing W to bf16, adding B A at high precision, then quantizing again.
[cf1 §4.3; kwkr §4.4]: the merge loses precision twice -- once when the sum is
rounded to the 16-bit weight dtype, once in the requantization.

Reading (the pages fix neither the order nor the precision of the sum): for
every (n, k),
    acc = sum_j B[n][j] A[j][k]   accumulated in binary32 in rank order
          (j = 0, 1, ..., r-1; each product of two bf16 values is exact),
    t   = fp32(s * acc),          s = alpha / r,
    m   = fp32(w + t),            w = the dequantized base weight (bf16),
    merged = bf16_rne(m).
The merged weight is then quantized with the ordinary quantizer of the
chosen format (``nf4.quantize`` or ``formats``).  With the fp16 compute type
[rkmt §3.3; kwkr §4.3] w, A and B are fp16 and the last rounding is to fp16
(``dtype="f16"``).
"""
from __future__ import annotations

import numpy as np

from .nf4 import narrow, widen


def merged_weight(wd_bits: np.ndarray, A_bits: np.ndarray, B_bits: np.ndarray, s: float,
                  dtype: str = "bf16") -> np.ndarray:
    """16-bit bits [N x K] of the merged weight (steps above)."""
    w = widen(np.asarray(wd_bits, dtype=np.uint16), dtype)
    A = widen(np.asarray(A_bits, dtype=np.uint16), dtype)        # [r x K]
    B = widen(np.asarray(B_bits, dtype=np.uint16), dtype)        # [N x r]
    N, K = w.shape
    acc = np.zeros((N, K), dtype=np.float32)
    for j in range(A.shape[0]):
        prod = np.multiply.outer(B[:, j], A[j, :]).astype(np.float32)   # exact: bf16 x bf16
        acc = (acc + prod).astype(np.float32)
    t = (np.float32(s) * acc).astype(np.float32)
    m = (w + t).astype(np.float32)
    return narrow(m.reshape(-1), dtype).reshape(N, K)


def merge_error_bound(wd_bits, A_bits, B_bits, s: float, dtype: str = "bf16") -> np.ndarray:
    """Per-element bound on |merged - (w + s B A)| (float64): the binary32
    sum of r exact products (each step rounds by at most half an ulp of the
    running sum, bounded by the sum of |products| times 2^-24), the product
    with s, the addition, then the rounding of the result to the compute type
    (half an ulp: 2^-8 relative for bf16; 2^-11 relative for fp16, and at
    least the subnormal half-ulp 2^-25)."""
    w = widen(np.asarray(wd_bits, dtype=np.uint16), dtype).astype(np.float64)
    A = widen(np.asarray(A_bits, dtype=np.uint16), dtype).astype(np.float64)
    B = widen(np.asarray(B_bits, dtype=np.uint16), dtype).astype(np.float64)
    r = A.shape[0]
    mag = np.abs(B) @ np.abs(A)                                   # sum_j |b a|
    exact = w + s * (B @ A)
    acc_err = abs(s) * mag * r * 2.0 ** -24
    fp32_err = (np.abs(exact) + acc_err) * 2.0 ** -23 + abs(s) * mag * 2.0 ** -24
    if dtype == "f16":
        last = np.maximum((np.abs(exact) + acc_err + fp32_err) * 2.0 ** -11, 2.0 ** -25)
    else:
        last = (np.abs(exact) + acc_err + fp32_err) * 2.0 ** -8
    return last + acc_err + fp32_err
