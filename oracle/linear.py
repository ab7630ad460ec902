"""Oracle: the LoRA-augmented quantized linear layer, forward and backward.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

Shapes and orientation [lqnn §3.2; cf1 §3.2]: the frozen weight W is
[N x K] (out_features x in_features, as a torch Linear weight), A is [r x K],
B is [N x r], X is [M x K] (M tokens), Y and dY are [M x N], and the adapter
scaling is s = alpha / r.  ``Wd`` is the dequantized bf16 weight (``nf4``).

Forward [cf1 §2.1, §3.2; lqnn §3.2, §3.3]:
    h = W0 x + (B A) x   for each token, i.e.  Y = X Wd^T + s (X A^T) B^T
Backward [cf1 §2.1: dL/dx = dL/dy W0^T; lqnn §3.3 and zky: only A and B
are trained, the quantized base gets no gradient]:
    U  = dY B
    dX = dY Wd + s U A
    dA = s U^T X
    dB = s dY^T (X A^T)

Everything is the plain definition, evaluated in float64 from exact bf16
inputs (a product of two bf16 values is exact in float64); the matrix products
are numpy's.  No bias and no dropout (both off for parity).

Compute type [rkmt §3.3; kwkr §4.3]: with ``dtype="f16"`` the 16-bit inputs
(Wd, X, A, B, dY given as uint16 bits) are IEEE fp16 instead of bf16; the
products stay exact in float64 (11 x 11 significant bits).
"""
from __future__ import annotations

import numpy as np

from .nf4 import widen


def _f64(bits_or_f, dtype="bf16"):
    a = np.asarray(bits_or_f)
    if a.dtype == np.uint16:
        return widen(a, dtype).astype(np.float64)
    return a.astype(np.float64)


def forward(Wd, X, A=None, B=None, s: float = 0.0, dtype: str = "bf16"):
    """-> (Y [M x N] float64, T = X A^T [M x r] float64 or None)."""
    Wd, X = _f64(Wd, dtype), _f64(X, dtype)
    Y = X @ Wd.T
    T = None
    if A is not None and B is not None and np.asarray(A).shape[0] > 0:
        A, B = _f64(A, dtype), _f64(B, dtype)
        T = X @ A.T
        Y = Y + float(s) * (T @ B.T)
    return Y, T


def backward(Wd, X, dY, A=None, B=None, s: float = 0.0, dtype: str = "bf16"):
    """-> (dX [M x K], dA [r x K] or None, dB [N x r] or None), float64."""
    Wd, X, dY = _f64(Wd, dtype), _f64(X, dtype), _f64(dY, dtype)
    dX = dY @ Wd
    dA = dB = None
    if A is not None and B is not None and np.asarray(A).shape[0] > 0:
        A, B = _f64(A, dtype), _f64(B, dtype)
        U = dY @ B
        T = X @ A.T
        dX = dX + float(s) * (U @ A)
        dA = float(s) * (U.T @ X)
        dB = float(s) * (dY.T @ T)
    return dX, dA, dB


def forward_rows(Wd_rows, X, rows, A=None, B_rows=None, s: float = 0.0, dtype: str = "bf16"):
    """Forward restricted to output columns ``rows`` of Y (rows of W), for
    sampled parity at sizes where the full product is too slow."""
    Y, _ = forward(Wd_rows, X, A, B_rows, s, dtype)
    return Y
