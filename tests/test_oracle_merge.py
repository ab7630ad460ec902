"""Pins of the adapter-merge oracle against special cases, exact integer
arithmetic and the derived error bound.  CPU only."""
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import merge as OM
from oracle import nf4


def bf(x):
    return nf4.f32_to_bf16_rne(np.asarray(x, dtype=np.float32).reshape(-1)).reshape(np.shape(x))


def f(bits):
    return nf4.bf16_to_f32(np.asarray(bits, dtype=np.uint16)).astype(np.float64)


def test_zero_adapter_is_identity():
    rng = np.random.default_rng(0)
    w = bf(rng.standard_normal((5, 64)) * 0.02)
    A = bf(rng.standard_normal((4, 64)) * 0.01)
    B = np.zeros((5, 4), dtype=np.uint16)
    assert np.array_equal(OM.merged_weight(w, A, B, 2.0), w)
    assert np.array_equal(OM.merged_weight(w, A[:0], B[:, :0], 2.0), w)


def test_exact_integer_case_by_fractions():
    # small integers (exact in bf16): every partial sum, the product with s
    # and the addition are exact in binary32, so the result is the bf16
    # rounding of the exact value, computed here with fractions and torch's
    # float64 -> bf16 conversion
    rng = np.random.default_rng(1)
    N, K, r, s = 6, 64, 7, 2.0
    A = rng.integers(-8, 9, size=(r, K)).astype(np.float32)
    B = rng.integers(-8, 9, size=(N, r)).astype(np.float32)
    W = (rng.integers(-300, 301, size=(N, K)) / 16.0).astype(np.float32)
    Ab, Bb, Wb = bf(A), bf(B), bf(W)
    got = OM.merged_weight(Wb, Ab, Bb, s)
    exact = np.empty((N, K))
    for n in range(N):
        for k in range(K):
            acc = sum(Fraction(float(B[n, j])) * Fraction(float(A[j, k])) for j in range(r))
            exact[n, k] = float(Fraction(float(f(Wb)[n, k])) + Fraction(s) * acc)
    want = torch.from_numpy(exact).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(got, want)


@pytest.mark.parametrize("seed,r", [(2, 8), (3, 64), (4, 16)])
def test_within_derived_bound_of_the_exact_sum(seed, r):
    rng = np.random.default_rng(seed)
    N, K, s = 24, 128, 128.0 / 64
    W = bf(rng.standard_normal((N, K)) * 0.02)
    A = bf(rng.standard_normal((r, K)) * 0.01)
    B = bf(rng.standard_normal((N, r)) * 0.01)
    B[3] = bf(np.full(r, 4.0))            # a row whose adapter term dominates
    got = f(OM.merged_weight(W, A, B, s))
    exact = f(W) + s * (f(B) @ f(A))
    bound = OM.merge_error_bound(W, A, B, s)
    assert np.all(np.abs(got - exact) <= bound)
    # the bf16 rounding is the dominant loss: about half an ulp is reached
    ulp = np.abs(exact) * 2.0 ** -7
    assert np.max(np.abs(got - exact) / np.where(ulp > 0, ulp, 1)) > 0.4


def test_requantized_merge_within_the_quantizer_bound():
    rng = np.random.default_rng(5)
    N, K, r, s = 16, 256, 8, 2.0
    lv, mid = nf4.codebook()
    W = bf(rng.standard_normal((N, K)) * 0.02)
    c, q, st = nf4.quantize(W, mid)
    Wd = nf4.dequantize(c, q, st, lv).reshape(N, K)
    A = bf(rng.standard_normal((r, K)) * 0.01)
    B = bf(rng.standard_normal((N, r)) * 0.01)
    M = OM.merged_weight(Wd, A, B, s)
    c2, q2, st2 = nf4.quantize(M, mid)
    M2 = nf4.dequantize(c2, q2, st2, lv)
    err = np.abs(f(M2).reshape(-1) - f(M).reshape(-1))
    assert np.all(err <= nf4.dequant_error_bound(M.reshape(-1), lv))
