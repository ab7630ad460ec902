"""Pins of the fp16 compute type in the oracle (CPU only): the binary16
conversions against numpy's own IEEE half type and a brute-force nearest-value
search over the whole fp16 grid; quantization of fp16 weights against the
pinned bf16 path on values exact in both types; the dequantized weight, the
error bound, the linear layer and the merge in fp16."""
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import linear as olin
from oracle import merge as OM
from oracle import nf4

LV, MID = nf4.codebook()


def test_widen_every_pattern_matches_ieee_half():
    bits = np.arange(1 << 16, dtype=np.uint16)
    got = nf4.f16_to_f32(bits)
    ref = bits.view(np.float16).astype(np.float32)
    same = (got.view(np.uint32) == ref.view(np.uint32)) | (np.isnan(got) & np.isnan(ref))
    assert same.all()
    hand = {0x3C00: 1.0, 0x0001: 2.0 ** -24, 0x03FF: 1023 * 2.0 ** -24, 0x0400: 2.0 ** -14,
            0x7BFF: 65504.0, 0xC000: -2.0, 0x3555: 1365 / 4096, 0x7C00: np.inf, 0xFC00: -np.inf}
    for b, v in hand.items():
        assert nf4.f16_to_f32(np.array([b], np.uint16))[0] == np.float32(v)


def _nearest_even_grid(x):
    """Brute force: the nearest finite fp16 to each fp32 magnitude by search
    over the sorted grid of all positive patterns, ties to the even pattern,
    magnitudes at or above 65520 (65504 plus half its ulp) to infinity."""
    pos = np.arange(0x7C00, dtype=np.uint16)                      # +0 .. 65504
    vals = nf4.f16_to_f32(pos).astype(np.float64)
    a = np.abs(x.astype(np.float64))
    hi = np.clip(np.searchsorted(vals, a, side="left"), 0, pos.size - 1)
    lo = np.clip(hi - 1, 0, None)
    dlo, dhi = a - vals[lo], vals[hi] - a
    pick = np.where(dlo < dhi, lo, np.where(dhi < dlo, hi, np.where(pos[lo] % 2 == 0, lo, hi)))
    pick = np.where(a <= vals[0], 0, pick)
    out = pos[pick].astype(np.int64)
    out = np.where(a >= 65520.0, 0x7C00, out)
    return (out | np.where(np.signbit(x), 0x8000, 0)).astype(np.uint16)


def test_round_matches_brute_force_and_ieee_half():
    rng = np.random.default_rng(3)
    parts = [rng.standard_normal(200000) * 10.0 ** rng.uniform(-9, 5, 200000),   # every binade
             rng.uniform(0, 2.0 ** -14, 50000),                                  # subnormal range
             rng.uniform(65000, 66000, 20000)]                                   # overflow edge
    x = np.concatenate(parts).astype(np.float32)
    got = nf4.f32_to_f16_rne(x)
    assert np.array_equal(got, _nearest_even_grid(x))
    with np.errstate(over="ignore"):
        assert np.array_equal(got, x.astype(np.float16).view(np.uint16))


def test_round_ties_go_to_even_pattern():
    # exact midpoints of adjacent fp16 values (exact in fp32): normal and subnormal
    pos = np.array([0x3C00, 0x3C01, 0x0001, 0x0002, 0x03FF, 0x7BFE, 0x1234, 0x1235], np.uint16)
    a = nf4.f16_to_f32(pos).astype(np.float64)
    b = nf4.f16_to_f32(pos + 1).astype(np.float64)
    mid = ((a + b) / 2).astype(np.float32)
    got = nf4.f32_to_f16_rne(mid)
    want = np.where(pos % 2 == 0, pos, pos + 1).astype(np.uint16)
    assert np.array_equal(got, want)
    assert nf4.f32_to_f16_rne(np.float32([65519.996, 65520.0, -65520.0, 2.0 ** -26, 2.0 ** -25 * 1.5])).tolist() == \
        [0x7BFF, 0x7C00, 0xFC00, 0x0000, 0x0001]


def _both(k_ints, scale_pow):
    """Values k * 2^scale_pow with |k| < 256: exact in bf16 and in fp16."""
    v = (np.asarray(k_ints, np.float64) * 2.0 ** scale_pow).astype(np.float32)
    return nf4.f32_to_bf16_rne(v), nf4.f32_to_f16_rne(v)


@pytest.mark.parametrize("dq", [True, False])
def test_f16_quantize_equals_bf16_path_on_common_values(dq):
    rng = np.random.default_rng(4)
    k = rng.integers(-255, 256, size=64 * 300)
    k[:64] = 0                                               # an all-zero block
    b16, h16 = _both(k, -12)
    if dq:
        cb, qb, sb = nf4.quantize(b16, MID)
        ch, qh, sh = nf4.quantize(h16, MID, dtype="f16")
        assert np.array_equal(cb, ch) and np.array_equal(qb, qh) and np.array_equal(sb, sh)
        s = nf4.block_scale(qh, sh)
        wd = nf4.dequantize(ch, qh, sh, LV, dtype="f16")
    else:
        cb, ab = nf4.quantize_nodq(b16, MID)
        ch, ah = nf4.quantize_nodq(h16, MID, dtype="f16")
        assert np.array_equal(cb, ch) and np.array_equal(ab, ah)
        s = ah
        wd = nf4.dequantize_nodq(ch, ah, LV, dtype="f16")
    # the fp16 weight is the IEEE-half rounding of the same fp32 product
    prod = (LV[nf4.unpack(ch)] * np.repeat(s, 64)).astype(np.float32)
    assert np.array_equal(wd, prod.astype(np.float16).view(np.uint16))
    # fp16 keeps 11 significant bits: never farther from the product than bf16
    wb = nf4.bf16_to_f32(nf4.f32_to_bf16_rne(prod)).astype(np.float64)
    wh = nf4.f16_to_f32(wd).astype(np.float64)
    normal = np.abs(prod) >= 2.0 ** -14
    assert np.all(np.abs(wh - prod)[normal] <= np.abs(wb - prod)[normal])


@pytest.mark.parametrize("scale", [0.02, 2e-6])
def test_f16_error_bound(scale):
    # 2e-6: every weight and most products are fp16 subnormals
    rng = np.random.default_rng(5)
    x = (rng.standard_normal(64 * 512) * scale).astype(np.float32)
    x[rng.choice(x.size, 40, replace=False)] *= 20
    h = nf4.f32_to_f16_rne(x)
    for dq in (True, False):
        if dq:
            c, q, s = nf4.quantize(h, MID, dtype="f16")
            w = nf4.dequantize(c, q, s, LV, dtype="f16")
        else:
            c, am = nf4.quantize_nodq(h, MID, dtype="f16")
            w = nf4.dequantize_nodq(c, am, LV, dtype="f16")
        err = np.abs(nf4.f16_to_f32(w).astype(np.float64) - nf4.f16_to_f32(h))
        assert np.all(err <= nf4.dequant_error_bound(h, LV, double_quant=dq, dtype="f16"))


def test_f16_linear_matches_torch_autograd_and_special_cases():
    rng = np.random.default_rng(6)
    M, N, K, r, s = 5, 7, 128, 3, 2.0
    h = lambda a: nf4.f32_to_f16_rne(np.asarray(a, np.float32))
    W, X = h(rng.standard_normal((N, K)) * 0.02), h(rng.standard_normal((M, K)))
    A, B = h(rng.standard_normal((r, K)) * 0.01), h(rng.standard_normal((N, r)) * 0.01)
    dY = h(rng.standard_normal((M, N)))
    t = lambda b: torch.from_numpy(b.view(np.float16).astype(np.float64))
    Wt, Xt, At, Bt, dYt = t(W), t(X).requires_grad_(), t(A).requires_grad_(), t(B).requires_grad_(), t(dY)
    Yt = Xt @ Wt.T + s * (Xt @ At.T) @ Bt.T
    Yt.backward(dYt)
    Y, _ = olin.forward(W, X, A, B, s, dtype="f16")
    dX, dA, dB = olin.backward(W, X, dY, A, B, s, dtype="f16")
    assert np.allclose(Y, Yt.detach().numpy(), rtol=1e-13, atol=1e-15)
    assert np.allclose(dX, Xt.grad.numpy(), rtol=1e-13, atol=1e-15)
    assert np.allclose(dA, At.grad.numpy(), rtol=1e-13, atol=1e-15)
    assert np.allclose(dB, Bt.grad.numpy(), rtol=1e-13, atol=1e-15)
    # identity rows read the weight back exactly; B = 0 leaves the base product
    eye = h(np.eye(K)[:4])
    Yi, _ = olin.forward(W, eye, dtype="f16")
    assert np.array_equal(Yi, W.view(np.float16).astype(np.float64)[:, :4].T)
    Y0, _ = olin.forward(W, X, A, np.zeros_like(B), s, dtype="f16")
    assert np.array_equal(Y0, olin.forward(W, X, dtype="f16")[0])


def test_f16_merge_exact_integer_case():
    # small integers: the binary32 steps are exact, so the merge is the fp16
    # rounding of the exact value (fractions, then numpy's float64 -> half)
    rng = np.random.default_rng(7)
    N, K, r, s = 6, 64, 5, 2.0
    A = rng.integers(-8, 9, size=(r, K)).astype(np.float32)
    B = rng.integers(-8, 9, size=(N, r)).astype(np.float32)
    W = (rng.integers(-300, 301, size=(N, K)) / 16.0).astype(np.float32)
    h = lambda a: nf4.f32_to_f16_rne(a.reshape(-1)).reshape(a.shape)
    got = OM.merged_weight(h(W), h(A), h(B), s, dtype="f16")
    exact = np.empty((N, K))
    for n in range(N):
        for k in range(K):
            acc = sum(Fraction(float(B[n, j])) * Fraction(float(A[j, k])) for j in range(r))
            exact[n, k] = float(Fraction(float(W[n, k])) + Fraction(s) * acc)
    assert np.array_equal(got, exact.astype(np.float16).view(np.uint16))
    bound = OM.merge_error_bound(h(W), h(A), h(B), s, dtype="f16")
    assert np.all(np.abs(nf4.f16_to_f32(got) - exact) <= bound)
