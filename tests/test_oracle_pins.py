"""Pins of the CPU oracle against what the pages and the mathematics fix.

Nothing here compares the oracle with itself: each check uses a value printed
on a page (tests/golden/*), a different library routine, brute force, or an
invariant that a plausible slip (dropped term, wrong sign or index, transposed
operand) would break.
"""
import math
import os

import numpy as np
import pytest
import torch
from scipy.optimize import brentq
from scipy.stats import norm

from oracle import affine, linear, nf4
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    out = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            parts = line.split()
            out[parts[0]] = [float(p) for p in parts[1:]]
    return out


# ---------------------------------------------------------------- affine (kwkr §2.1)
def test_affine_worked_example_int8():
    g = _golden("affine_int8_example.txt")
    scale, zp = affine.params(g["r_min"][0], g["r_max"][0], int(g["q_min"][0]), int(g["q_max"][0]))
    assert abs(float(scale) - g["scale"][0]) <= g["scale"][1]
    assert zp == int(g["zero_point"][0])
    q0 = affine.quantize(np.float32(0.0), scale, zp)
    assert int(q0) == int(g["q_of_zero"][0])
    assert float(affine.dequantize(q0, scale, zp)) == g["dq_of_zero"][0]


def test_affine_roundtrip_error_and_clamp():
    scale, zp = affine.params(-2.0, 2.0)
    r = np.linspace(-2.0, 2.0, 10001, dtype=np.float32)
    q = affine.quantize(r, scale, zp)
    assert q.min() >= 0 and q.max() <= 255
    err = np.abs(affine.dequantize(q, scale, zp) - r)
    # interior points are within half a step; only the clamped top end may exceed
    interior = r < 2.0 - float(scale)
    assert np.all(err[interior] <= 0.5 * float(scale) * (1 + 1e-5))


# ---------------------------------------------------------------- storage closed forms
def test_overhead_closed_forms_7b():
    g = _golden("dq_overhead_7b.txt")
    P = g["params"][0]

    def close(key, val):
        ref, tol = g[key]
        assert abs(val - ref) <= tol * abs(ref) + 1e-12, (key, val, ref)

    nodq = nf4.model_bytes(P, double_quant=False, zero_point_bytes=4)   # rkmt §1.3: scale + zero-point
    dq = nf4.model_bytes(P, double_quant=True)
    close("blocks", nodq["blocks"])
    close("codes_GB", nodq["codes"] / 1e9)
    close("no_dq_constants_GB", nodq["constants"] / 1e9)
    close("no_dq_total_GB", nodq["total"] / 1e9)
    close("no_dq_bits_per_param", nf4.bits_per_param(double_quant=False, zero_point_bytes=4) - 4)
    close("dq_first_level_fp32_GB", nf4.model_bytes(P, double_quant=False)["constants"] / 1e9)
    close("dq_second_level_blocks", math.ceil(dq["blocks"] / 256))
    close("dq_second_level_MB", math.ceil(dq["blocks"] / 256) * 4 / 1e6)
    close("dq_u8_scales_GB", dq["blocks"] / 1e9)
    close("dq_constants_GB", dq["constants"] / 1e9)
    close("dq_saved_GB", (nodq["constants"] - dq["constants"]) / 1e9)
    close("dq_total_GB", dq["total"] / 1e9)
    close("dq_reduction_percent", 100 * (nodq["total"] - dq["total"]) / nodq["total"])
    close("dq_bits_per_param_overhead", nf4.bits_per_param() - 4)
    close("absmax_only_bits_per_param", nf4.bits_per_param(double_quant=False) - 4)
    close("dq_saving_bits_per_param", nf4.bits_per_param(double_quant=False) - nf4.bits_per_param())


@pytest.mark.parametrize("n,k", [(1, 64), (3, 128), (7, 320), (4096, 4096), (11008, 4096)])
def test_array_sizes_match_closed_form(n, k):
    codes, qs, st = nf4.nf4_bytes(n, k)
    assert codes * 2 == n * k and qs * 64 == n * k
    assert st == 4 * ((n * k // 64 + 255) // 256)
    if n * k <= 1 << 16:
        _, mids = nf4.codebook()
        w = synth.normal_bf16((n, k), 0.02, seed=n * 131 + k)
        c, q, s = nf4.quantize(w, mids)
        assert c.nbytes == codes and q.nbytes == qs and s.nbytes == st


# ---------------------------------------------------------------- bf16 rounding
def test_bf16_rne_matches_torch():
    g = synth.rng(7)
    x = np.concatenate([
        g.standard_normal(200000).astype(np.float32) * 10.0 ** g.integers(-30, 30, 200000),
        # exact ties: low 16 bits == 0x8000, both parities of bit 16
        (np.arange(1, 5000, dtype=np.uint32) << 17 | 0x8000).view(np.float32),
        (np.arange(1, 5000, dtype=np.uint32) << 17 | 0x18000).view(np.float32),
        np.array([0.0, -0.0, np.inf, -np.inf, 3.4e38, -3.4e38, 1e-45], dtype=np.float32),
    ]).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(nf4.f32_to_bf16_rne(x), ref)
    assert np.array_equal(nf4.bf16_to_f32(ref), torch.from_numpy(ref.view(np.int16)).view(torch.bfloat16).float().numpy())


# ---------------------------------------------------------------- codebook
def test_codebook_invariants():
    lv, mid = nf4.codebook()
    assert lv.dtype == np.float32 and lv.shape == (16,) and mid.shape == (15,)
    assert lv[0] == -1.0 and lv[15] == 1.0 and lv[7] == 0.0
    assert np.all(np.diff(lv) > 0)
    assert np.all(mid > lv[:-1]) and np.all(mid < lv[1:])
    assert np.sum(lv < 0) == 7 and np.sum(lv > 0) == 8


def test_codebook_equal_probability_spacing():
    """zky 5.8 "NF4": levels follow the normal distribution so that each gets a
    similar share.  Checked through the normal CDF (scipy.stats.norm.cdf) and a
    root-found normalizer, not through the inverse CDF the oracle uses."""
    lv, _ = nf4.codebook()
    c_pos = brentq(lambda t: norm.cdf(t) - (1 - 1 / 32), 0.1, 6, xtol=1e-14)
    c_neg = brentq(lambda t: norm.cdf(t) - (1 - 1 / 30), 0.1, 6, xtol=1e-14)
    pos = norm.cdf(lv[8:].astype(np.float64) * c_pos) - 0.5
    neg = norm.cdf(-lv[:7][::-1].astype(np.float64) * c_neg) - 0.5
    assert np.allclose(pos, (np.arange(1, 9)) * (0.5 - 1 / 32) / 8, atol=2e-7)
    assert np.allclose(neg, (np.arange(1, 8)) * (0.5 - 1 / 30) / 7, atol=2e-7)


def _brute_nearest(v32, lv):
    """argmin_k |v - level_k| in float64; ties to the lower index (argmin's first)."""
    d = np.abs(v32.astype(np.float64)[:, None] - lv.astype(np.float64)[None, :])
    return np.argmin(d, axis=1).astype(np.uint8)


def test_encode_equals_brute_force_nearest_level():
    """Both encodings are monotone step functions of v, so they agree on every
    fp32 in [-1, 1] iff they agree around each switching point: the fp32 values
    within 64 ulps of every midpoint and of every exact level mean are checked,
    plus a random sample, every bf16 value in [-1, 1] and the levels themselves."""
    lv, mid = nf4.codebook()
    pts = []
    for k in range(15):
        exact = (float(lv[k]) + float(lv[k + 1])) / 2.0
        for centre in (mid[k], np.float32(exact)):
            u = np.array([centre], dtype=np.float32).view(np.int32)[0]
            off = np.arange(-64, 65, dtype=np.int64)
            if centre < 0:
                off = -off
            pts.append((u + off).astype(np.int32).view(np.float32))
    g = synth.rng(11)
    pts.append(g.uniform(-1, 1, 1 << 20).astype(np.float32))
    allb = (np.arange(65536, dtype=np.uint32) << 16).view(np.float32)
    pts.append(allb[np.abs(allb) <= 1])
    pts.append(lv)
    pts.append(np.array([-1.0, 1.0, 0.0, -0.0], dtype=np.float32))
    v = np.concatenate(pts).astype(np.float32)
    v = v[np.abs(v) <= 1]
    assert np.array_equal(nf4.encode(v, mid), _brute_nearest(v, lv))


# ---------------------------------------------------------------- quantize / dequantize
def test_pack_layout():
    codes = np.arange(16, dtype=np.uint8)
    # word w holds elements 8w..8w+7; byte j = code(8w+j) | code(8w+j+4) << 4
    assert list(nf4.pack(codes)) == [0x40, 0x51, 0x62, 0x73, 0xC8, 0xD9, 0xEA, 0xFB]
    g = synth.rng(3)
    c = g.integers(0, 16, 4096).astype(np.uint8)
    assert np.array_equal(nf4.unpack(nf4.pack(c)), c)


def _bits(vals):
    return torch.tensor(vals, dtype=torch.float32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def test_special_blocks():
    lv, mid = nf4.codebook()
    w = np.zeros((4, 64), dtype=np.uint16)                 # block 0: all zero
    w[1] = _bits([0.25] * 64)                               # block 1: all equal, positive
    w[2] = _bits([-0.5] * 64)                               # block 2: all equal, negative
    row = np.linspace(-3.0, 1.0, 64).astype(np.float32)     # block 3: absmax element negative
    w[3] = _bits(row)
    codes, qs, st = nf4.quantize(w, mid)
    c = nf4.unpack(codes).reshape(4, 64)
    assert np.all(c[0] == 7) and np.all(c[1] == 15) and np.all(c[2] == 0)
    assert c[3][0] == 0                                     # -absmax -> level -1
    # the group's largest absmax gets qscale 255 exactly; others below
    am = nf4.block_absmax(w)
    assert qs[np.argmax(am)] == 255 and qs[0] == 0
    assert np.all(qs <= 255)
    # the block holding the group max dequantizes its extreme to +-c2 exactly
    d = nf4.bf16_to_f32(nf4.dequantize(codes, qs, st, lv)).reshape(4, 64)
    assert d[3][0] == -3.0
    assert np.all(d[0] == 0.0)


def test_zero_group_and_short_last_group():
    lv, mid = nf4.codebook()
    n_blocks = 256 + 44                                      # second group is short
    w = synth.normal_bf16((n_blocks, 64), 0.02, seed=5)
    w[:256] = 0                                              # first group all zero
    codes, qs, st = nf4.quantize(w, mid)
    assert st.shape == (2,) and st[0] == 0 and np.all(qs[:256] == 0)
    assert st[1] > 0 and qs[256:].max() == 255
    d = nf4.bf16_to_f32(nf4.dequantize(codes, qs, st, lv))
    assert np.all(d[:256 * 64] == 0)


def test_dequant_hand_values():
    lv, _ = nf4.codebook()
    # qscale 3 * step 0.25 = 0.75 exactly; level +-1 -> +-0.75, level 0 -> 0
    codes = nf4.pack(np.array([15, 0, 7, 15, 0, 7, 15, 0] * 8, dtype=np.uint8))
    d = nf4.bf16_to_f32(nf4.dequantize(codes, np.array([3], np.uint8), np.array([0.25], np.float32), lv))
    assert list(d[:8]) == [0.75, -0.75, 0.0, 0.75, -0.75, 0.0, 0.75, -0.75]


def test_qscale_is_nearest_multiple_of_step():
    """Brute force over all 256 u8 values: qscale is the nearest multiple of the
    stored step to absmax (exact ties aside)."""
    _, mid = nf4.codebook()
    w = synth.normal_bf16((1024, 64), 0.02, seed=9, outlier_rate=0.01, outlier_scale=20)
    _, qs, st = nf4.quantize(w, mid)
    am = nf4.block_absmax(w).astype(np.float64)
    grid = np.arange(256, dtype=np.float64)
    for g in range(st.size):
        a = am[g * 256:(g + 1) * 256]
        d = np.abs(grid[None, :] * float(st[g]) - a[:, None])
        best = np.argmin(d, axis=1)
        frac = a / float(st[g]) - np.floor(a / float(st[g]))
        near_tie = np.abs(frac - 0.5) < 1e-5
        assert np.all((best == qs[g * 256:(g + 1) * 256]) | near_tie)


@pytest.mark.parametrize("sigma,outliers", [(0.02, 0.0), (0.015, 0.001), (1.0, 0.05)])
def test_dequant_error_within_derived_bound(sigma, outliers):
    lv, mid = nf4.codebook()
    w = synth.normal_bf16((256, 1024), sigma, seed=21, outlier_rate=outliers, outlier_scale=20)
    codes, qs, st = nf4.quantize(w, mid)
    d = nf4.bf16_to_f32(nf4.dequantize(codes, qs, st, lv)).astype(np.float64)
    x = nf4.bf16_to_f32(w.reshape(-1)).astype(np.float64)
    bound = nf4.dequant_error_bound(w, lv)
    assert np.all(np.abs(d - x) <= bound)
    # and the bound is not vacuous: half the widest codebook gap (0.151) times
    # absmax, plus about half a second-level step
    am = np.repeat(nf4.block_absmax(w).astype(np.float64), 64)
    step_el = np.repeat(st.astype(np.float64), 64 * 256)[: am.size]
    assert np.all(bound <= 0.16 * am + 0.6 * step_el + 1e-30)


# ------------------------------------------ without double quantization (rkmt §1.2, §2.3)
def test_nodq_special_blocks_and_hand_values():
    """fp32 absmax kept per block: the extremes dequantize to +-absmax exactly,
    zero blocks to zeros, and level 0 to exact zeros."""
    lv, mid = nf4.codebook()
    w = np.zeros((3, 64), dtype=np.uint16)
    w[1] = _bits([0.25] * 64)
    row = np.linspace(-3.0, 1.0, 64).astype(np.float32)
    w[2] = _bits(row)
    codes, am = nf4.quantize_nodq(w, mid)
    assert am.dtype == np.float32 and am.tolist() == [0.0, 0.25, 3.0]
    c = nf4.unpack(codes).reshape(3, 64)
    assert np.all(c[0] == 7) and np.all(c[1] == 15) and c[2][0] == 0
    d = nf4.bf16_to_f32(nf4.dequantize_nodq(codes, am, lv)).reshape(3, 64)
    assert np.all(d[0] == 0.0) and np.all(d[1] == 0.25) and d[2][0] == -3.0
    # hand case: absmax 0.75 (exact in bf16): levels +-1 -> +-0.75, level 0 -> 0
    hand = nf4.pack(np.array([15, 0, 7, 15, 0, 7, 15, 0] * 8, dtype=np.uint8))
    dh = nf4.bf16_to_f32(nf4.dequantize_nodq(hand, np.array([0.75], np.float32), lv))
    assert list(dh[:8]) == [0.75, -0.75, 0.0, 0.75, -0.75, 0.0, 0.75, -0.75]


def test_nodq_absmax_by_python_loops_and_codes_match_double_quant():
    """absmax is the block maximum of |w| (python loops over a small weight);
    the first level does not depend on the second, so the codes equal those
    of the double-quantized format."""
    _, mid = nf4.codebook()
    w = synth.normal_bf16((7, 192), 0.02, seed=31, outlier_rate=0.02, outlier_scale=20)
    codes, am = nf4.quantize_nodq(w, mid)
    x = nf4.bf16_to_f32(w.reshape(-1))
    for b in range(am.size):
        assert am[b] == max(abs(float(v)) for v in x[64 * b:64 * b + 64])
    codes_dq, _, _ = nf4.quantize(w, mid)
    assert np.array_equal(codes, codes_dq)


@pytest.mark.parametrize("sigma,outliers", [(0.02, 0.0), (1.0, 0.05)])
def test_nodq_error_within_derived_bound(sigma, outliers):
    lv, mid = nf4.codebook()
    w = synth.normal_bf16((128, 1024), sigma, seed=23, outlier_rate=outliers, outlier_scale=20)
    codes, am = nf4.quantize_nodq(w, mid)
    d = nf4.bf16_to_f32(nf4.dequantize_nodq(codes, am, lv)).astype(np.float64)
    x = nf4.bf16_to_f32(w.reshape(-1)).astype(np.float64)
    bound = nf4.dequant_error_bound(w, lv, double_quant=False)
    assert np.all(np.abs(d - x) <= bound)
    amb = np.repeat(am.astype(np.float64), 64)
    assert np.all(bound <= 0.16 * amb + 1e-30)


def test_blocks_to_storage_uses_the_scale_positions():
    g = np.random.default_rng(4)
    n, k = 37, 192
    qs = g.integers(0, 256, n * k // 64, dtype=np.uint8)
    am = g.random(n * k // 64).astype(np.float32)
    _, qst = nf4.to_storage(np.zeros(n * k // 2, np.uint8), qs, n, k)
    assert np.array_equal(nf4.blocks_to_storage(qs, n, k), qst)
    pos = nf4.storage_positions(n, k)
    assert np.array_equal(nf4.blocks_to_storage(am, n, k)[pos], am)


# ---------------------------------------------------------------- linear algebra
def _tiny(seed, M=3, N=5, K=64, r=2):
    X = synth.normal_bf16((M, K), 1.0, seed)
    W = synth.normal_bf16((N, K), 0.5, seed + 1)
    A = synth.normal_bf16((r, K), 0.3, seed + 2)
    B = synth.normal_bf16((N, r), 0.3, seed + 3)
    dY = synth.normal_bf16((M, N), 1.0, seed + 4)
    return X, W, A, B, dY


def _f(b):
    return nf4.bf16_to_f32(b).astype(np.float64)


def test_forward_equals_python_loops():
    X, W, A, B, _ = _tiny(100)
    s = 2.0
    Y, T = linear.forward(W, X, A, B, s)
    x, w, a, b = _f(X), _f(W), _f(A), _f(B)
    M, K = x.shape
    N, r = b.shape
    for m in range(M):
        t = [math.fsum(x[m, k] * a[j, k] for k in range(K)) for j in range(r)]
        assert np.allclose(T[m], t, rtol=1e-14, atol=1e-14)
        for n in range(N):
            base = math.fsum(x[m, k] * w[n, k] for k in range(K))
            lora = math.fsum(t[j] * b[n, j] for j in range(r))
            assert abs(Y[m, n] - (base + s * lora)) <= 1e-12 * (1 + abs(base))


def test_backward_equals_torch_autograd():
    X, W, A, B, dY = _tiny(200, M=4, N=6, K=128, r=3)
    s = 0.5
    dX, dA, dB = linear.backward(W, X, dY, A, B, s)
    x = torch.tensor(_f(X), requires_grad=True)
    a = torch.tensor(_f(A), requires_grad=True)
    b = torch.tensor(_f(B), requires_grad=True)
    w = torch.tensor(_f(W))
    y = x @ w.T + s * (x @ a.T) @ b.T
    y.backward(torch.tensor(_f(dY)))
    assert np.allclose(dX, x.grad.numpy(), rtol=1e-13, atol=1e-13)
    assert np.allclose(dA, a.grad.numpy(), rtol=1e-13, atol=1e-13)
    assert np.allclose(dB, b.grad.numpy(), rtol=1e-13, atol=1e-13)


def test_special_cases_b0_w0_r0_identity():
    X, W, A, B, dY = _tiny(300, M=4, N=7, K=64, r=2)
    base, _ = linear.forward(W, X)
    # B = 0: the adapter contributes nothing (cf1 §3.2: output equals the base)
    Y0, _ = linear.forward(W, X, A, np.zeros_like(B), 3.0)
    assert np.array_equal(Y0, base)
    # W = 0: only the adapter
    Yl, T = linear.forward(np.zeros_like(W), X, A, B, 3.0)
    assert np.allclose(Yl, 3.0 * T @ _f(B).T, rtol=1e-14, atol=0)
    # r = 0: base only
    Yr, Tr = linear.forward(W, X, A[:0], B[:, :0], 3.0)
    assert Tr is None and np.array_equal(Yr, base)
    # identity rows of X pick columns of W
    I = _bits(np.eye(64, dtype=np.float32)[:7])
    Yi, _ = linear.forward(W, I)
    assert np.array_equal(Yi, _f(W)[:, :7].T)


def test_adjoint_identity():
    X, W, A, B, dY = _tiny(400, M=8, N=9, K=192, r=4)
    Y, _ = linear.forward(W, X)
    dX, _, _ = linear.backward(W, X, dY)
    lhs = np.sum(_f(dY) * Y)
    rhs = np.sum(dX * _f(X))
    assert abs(lhs - rhs) <= 1e-12 * (abs(lhs) + 1)


def test_full_path_small():
    """quantize -> dequantize -> forward at a tiny size, against the float64
    product of the original bf16 weight within the dequantization bound."""
    lv, mid = nf4.codebook()
    X, W, A, B, _ = _tiny(500, M=2, N=4, K=256, r=2)
    codes, qs, st = nf4.quantize(W, mid)
    Wd = nf4.dequantize(codes, qs, st, lv).reshape(W.shape)
    Yq, _ = linear.forward(Wd, X, A, B, 2.0)
    Yf, _ = linear.forward(W, X, A, B, 2.0)
    bound = nf4.dequant_error_bound(W, lv).reshape(W.shape)
    err_max = np.abs(_f(X)) @ bound.T
    assert np.all(np.abs(Yq - Yf) <= err_max + 1e-12)


# --------------------------------------------------------------------------- storage order
def test_storage_positions_small_cases_by_hand():
    # 3 rows (one partial group of R = 3), 2 blocks per row: k-block-major, then row
    assert nf4.storage_positions(3, 128).tolist() == [0, 3, 1, 4, 2, 5]
    # 17 rows: a full group (R = 16) then a group of one row (R = 1)
    pos = nf4.storage_positions(17, 128).reshape(17, 2)
    assert pos[0].tolist() == [0, 16]
    assert pos[15].tolist() == [15, 31]
    assert pos[16].tolist() == [32, 33]


@pytest.mark.parametrize("n,k", [(1, 64), (16, 256), (17, 320), (100, 11008), (4096, 128)])
def test_storage_positions_are_a_permutation_with_contiguous_row_runs(n, k):
    pos = nf4.storage_positions(n, k)
    nkb = k // 64
    assert np.array_equal(np.sort(pos), np.arange(n * nkb))
    grid = pos.reshape(n, nkb)
    for g0 in range(0, n, 16):
        rows = grid[g0:g0 + 16]
        # the rows of a group hold one contiguous, row-ordered run at each k-block
        assert np.all(np.diff(rows, axis=0) == 1)
        assert np.all(np.diff(rows[0]) == rows.shape[0])


def test_storage_round_trip():
    g = np.random.default_rng(3)
    n, k = 37, 192
    codes = g.integers(0, 256, n * k // 2, dtype=np.uint8)
    qs = g.integers(0, 256, n * k // 64, dtype=np.uint8)
    cst, qst = nf4.to_storage(codes, qs, n, k)
    c2, q2 = nf4.from_storage(cst, qst, n, k)
    assert np.array_equal(c2, codes) and np.array_equal(q2, qs)
    # a block keeps its 32 bytes together
    b = 5 * 3 + 2
    p = nf4.storage_positions(n, k)[b]
    assert np.array_equal(cst[32 * p:32 * p + 32], codes[32 * b:32 * b + 32])
    assert qst[p] == qs[b]
