"""Pins of the alternate-format oracle (asymmetric uint4 and Q8_0 blocks)
against hand-derived values, brute force and closed forms.  CPU only."""
import numpy as np
import pytest

from oracle import formats as F
from oracle import nf4


def bf(x):
    return nf4.f32_to_bf16_rne(np.asarray(x, dtype=np.float32).reshape(-1))


def f(bits):
    return nf4.bf16_to_f32(np.asarray(bits, dtype=np.uint16)).astype(np.float64)


def u4_codes(codes):
    return nf4.unpack(codes).astype(np.int64)


# ---------------------------------------------------------------- uint4
def test_u4_hand_values_symmetric_range():
    # a block spanning [-2, 2] (rkmt §2.1 with the INT8 example's range of
    # kwkr §2.1): scale = fp32(4 / 15) = 0x3E888889 = 0.26666668057, a little
    # above 4/15.  The zero-point comes from the range: -lo * 15 / (hi - lo) =
    # 7.5 exactly, rint_even -> 8 (the reading that gives kwkr §2.1's printed
    # 128 for the INT8 case).  The alternative reading, the binary32 quotient
    # -lo / fp32(scale) = 7.49999952, would round to 7.
    x = np.zeros(64, np.float32)
    x[0], x[1], x[2], x[3] = -2.0, 2.0, 0.0, 1.0
    codes, s, z = F.u4_quantize(bf(x))
    assert s[0] == np.float32(0.2666666805744171) and s.view(np.uint32)[0] == 0x3E888889
    assert z[0] == 8.0
    assert np.rint(np.divide(np.float32(2.0), s[0], dtype=np.float32)) == 7.0   # the other reading
    q = u4_codes(codes)
    # -2: rint(-7.4999995) = -7 -> 1;  2: 7 -> 15;  0 -> zp;  1: rint(3.7499998) = 4 -> 12
    assert list(q[:4]) == [1, 15, 8, 12]
    w = f(F.u4_dequantize(codes, s, z))
    # bf16 of -7 s = -1.8666667 is -1.8671875; of 4 s = 1.0666667 is 1.0703125;
    # zero is exact.  Both ends sit half a grid step inside the range.
    assert list(w[:4]) == [-1.8671875, 1.8671875, 0.0, 1.0703125]
    assert np.all(np.abs(w - f(bf(x))) <= F.u4_error_bound(bf(x), s))


def test_u4_one_sign_block_widened_to_zero():
    x = np.linspace(0.5, 1.0, 64).astype(np.float32)
    codes, s, z = F.u4_quantize(bf(x))
    # lo widened to 0: scale = fp32(1 / 15), zero-point 0, the maximum on code 15
    assert s[0] == np.float32(0.0666666701436042) and z[0] == 0.0
    q = u4_codes(codes)
    # scale is a little above 1/15 (0x3D888889): 0.5 / scale = 7.4999996 -> 7
    assert q.max() == 15 and q.min() == 7
    assert f(F.u4_dequantize(codes, s, z))[63] == 1.0
    # all negative: hi widened to 0 (the same scale), zero-point 15, -1 on
    # code 0 and -0.5 on rint(-7.4999996) + 15 = 8
    codes, s, z = F.u4_quantize(bf(-x))
    assert s[0] == np.float32(0.0666666701436042) and z[0] == 15.0
    q = u4_codes(codes)
    assert q[63] == 0 and q[0] == 8


def test_u4_zero_block_and_exact_zero():
    x = np.zeros(128, np.float32)
    x[64:] = np.linspace(-0.3, 0.7, 64)
    x[70] = 0.0
    codes, s, z = F.u4_quantize(bf(x))
    assert s[0] == 0.0 and z[0] == 0.0 and np.all(u4_codes(codes)[:64] == 0)
    w = f(F.u4_dequantize(codes, s, z))
    assert np.all(w[:64] == 0.0) and w[70] == 0.0      # zero is on the grid
    assert 0 <= z[1] <= 15 and z[1] == np.round(z[1])


def _u4_brute(xb, s, z):
    grid = s * (np.arange(16, dtype=np.float64) - z)
    return np.abs(xb[:, None] - grid[None, :])


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_u4_codes_are_the_nearest_grid_point(seed):
    rng = np.random.default_rng(seed)
    x = (rng.standard_normal((16, 64)) * 0.02).astype(np.float32)
    x[3] = np.abs(x[3])                  # one-sign blocks
    x[4] = -np.abs(x[4])
    x[5, 7] = 0.6                        # an outlier
    b = bf(x)
    codes, s, z = F.u4_quantize(b)
    q = u4_codes(codes).reshape(16, 64)
    xf = f(b).reshape(16, 64)
    for i in range(16):
        d = _u4_brute(xf[i], float(s[i]), float(z[i]))
        chosen = d[np.arange(64), q[i]]
        assert np.all(chosen <= d.min(axis=1) + float(s[i]) * 2.0 ** -18)


@pytest.mark.parametrize("sigma,outliers", [(0.02, 0), (0.015, 0.001)])
def test_u4_error_within_derived_bound(sigma, outliers):
    rng = np.random.default_rng(7)
    x = (rng.standard_normal(64 * 512) * sigma).astype(np.float32)
    if outliers:
        idx = rng.choice(x.size, int(x.size * outliers) + 1, replace=False)
        x[idx] *= 20
    b = bf(x)
    codes, s, z = F.u4_quantize(b)
    err = np.abs(f(F.u4_dequantize(codes, s, z)) - f(b))
    bound = F.u4_error_bound(b, s)
    assert np.all(err <= bound)
    # the bound is tight to within the bf16 term: half a grid step is reached
    assert np.max(err / np.repeat(s, 64)) > 0.45


def test_u4_sizes_closed_form():
    # rkmt §1.3: fp32 scale + fp32 zero-point per 64-block = 8 bytes, 1 bit per
    # weight, 4-bit codes become about 5 bits; 7e9 weights -> 0.875 GB of constants
    c, p = F.u4_bytes(4096, 4096)
    assert c == 4096 * 4096 // 2 and p == 8 * 4096 * 4096 // 64
    assert (c + p) * 8 / (4096 * 4096) == 5.0
    assert p / (4096 * 4096) * 7e9 / 1e9 == pytest.approx(0.875)


# ---------------------------------------------------------------- Q8_0
def test_q8_hand_values_exact_scale():
    # absmax 127/128: d = 2^-7 exactly, so x = k 2^-7 encodes to k and halves
    # go to the even integer
    x = np.zeros(64, np.float32)
    x[0] = 127 / 128
    x[1], x[2], x[3], x[4], x[5] = 5 * 2.0 ** -7, 1.5 * 2.0 ** -7, 2.5 * 2.0 ** -7, -1.5 * 2.0 ** -7, -127 / 128
    q, d16 = F.q8_quantize(bf(x))
    assert d16[0] == np.float16(2.0 ** -7)
    assert list(q[:6]) == [127, 5, 2, 2, -2, -127]
    w = f(F.q8_dequantize(q, d16))
    assert w[0] == 127 / 128 and w[1] == 5 * 2.0 ** -7 and w[3] == 2 * 2.0 ** -7


def test_q8_hand_values_rounded_scale():
    # absmax 1: d = fp32(1 / 127) = 2^-7 * 1.0078740; in fp16 (10 fraction bits)
    # the fraction 8.06 / 1024 rounds to 8 / 1024: d16 = 2^-7 + 2^-14
    x = np.zeros(32, np.float32)
    x[0], x[1], x[2] = 1.0, -1.0, 0.5
    q, d16 = F.q8_quantize(bf(np.concatenate([x, x])))
    assert d16[0] == np.float16(2.0 ** -7 + 2.0 ** -14) and d16[1] == d16[0]
    # 1 / d16 = 127.0078 -> 127;  0.5 / d16 = 63.504 -> 64
    assert list(q[:3]) == [127, -127, 64]


def test_q8_subnormal_scale_clamps_and_zero_scale():
    # absmax 2^-16: d = 2.016 * 2^-24 rounds to the fp16 subnormal 2^-23, and
    # 2^-16 / 2^-23 = 128 clamps to 127;  absmax 2^-20: d16 rounds to 0 and
    # every code is 0
    x = np.zeros(96, np.float32)
    x[0], x[1] = 2.0 ** -16, -(2.0 ** -17)
    x[32] = 2.0 ** -20
    x[64] = 0.0
    b = bf(np.concatenate([x, np.zeros(32, np.float32)]))
    q, d16 = F.q8_quantize(b)
    assert d16[0] == np.float16(2.0 ** -23) and q[0] == 127 and q[1] == -64
    assert d16[1] == 0 and np.all(q[32:64] == 0)
    assert d16[2] == 0 and np.all(q[64:96] == 0)
    err = np.abs(f(F.q8_dequantize(q, d16)) - f(b))
    assert err[0] == 2.0 ** -23 and err[32] == 2.0 ** -20
    # the negative end clamps to -127 as well (the grid is symmetric)
    qn, _ = F.q8_quantize(b ^ np.uint16(0x8000))
    assert qn[0] == -127 and qn[1] == 64
    assert np.all(err <= F.q8_error_bound(b, d16))


@pytest.mark.parametrize("seed", [0, 1])
def test_q8_codes_are_the_nearest_grid_point_and_odd(seed):
    rng = np.random.default_rng(seed)
    x = (rng.standard_normal((8, 64)) * 0.02).astype(np.float32)
    x[2, 5] = 0.5
    b = bf(x)
    q, d16 = F.q8_quantize(b)
    xf = f(b).reshape(-1, 32)
    qq = q.astype(np.int64).reshape(-1, 32)
    grid_c = np.arange(-127, 128, dtype=np.float64)
    for i in range(xf.shape[0]):
        d = float(d16[i])
        dist = np.abs(xf[i][:, None] - d * grid_c[None, :])
        chosen = dist[np.arange(32), qq[i] + 127]
        assert np.all(chosen <= dist.min(axis=1) + d * 2.0 ** -17)
    # symmetric: negating the weight negates the codes, keeps the scales
    qn, dn = F.q8_quantize(b ^ np.uint16(0x8000))
    assert np.array_equal(qn, -q) and np.array_equal(dn, d16)


@pytest.mark.parametrize("sigma,outliers", [(0.02, 0), (0.015, 0.001)])
def test_q8_error_within_derived_bound(sigma, outliers):
    rng = np.random.default_rng(11)
    x = (rng.standard_normal(64 * 512) * sigma).astype(np.float32)
    if outliers:
        idx = rng.choice(x.size, int(x.size * outliers) + 1, replace=False)
        x[idx] *= 20
    b = bf(x)
    q, d16 = F.q8_quantize(b)
    err = np.abs(f(F.q8_dequantize(q, d16)) - f(b))
    assert np.all(err <= F.q8_error_bound(b, d16))
    assert np.max(np.abs(q)) == 127


def test_q8_sizes_closed_form():
    # cf1 §1.1: 32 weights share one fp16 scale, a little over one byte per
    # weight; a 3.8B model is 7.6 GB in bf16 and about 4 GB in Q8_0
    c, s = F.q8_bytes(3072, 8192)
    assert (c + s) / (3072 * 8192) == 34 / 32
    assert 3.8e9 * 2 / 1e9 == pytest.approx(7.6)
    assert 3.8e9 * (c + s) / (3072 * 8192) / 1e9 == pytest.approx(4.0375)


# ---------------------------------------------------------------- storage
@pytest.mark.parametrize("n,k", [(20, 128), (16, 64), (3, 192)])
def test_storage_round_trips_and_uses_the_block_order(n, k):
    rng = np.random.default_rng(n + k)
    b = bf(rng.standard_normal(n * k) * 0.02)
    codes, s, z = F.u4_quantize(b)
    cs, ps = F.u4_to_storage(codes, s, z, n, k)
    c2, s2, z2 = F.u4_from_storage(cs, ps, n, k)
    assert np.array_equal(c2, codes) and np.array_equal(s2, s) and np.array_equal(z2, z)
    pos = nf4.storage_positions(n, k)
    assert np.array_equal(cs.reshape(-1, 32)[pos[1]], codes.reshape(-1, 32)[1])
    assert ps[pos[1], 0] == s[1] and ps[pos[1], 1] == z[1]
    q, d16 = F.q8_quantize(b)
    qs, ds = F.q8_to_storage(q, d16, n, k)
    q2, d2 = F.q8_from_storage(qs, ds, n, k)
    assert np.array_equal(q2, q) and np.array_equal(d2, d16)
    assert np.array_equal(qs.reshape(-1, 64)[pos[1]], q.reshape(-1, 64)[1])
    assert ds[pos[1], 1] == d16[3]
