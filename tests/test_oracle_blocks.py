"""Pins of the NF4 oracle at block sizes 32 and 128 (CPU only): closed-form
sizes, hand-made blocks, reductions to the 64-block format, the derived error
bound and the storage order of the scales."""
import numpy as np
import pytest

from oracle import nf4


LV, MID = nf4.codebook()


def bf(x):
    return nf4.f32_to_bf16_rne(np.asarray(x, dtype=np.float32).reshape(-1))


def f(bits):
    return nf4.bf16_to_f32(np.asarray(bits, dtype=np.uint16)).astype(np.float64)


def nearest_level(v):
    return int(np.argmin(np.abs(LV.astype(np.float64) - v)))


@pytest.mark.parametrize("block,bits", [(32, 4 + 8 / 32 + 32 / (32 * 256)), (64, 4 + 8 / 64 + 32 / (64 * 256)),
                                        (128, 4 + 8 / 128 + 32 / (128 * 256))])
def test_sizes_closed_form(block, bits):
    # rkmt §1.2: smaller blocks quantize more finely and carry more constants
    n, k = 4096, 4096
    c, q, s = nf4.nf4_bytes(n, k, block)
    assert c == n * k // 2 and q == n * k // block and s == 4 * (-(-(n * k // block) // 256))
    assert (c + q + s) * 8 / (n * k) == pytest.approx(bits)
    assert nf4.bits_per_param(block=block) == pytest.approx(bits)
    assert nf4.bits_per_param(block=block, double_quant=False) == 4 + 32 / block


def test_block128_scales_two_units_together():
    # first 64 weights peak at 0.5, the next 64 at 1.0: with block 128 both
    # halves are normalized by 1.0, so 0.5 encodes to the level nearest 0.5;
    # with block 64 it is the first unit's maximum and encodes to code 15
    x = np.zeros(128, np.float32)
    x[10], x[100] = 0.5, 1.0
    c128, am128 = nf4.quantize_nodq(bf(x), MID, block=128)
    c64, am64 = nf4.quantize_nodq(bf(x), MID, block=64)
    assert list(am128) == [1.0] and list(am64) == [0.5, 1.0]
    assert nf4.unpack(c128)[10] == nearest_level(0.5)
    assert nf4.unpack(c64)[10] == 15 and nf4.unpack(c128)[100] == 15


def test_block32_scales_each_half():
    x = np.zeros(64, np.float32)
    x[5], x[40] = 0.25, -2.0
    c32, am32 = nf4.quantize_nodq(bf(x), MID, block=32)
    assert list(am32) == [0.25, 2.0]
    code = nf4.unpack(c32)
    assert code[5] == 15 and code[40] == 0 and code[0] == 7 and code[33] == 7
    w = f(nf4.dequantize_nodq(c32, am32, LV, block=32))
    assert w[5] == 0.25 and w[40] == -2.0


@pytest.mark.parametrize("block", [32, 128])
def test_equal_absmax_reduces_to_64_blocks(block):
    # when every block of the other size has the same absmax as the 64-blocks
    # it overlaps, the codes and the dequantized weights are those of block 64
    rng = np.random.default_rng(block)
    x = (rng.standard_normal((8, 256)) * 0.02).astype(np.float32)
    x = x.reshape(-1, 32)
    x[:, 0] = 0.1                     # the same maximum in every 32 weights
    b = bf(x)
    c, q, s = nf4.quantize(b, MID, block=block)
    c64, q64, s64 = nf4.quantize(b, MID)
    assert np.array_equal(c, c64)
    assert np.array_equal(nf4.dequantize(c, q, s, LV, block=block), nf4.dequantize(c64, q64, s64, LV))


@pytest.mark.parametrize("dq", [True, False])
def test_error_bound_and_block_size_ordering(dq):
    rng = np.random.default_rng(9)
    x = (rng.standard_normal(128 * 512) * 0.015).astype(np.float32)
    idx = rng.choice(x.size, 70, replace=False)
    x[idx] *= 20
    b = bf(x)
    means = []
    for block in (32, 64, 128):
        if dq:
            c, q, s = nf4.quantize(b, MID, block=block)
            w = f(nf4.dequantize(c, q, s, LV, block=block))
        else:
            c, am = nf4.quantize_nodq(b, MID, block=block)
            w = f(nf4.dequantize_nodq(c, am, LV, block=block))
        err = np.abs(w - f(b))
        assert np.all(err <= nf4.dequant_error_bound(b, LV, double_quant=dq, block=block))
        means.append(err.mean())
    assert means[0] < means[1] < means[2]      # smaller blocks, finer quantization


def test_scale_storage_orders_by_hand():
    n, k = 3, 256
    # block 128: 2 block columns, 3 rows in the one row group: (row, kb) -> kb * 3 + row
    a = np.arange(6, dtype=np.float32)           # flat: row 0 kb 0, row 0 kb 1, row 1 kb 0, ...
    st = nf4.scales_to_storage(a, n, k, 128)
    assert list(st) == [0, 2, 4, 1, 3, 5]
    assert np.array_equal(nf4.scales_from_storage(st, n, k, 128), a)
    # block 32: the pair of each 64-unit moves with the unit (unit order kb * 3 + row)
    a = np.arange(24, dtype=np.float32)          # 8 32-blocks per row
    st = nf4.scales_to_storage(a, n, k, 32)
    assert list(st[:6]) == [0, 1, 8, 9, 16, 17] and list(st[6:8]) == [2, 3]
    assert np.array_equal(nf4.scales_from_storage(st, n, k, 32), a)
