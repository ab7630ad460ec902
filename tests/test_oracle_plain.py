"""Pins of the plain-layout oracle (``oracle/plain.py``): hand bytes of the
plain nibble order, hand positions of the library's block order, and the
element codes both layouts carry.  CPU only."""
import numpy as np

import synth
from oracle import formats as F
from oracle import nf4
from oracle import plain as P


def test_pack_plain_hand_bytes():
    codes = np.arange(16, dtype=np.uint8)
    # byte j = code(2j) | code(2j+1) << 4
    assert list(P.pack_plain(codes)) == [0x10, 0x32, 0x54, 0x76, 0x98, 0xBA, 0xDC, 0xFE]
    assert list(P.pack_plain(np.array([15, 0, 0, 15], dtype=np.uint8))) == [0x0F, 0xF0]
    c = synth.rng(11).integers(0, 16, 4096).astype(np.uint8)
    assert np.array_equal(P.unpack_plain(P.pack_plain(c)), c)


def test_plain_and_word_layouts_hold_the_same_codes():
    c = synth.rng(12).integers(0, 16, 64 * 10).astype(np.uint8)
    word = nf4.pack(c)
    pl, _, _ = P.nf4_plain(word, np.zeros(10, np.uint8), np.zeros(1, np.float32))
    assert np.array_equal(P.unpack_plain(pl), c)
    # the two byte orders differ (the same bytes would make the conversion moot)
    assert not np.array_equal(pl, word)
    # element 1 sits in the high nibble of plain byte 0 and in the low nibble
    # of word byte 1
    assert pl[0] >> 4 == c[1] and word[1] & 0xF == c[1]


def _hand_position(row, kb, n, nkb):
    """Storage position of unit (row, kb): rows in groups of 16 (the last
    group R = n - g0 rows), inside a group k-block-major."""
    g0 = 16 * (row // 16)
    R = min(16, n - g0)
    return g0 * nkb + kb * R + (row - g0)


def test_storage_order_hand_positions():
    n, k = 20, 128                      # two row groups: 16 rows and 4 rows
    nkb = k // 64
    assert _hand_position(17, 1, n, nkb) == 16 * 2 + 1 * 4 + 1 == 37
    assert _hand_position(3, 1, n, nkb) == 16 + 3
    rng = synth.rng(13)
    codes = rng.integers(0, 256, n * k // 2).astype(np.uint8)       # flat word-layout bytes
    qs = rng.integers(0, 256, n * nkb).astype(np.uint8)
    st = rng.random(1).astype(np.float32)
    c_s, q_s, s_s = P.nf4_storage(codes, qs, st, n, k)
    for row in (0, 3, 15, 16, 17, 19):
        for kb in range(nkb):
            p, f = _hand_position(row, kb, n, nkb), row * nkb + kb
            assert np.array_equal(c_s[32 * p:32 * p + 32], codes[32 * f:32 * f + 32])
            assert q_s[p] == qs[f]
    assert np.array_equal(s_s, st)


def test_single_level_and_block_sizes():
    n, k = 5, 256
    rng = synth.rng(14)
    codes = rng.integers(0, 256, n * k // 2).astype(np.uint8)
    # single level, block 64: the fp32 absmax follows the unit order; plain keeps it flat
    am = rng.random(n * k // 64).astype(np.float32)
    c_s, q_s, s_s = P.nf4_storage(codes, am, None, n, k)
    assert q_s is None
    nkb = k // 64
    for row in range(n):
        for kb in range(nkb):
            assert s_s[_hand_position(row, kb, n, nkb)] == am[row * nkb + kb]
    pc, pq, ps = P.nf4_plain(codes, am)
    assert pq is None and np.array_equal(ps, am)
    # block 32: the unit's two scales at 2p, 2p + 1
    q32 = rng.integers(0, 256, n * k // 32).astype(np.uint8)
    _, q_s, _ = P.nf4_storage(codes, q32, np.zeros(1, np.float32), n, k, block=32)
    for row in range(n):
        for kb in range(nkb):
            p, f = _hand_position(row, kb, n, nkb), row * nkb + kb
            assert q_s[2 * p] == q32[2 * f] and q_s[2 * p + 1] == q32[2 * f + 1]
    # block 128: one scale per unit pair, the same row-group order over k/128 columns
    q128 = rng.integers(0, 256, n * k // 128).astype(np.uint8)
    _, q_s, _ = P.nf4_storage(codes, q128, np.zeros(1, np.float32), n, k, block=128)
    for row in range(n):
        for kb in range(k // 128):
            assert q_s[_hand_position(row, kb, n, k // 128)] == q128[row * (k // 128) + kb]


def test_u4_and_q8_plain_hand_values():
    w = np.zeros((1, 128), dtype=np.float32)
    w[0, :64] = np.linspace(-2, 2, 64)
    w[0, 64:] = np.linspace(0, 1, 64)
    bits = nf4.f32_to_bf16_rne(w.reshape(-1))
    codes, scale, zp = F.u4_quantize(bits)
    pc, ps = P.u4_plain(codes, scale, zp)
    assert list(ps) == [scale[0], zp[0], scale[1], zp[1]]
    assert zp[0] == 8 and zp[1] == 0           # [-2, 2] and [0, 1] blocks
    assert np.array_equal(P.unpack_plain(pc), nf4.unpack(codes))
    q = np.array([-1, 1, 127, -127] + [0] * 60, dtype=np.int8)
    d16 = np.array([1.0, 0.5], dtype=np.float16)
    qc, qsb = P.q8_plain(q, d16)
    assert list(qc[:4]) == [0xFF, 0x01, 0x7F, 0x81]
    assert list(qsb) == [0x00, 0x3C, 0x00, 0x38]   # fp16 1.0 = 0x3C00, 0.5 = 0x3800, little-endian
    c_s, s_s = P.q8_storage(q, d16, 1, 64)
    assert np.array_equal(c_s, qc) and np.array_equal(s_s, qsb)   # one unit: same order
