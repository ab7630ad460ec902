"""Oracle: NF4 blockwise quantization with double quantization (DQ).

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).  Plain numpy; every
floating-point step that decides an integer is done in IEEE binary32 exactly as
stated below, everything else in float64.

What is computed, in the pages' order
-------------------------------------
1. Block-wise first level [rkmt §1.2, §2.1; zky "three parts"]: the flat
   row-major weight is cut into fixed 64-element blocks; each block gets its own
   scale, its absolute maximum ``absmax_b`` (an fp32 value; exact, since the
   weights are bf16).
2. NF4 encode [zky "NF4"; lqnn §2.1]: each element is normalized by its block's
   absmax into [-1, 1] (binary32 division, correctly rounded) and mapped to the
   nearest of the 16 NF4 levels.  Ties go to the lower code.  An all-zero block
   (absmax 0) encodes every element as the level 0.
3. Packing [rkmt §4.2: 4-bit data packed in uint8 storage]: two codes per
   byte.  Reading (the pages fix no nibble order): within each 4-byte word that
   holds elements 8w .. 8w+7, byte j (j = 0..3) holds code(8w+j) in bits 0-3 and
   code(8w+j+4) in bits 4-7.
4. Double quantization [rkmt §1.3, §2.2, §2.3; zky "double quantization"]:
   the block absmax values are quantized again to 8 bits in groups of 256
   consecutive blocks, each group keeping one fp32 second-level constant.
   Reading: unsigned, scale only (the scales are non-negative, so the range
   [0, c2] has zero-point 0): ``step_g = fp32(c2 / 255)`` with ``c2`` the group's
   largest absmax, ``qscale_b = min(255, rint_even(fp32(absmax_b / step_g)))``
   (0 when step_g is 0).  The first-level zero-point is not stored: NF4 is
   absmax-symmetric and has an exact zero level.
5. Dequantization [lqnn §3.3; zky "a counter-intuitive combination"]:
   ``s'_b = fp32(qscale_b * step_g)``, ``w = bf16_rne(fp32(level[code] * s'_b))``.
6. Storage order (a layout choice of this implementation; the pages fix only
   that the 4-bit codes live in uint8 storage, rkmt §4.2): the 32 code bytes
   and the 8-bit scale of each block are stored with the rows taken in groups
   of 16 and, inside a group, the blocks ordered by k-block, then by row.  The
   fp32 second-level constants stay indexed by the flat block.  ``quantize``
   returns the flat (logical) order; ``to_storage`` / ``from_storage`` convert.

Other block sizes [rkmt §1.2: smaller blocks quantize more finely and cost
more constants; zky "double quantization"]: every step above runs on blocks of
32 or 128 consecutive weights instead of 64 (``block=``), second-level groups
still holding 256 block scales.  Codes keep the 64-weight word layout and unit
order; the scales are stored with ``scales_to_storage``: block 32 as the pair of
scales of a 64-weight unit at 2p, 2p + 1 (p the unit's position), block 128 in
the row-group order over the k/128 block columns.

Without double quantization [rkmt §1.2, §2.3: one fp32 scale per 64-block,
0.5 bit per parameter; zky "double quantization" names the saving]: steps 1-3
only; the block keeps its fp32 absmax as the scale (``quantize_nodq``), and
``w = bf16_rne(fp32(level[code] * absmax_b))`` (``dequantize_nodq``).  The
absmax array uses the same storage order as the 8-bit scales
(``blocks_to_storage``).

The codebook [zky "NF4": levels placed by the normal distribution so that each
level receives about the same share of weights; kwkr §2.1: zero must be exactly
representable].  Reading: 8 positive levels Phi^-1(p_j) for p_j equally spaced
in (0.5, 1 - 1/32], 7 negative levels -Phi^-1(q_j) for q_j equally spaced in
(0.5, 1 - 1/30], an exact 0, each side divided by its largest magnitude so the
table spans [-1, 1]; computed in float64 and rounded to fp32.  Midpoint k is the
largest fp32 not above the exact mean of levels k and k+1, so that
``code = #{k : v > mid[k]}`` is exactly "nearest level, ties to the lower code"
for every fp32 v.

Compute type [rkmt §3.3: the compute dtype is float16 or bfloat16; kwkr §4.3:
fall back to fp16 where bf16 is unsupported]: the dequantized weight is
rounded (nearest, ties to even) to the compute type instead of bf16, and a
weight given in fp16 is read as fp16 (``dtype="f16"``); codes and scales are
computed the same way from the exact fp32 values.

Parity unpinned: the level values themselves rest on the construction rule
(the pages print no table); the 8-bit second-level format is pinned by the
closed-form storage sizes only.
"""
from __future__ import annotations

import math

import numpy as np
from scipy.special import ndtri

BLOCK = 64      # elements per first-level block [rkmt §1.2]
GROUP = 256     # first-level scales per second-level group [rkmt §2.2]


# --------------------------------------------------------------------------
# bf16 <-> fp32, written from the definition of the formats
# --------------------------------------------------------------------------
def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """bf16 is the upper half of an fp32 bit pattern: widening is exact."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def f32_to_bf16_rne(x: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16, nearest with ties to even; NaN stays NaN (quiet)."""
    u = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    rounded = ((u + 0x7FFF + lsb) >> 16).astype(np.uint32)
    nan = np.isnan(np.asarray(x, dtype=np.float32))
    quiet = ((u >> 16) | 0x40).astype(np.uint32)
    return np.where(nan, quiet, rounded).astype(np.uint16)


# --------------------------------------------------------------------------
# IEEE binary16 (fp16) <-> fp32, written from the definition of the format
# [kwkr §1.1; lqnn §2.1: 1 sign bit, 5 exponent bits, 10 mantissa bits]
# --------------------------------------------------------------------------
def f16_to_f32(bits: np.ndarray) -> np.ndarray:
    """fp16 bits -> fp32 (exact: every fp16 value is an fp32 value).
    Exponent field 0: subnormal m * 2^-24; 31: infinity or NaN; otherwise
    (1024 + m) * 2^(e - 25)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.int64)
    sign = np.where(b >> 15, -1.0, 1.0)
    e = (b >> 10) & 0x1F
    m = b & 0x3FF
    mag = np.where(e == 0, np.ldexp(m.astype(np.float64), -24),
                   np.ldexp((1024 + m).astype(np.float64), (e - 25).astype(np.int64)))
    mag = np.where(e == 31, np.where(m == 0, np.inf, np.nan), mag)
    return (sign * mag).astype(np.float32)


def f32_to_f16_rne(x: np.ndarray) -> np.ndarray:
    """Round fp32 to fp16 bits, nearest with ties to even, subnormals kept,
    magnitudes from 65520 up to infinity, NaN to a quiet NaN.  The fp32 value
    is exact in float64; it is divided by the fp16 unit in the last place of
    its binade (2^-24 below 2^-14), a power of two, so the quotient is exact,
    and that quotient is rounded half to even."""
    v = np.asarray(x, dtype=np.float32).astype(np.float64)
    neg = np.signbit(v)
    a = np.abs(v)
    fin = np.isfinite(a)
    a0 = np.where(fin & (a > 0), a, 1.0)
    _, e = np.frexp(a0)                               # a = f * 2^e, f in [0.5, 1)
    ef = np.clip(e - 1, -14, 15)                      # binade exponent, floor(log2 a)
    ulp_exp = (ef - 10).astype(np.int64)
    q = np.ldexp(np.where(fin, a, 0.0), -ulp_exp)     # exact
    r = np.rint(q).astype(np.int64)                   # half to even
    val = np.ldexp(r.astype(np.float64), ulp_exp)
    bits = np.where(a < 2.0 ** -14, r, ((ef + 15).astype(np.int64) << 10) + r - 1024)
    bits = np.where(val > 65504.0, 0x7C00, bits)
    bits = np.where(np.isinf(a), 0x7C00, bits)
    bits = np.where(np.isnan(v), 0x7E00, bits)
    bits = bits | np.where(neg, 0x8000, 0)
    return bits.astype(np.uint16)


DTYPES = ("bf16", "f16")   # 16-bit compute types [rkmt §3.3; kwkr §4.3]


def widen(bits: np.ndarray, dtype: str = "bf16") -> np.ndarray:
    """16-bit weights or activations of the compute type -> fp32 (exact)."""
    if dtype == "bf16":
        return bf16_to_f32(bits)
    if dtype == "f16":
        return f16_to_f32(bits)
    raise ValueError(f"unknown compute dtype {dtype!r}")


def narrow(x: np.ndarray, dtype: str = "bf16") -> np.ndarray:
    """fp32 -> 16-bit bits of the compute type, round to nearest even."""
    if dtype == "bf16":
        return f32_to_bf16_rne(x)
    if dtype == "f16":
        return f32_to_f16_rne(x)
    raise ValueError(f"unknown compute dtype {dtype!r}")


# --------------------------------------------------------------------------
# codebook
# --------------------------------------------------------------------------
def codebook() -> tuple[np.ndarray, np.ndarray]:
    """Returns (levels float32[16] ascending, mids float32[15])."""
    p = np.linspace(0.5, 1.0 - 1.0 / 32.0, 9)[1:]        # 8 positive quantiles
    q = np.linspace(0.5, 1.0 - 1.0 / 30.0, 8)[1:]        # 7 negative quantiles
    pos = ndtri(p) / ndtri(1.0 - 1.0 / 32.0)
    neg = -ndtri(q) / ndtri(1.0 - 1.0 / 30.0)
    levels64 = np.concatenate([neg[::-1], [0.0], pos])
    levels = levels64.astype(np.float32)
    mids = np.empty(15, dtype=np.float32)
    for k in range(15):
        exact = (float(levels[k]) + float(levels[k + 1])) / 2.0   # exact in float64
        m = np.float32(exact)
        if float(m) > exact:                                       # round toward -inf
            m = np.nextafter(m, np.float32(-np.inf))
        mids[k] = m
    return levels, mids


# --------------------------------------------------------------------------
# storage sizes [rkmt §1.3, §2.3]
# --------------------------------------------------------------------------
def nf4_bytes(n: int, k: int, block: int = BLOCK) -> tuple[int, int, int]:
    """(code bytes, u8 scale bytes, fp32 second-level bytes) of an n x k weight."""
    numel = n * k
    if numel % BLOCK or numel % block:
        raise ValueError("numel must be a multiple of 64 and of the block")
    nblocks = numel // block
    ngroups = -(-nblocks // GROUP)
    return numel // 2, nblocks, 4 * ngroups


# --------------------------------------------------------------------------
# quantize / dequantize
# --------------------------------------------------------------------------
def encode(v: np.ndarray, mids: np.ndarray) -> np.ndarray:
    """Nearest NF4 level of normalized fp32 values, ties to the lower code."""
    v = np.asarray(v, dtype=np.float32)
    code = np.zeros(v.shape, dtype=np.uint8)
    for k in range(15):
        code += (v > mids[k]).astype(np.uint8)
    return code


def pack(code: np.ndarray) -> np.ndarray:
    """Codes (one per element, flat) -> bytes, in the word layout of step 3."""
    c = np.asarray(code, dtype=np.uint8).reshape(-1, 8)
    lo = c[:, 0:4]
    hi = c[:, 4:8]
    return (lo | (hi << 4)).astype(np.uint8).reshape(-1)


def unpack(codes: np.ndarray) -> np.ndarray:
    b = np.asarray(codes, dtype=np.uint8).reshape(-1, 4)
    out = np.empty((b.shape[0], 8), dtype=np.uint8)
    out[:, 0:4] = b & 0x0F
    out[:, 4:8] = b >> 4
    return out.reshape(-1)


def storage_positions(n: int, k: int, width: int = BLOCK) -> np.ndarray:
    """Storage position of every flat block b = row * (k/width) + kb (step 6):
    group start g0 = 16 * (row // 16), R = min(16, n - g0) rows in the group,
    position g0 * (k/width) + kb * R + (row - g0)."""
    nkb = k // width
    row = np.arange(n, dtype=np.int64)[:, None]
    kb = np.arange(nkb, dtype=np.int64)[None, :]
    g0 = (row // 16) * 16
    rows_in_group = np.minimum(16, n - g0)
    return (g0 * nkb + kb * rows_in_group + (row - g0)).reshape(-1)


def to_storage(codes: np.ndarray, qscale: np.ndarray, n: int, k: int):
    """Flat-order (codes, qscale) of an n x k weight -> storage order."""
    pos = storage_positions(n, k)
    cs = np.empty((pos.size, 32), dtype=np.uint8)
    cs[pos] = np.asarray(codes, dtype=np.uint8).reshape(-1, 32)
    qs = np.empty(pos.size, dtype=np.uint8)
    qs[pos] = np.asarray(qscale, dtype=np.uint8)
    return cs.reshape(-1), qs


def from_storage(codes: np.ndarray, qscale: np.ndarray, n: int, k: int):
    """Storage-order (codes, qscale) -> flat order."""
    pos = storage_positions(n, k)
    cs = np.asarray(codes, dtype=np.uint8).reshape(-1, 32)[pos]
    return cs.reshape(-1), np.asarray(qscale, dtype=np.uint8)[pos]


def block_absmax(w_bits: np.ndarray, block: int = BLOCK, dtype: str = "bf16") -> np.ndarray:
    x = widen(np.asarray(w_bits).reshape(-1), dtype).reshape(-1, block)
    return np.max(np.abs(x), axis=1).astype(np.float32)


def quantize_nodq(w_bits: np.ndarray, mids: np.ndarray, block: int = BLOCK, dtype: str = "bf16"):
    """Steps 1-3 only: 16-bit weight bits of the compute type (numel % 64 == 0
    and % block == 0) -> (codes uint8[numel/2], absmax float32[numel/block]),
    flat order."""
    flat = np.asarray(w_bits, dtype=np.uint16).reshape(-1)
    if flat.size % BLOCK or flat.size % block:
        raise ValueError("numel must be a multiple of 64 and of the block")
    x = widen(flat, dtype).reshape(-1, block)
    if not np.all(np.isfinite(x)):
        raise ValueError("non-finite weights are outside the contract")
    # step 1: first-level scale per 64-block
    absmax = np.max(np.abs(x), axis=1).astype(np.float32)
    # step 2: normalize (binary32 division) and encode
    safe = np.where(absmax == 0, np.float32(1), absmax).astype(np.float32)
    v = np.divide(x, safe[:, None], dtype=np.float32)
    v = np.where((absmax == 0)[:, None], np.float32(0), v).astype(np.float32)
    code = encode(v, mids)
    # step 3: pack two codes per byte
    return pack(code.reshape(-1)), absmax


def dequantize_nodq(codes, absmax, levels, block: int = BLOCK, dtype: str = "bf16") -> np.ndarray:
    """-> 16-bit bits (flat): rne(fp32(level[code] * absmax_b)) in the compute type."""
    code = unpack(codes)
    s_el = np.repeat(np.asarray(absmax, dtype=np.float32), block)
    prod = (np.asarray(levels, dtype=np.float32)[code] * s_el).astype(np.float32)
    return narrow(prod, dtype)


def blocks_to_storage(per_block: np.ndarray, n: int, k: int) -> np.ndarray:
    """Flat-order per-block array (any dtype) -> storage order (step 6)."""
    pos = storage_positions(n, k)
    a = np.asarray(per_block)
    out = np.empty_like(a)
    out[pos] = a
    return out


def quantize(w_bits: np.ndarray, mids: np.ndarray, block: int = BLOCK, dtype: str = "bf16"):
    """16-bit weight bits of the compute type (any shape, numel % 64 == 0 and
    % block == 0) -> (codes uint8[numel/2], qscale uint8[numel/block], step
    float32[ngroups])."""
    codes, absmax = quantize_nodq(w_bits, mids, block, dtype)
    # step 4: second level over groups of 256 block scales
    nblocks = absmax.size
    ngroups = -(-nblocks // GROUP)
    qscale = np.empty(nblocks, dtype=np.uint8)
    step = np.empty(ngroups, dtype=np.float32)
    for g in range(ngroups):
        a = absmax[g * GROUP:(g + 1) * GROUP]
        c2 = np.max(a)
        st = np.float32(c2) / np.float32(255.0)
        step[g] = st
        if st == 0:
            qscale[g * GROUP:(g + 1) * GROUP] = 0
        else:
            qv = np.rint(np.divide(a, st, dtype=np.float32))
            qscale[g * GROUP:(g + 1) * GROUP] = np.minimum(qv, 255).astype(np.uint8)
    return codes, qscale, step


def block_scale(qscale: np.ndarray, step: np.ndarray) -> np.ndarray:
    """s'_b = fp32(qscale_b * step_g)."""
    q = np.asarray(qscale, dtype=np.uint8).astype(np.float32)
    g = np.arange(q.size) // GROUP
    return (q * np.asarray(step, dtype=np.float32)[g]).astype(np.float32)


def dequantize(codes, qscale, step, levels, block: int = BLOCK, dtype: str = "bf16") -> np.ndarray:
    """-> 16-bit bits (flat): rne(fp32(level[code] * s'_b)) in the compute type."""
    code = unpack(codes)
    s = block_scale(qscale, step)
    s_el = np.repeat(s, block)
    prod = (np.asarray(levels, dtype=np.float32)[code] * s_el).astype(np.float32)
    return narrow(prod, dtype)


def dequantize_f32(codes, qscale, step, levels) -> np.ndarray:
    return bf16_to_f32(dequantize(codes, qscale, step, levels))


def scales_to_storage(per_block: np.ndarray, n: int, k: int, block: int = BLOCK) -> np.ndarray:
    """Flat-order per-block scales (8-bit or fp32) of an n x k weight ->
    storage order (step 6 for other block sizes): block 64 at the unit's
    position; block 32 as the pair of its unit at 2p, 2p + 1; block 128 in the
    same row-group order over the k/128 block columns."""
    a = np.asarray(per_block)
    if block == BLOCK:
        return blocks_to_storage(a, n, k)
    if block == 32:
        return blocks_to_storage(a.reshape(-1, 2), n, k).reshape(-1)
    pos = storage_positions(n, k, width=block)
    out = np.empty_like(a)
    out[pos] = a
    return out


def scales_from_storage(stored: np.ndarray, n: int, k: int, block: int = BLOCK) -> np.ndarray:
    a = np.asarray(stored)
    if block == 32:
        return a.reshape(-1, 2)[storage_positions(n, k)].reshape(-1)
    return a[storage_positions(n, k, width=block)]


def dequant_error_bound(w_bits: np.ndarray, levels: np.ndarray,
                        double_quant: bool = True, block: int = BLOCK,
                        dtype: str = "bf16") -> np.ndarray:
    """Per-element bound on |w - deq(q(w))| (float64), derived from the steps,
    independent of how ``quantize`` is written:

    * encode: the normalized value lies in a codebook interval [L_i, L_i+1] and
      the nearest level is at most half that gap away, plus the rounding of the
      binary32 quotient (2^-24 relative)            -> absmax * (gap/2 + 2^-23)
    * double quantization: qscale * step is within half a step of absmax, plus
      the binary32 roundings of c2/255, absmax/step and qscale*step
                                                     -> 0.5*step + 2^-15*step + 2^-22*absmax
      (multiplied by |level| <= 1)
    * the binary32 product level*s' and the final rounding to the compute
      type                                           -> 2^-23 |w| + half an ulp of |w|
      (bf16: 8 significant bits; fp16: 11, and never below the subnormal
      half-ulp 2^-25)
    """
    flat = np.asarray(w_bits, dtype=np.uint16).reshape(-1)
    x = widen(flat, dtype).astype(np.float64).reshape(-1, block)
    absmax = np.max(np.abs(x), axis=1)
    nblocks = absmax.size
    ngroups = -(-nblocks // GROUP)
    c2 = np.array([absmax[g * GROUP:(g + 1) * GROUP].max() for g in range(ngroups)])
    step = (c2 / 255.0)[np.arange(nblocks) // GROUP]
    lv = np.asarray(levels, dtype=np.float64)
    v = np.where(absmax[:, None] > 0,
                 x / np.where(absmax > 0, absmax, 1.0)[:, None], 0.0)
    idx = np.clip(np.searchsorted(lv, v, side="right") - 1, 0, 14)
    gap = lv[idx + 1] - lv[idx]
    enc = absmax[:, None] * (0.5 * gap + 2.0 ** -23)
    dq = (0.5 * step + 2.0 ** -15 * step + 2.0 ** -22 * absmax)[:, None]
    if not double_quant:   # the block keeps its exact absmax
        dq = np.zeros_like(dq)
    wmax = np.abs(x) + enc + dq
    _, e = np.frexp(np.maximum(wmax, np.finfo(np.float64).tiny))
    if dtype == "f16":
        half_ulp = np.maximum(np.ldexp(1.0, e - 12), 2.0 ** -25)
    else:
        half_ulp = np.ldexp(1.0, e - 9)
    bound = enc + dq + 2.0 ** -23 * wmax + half_ulp
    return bound.reshape(-1)


def bits_per_param(block: int = BLOCK, group: int = GROUP, double_quant: bool = True,
                   scale_bytes: int = 4, zero_point_bytes: int = 0) -> float:
    """Storage per weight in bits: 4-bit code plus the constants' share."""
    if double_quant:
        return 4.0 + 8.0 / block + 8.0 * 4 / (block * group)
    return 4.0 + 8.0 * (scale_bytes + zero_point_bytes) / block


def model_bytes(params: float, double_quant: bool = True,
                zero_point_bytes: int = 0) -> dict:
    """Byte totals for a model of ``params`` weights, as in [rkmt §2.3]."""
    nblocks = params / BLOCK
    codes = params * 4 / 8
    if double_quant:
        consts = nblocks * 1 + math.ceil(nblocks / GROUP) * 4
    else:
        consts = nblocks * (4 + zero_point_bytes)
    return {"blocks": nblocks, "codes": codes, "constants": consts,
            "total": codes + consts}
