"""Oracle: the two alternate block formats of the frozen base weight --
asymmetric 4-bit min/max blocks and Q8_0 blocks.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).  Plain numpy; every
floating-point step that decides an integer is done in IEEE binary32 (or the
binary16 rounding it names) exactly as stated; the rest is exact.

Asymmetric uint4, block 64 [rkmt §1.3, §2.1; kwkr §2.1]
------------------------------------------------------
Each 64-element block of the flat row-major weight is mapped onto the 16
integers 0..15 by a scale and a zero-point, both kept as fp32 (8 bytes per
block, 1 bit per weight on top of the 4-bit codes).
1. Range: ``lo = min(min_b, 0)``, ``hi = max(max_b, 0)``.  Reading: the range
   is widened to hold 0, so that the zero-point lies in [0, 15] and 0 is
   represented exactly (kwkr §2.1 gives exact zero as the point of the
   zero-point; rkmt §2.1 leaves a block of one sign open).
2. ``scale = fp32(fp32(hi - lo) / 15)`` [rkmt §2.1: (max - min) / 15].
3. ``zp = clamp(rint_even(-lo * 15 / (hi - lo)), 0, 15)`` [rkmt §2.1:
   round(-min / scale)], evaluated in float64 from the range, stored as an
   fp32 integer value.  Reading: -min / scale taken with the real scale
   (hi - lo) / 15, the same reading as the affine unit (``affine.params``),
   which is the one that reproduces kwkr §2.1's printed zero-point 128 for
   [-2, 2]; the quotient by the fp32-rounded scale would give 127 there, and
   7 instead of 8 for a [-2, 2] uint4 block.
4. ``q = clamp(rint_even(fp32(x / scale)) + zp, 0, 15)`` [kwkr §2.1 forward
   formula; the clamp is the reading of the affine unit: the pages are silent].
   A block with scale 0 (all zero) gets zp = 0 and q = 0.
5. Dequantize: ``w = bf16_rne(fp32(scale * (q - zp)))``.  Reading: rkmt §2.1
   prints the inverse as "q x scale + zero-point", which does not invert step
   4; kwkr §2.1's ``r = scale (q - zero_point)`` does, and is used.
Codes are packed two per byte exactly as the NF4 codes (``nf4.pack``).

Q8_0, block 32 [cf1 §1.1, §2.2; kwkr §2.1]
-----------------------------------------
Each 32-element block keeps 32 signed 8-bit values and one fp16 scale (34 bytes
per 32 weights, "a little over one byte" per weight).  Reading: the block is
quantized symmetrically (kwkr §2.1: zero-point 0, scale = max(|r|) / 127):
1. ``d = fp32(absmax_b / 127)``, ``d16 = fp16_rne(d)`` (the stored scale).
2. ``q = clamp(rint_even(fp32(x / fp32(d16))), -127, 127)``, 0 when d16 is 0.
3. Dequantize: ``w = bf16_rne(fp32(d16) * q)`` (the product is exact in fp32:
   11 + 7 significant bits).
Blocks whose absmax exceeds 127 * 65504 (d16 would overflow) are outside the
contract.

Storage (a layout choice of this implementation, as for NF4): the weight is
cut into 64-element units (row, kb) -- one uint4 block, or two Q8_0 blocks --
and the units are stored in the NF4 block order (``nf4.storage_positions``).
Per unit: uint4 -- 32 code bytes and the pair (scale, zp) as two float32;
Q8_0 -- 64 code bytes (int8, element order) and the two fp16 scales of its
blocks (elements 0-31, then 32-63).
"""
from __future__ import annotations

import numpy as np

from .nf4 import bf16_to_f32, blocks_to_storage, f32_to_bf16_rne, pack, storage_positions, unpack

U4_BLOCK = 64
Q8_BLOCK = 32
UNIT = 64       # elements per storage unit (one row, 64 consecutive k)


def _blocks(w_bits: np.ndarray, size: int) -> np.ndarray:
    flat = np.asarray(w_bits, dtype=np.uint16).reshape(-1)
    if flat.size % UNIT:
        raise ValueError("numel must be a multiple of 64")
    x = bf16_to_f32(flat).reshape(-1, size)
    if not np.all(np.isfinite(x)):
        raise ValueError("non-finite weights are outside the contract")
    return x


# --------------------------------------------------------------------------
# asymmetric uint4
# --------------------------------------------------------------------------
def u4_quantize(w_bits: np.ndarray):
    """bf16 weight bits (numel % 64 == 0) -> (codes uint8[numel/2] packed as
    NF4, scale float32[nb], zp float32[nb]), flat block order."""
    x = _blocks(w_bits, U4_BLOCK)
    # step 1: the block range, widened to hold 0
    lo = np.minimum(np.min(x, axis=1), np.float32(0)).astype(np.float32)
    hi = np.maximum(np.max(x, axis=1), np.float32(0)).astype(np.float32)
    # step 2: binary32 subtraction and division
    scale = np.divide((hi - lo).astype(np.float32), np.float32(15.0), dtype=np.float32)
    live = scale > 0
    safe = np.where(live, scale, np.float32(1)).astype(np.float32)
    # step 3: zero-point, an integer value in [0, 15] (0 for an all-zero
    # block): float64 from the range (15 * lo is exact, the subtraction and
    # the division round once each)
    lo64, hi64 = lo.astype(np.float64), hi.astype(np.float64)
    span = np.where(live, hi64 - lo64, 1.0)
    z = np.rint((-lo64 * 15.0) / span)
    zp = np.where(live, np.clip(z, 0, 15), 0).astype(np.int64)
    # step 4: codes
    qv = np.rint(np.divide(x, safe[:, None], dtype=np.float32)).astype(np.int64) + zp[:, None]
    code = np.where(live[:, None], np.clip(qv, 0, 15), 0).astype(np.uint8)
    return pack(code.reshape(-1)), np.where(live, scale, 0).astype(np.float32), zp.astype(np.float32)


def u4_dequantize(codes, scale, zp) -> np.ndarray:
    """-> bf16 bits (flat): bf16_rne(fp32(scale * (q - zp)))."""
    q = unpack(codes).astype(np.float32).reshape(-1, U4_BLOCK)
    d = (q - np.asarray(zp, dtype=np.float32)[:, None]).astype(np.float32)   # small integers, exact
    prod = (d * np.asarray(scale, dtype=np.float32)[:, None]).astype(np.float32)
    return f32_to_bf16_rne(prod.reshape(-1))


def u4_error_bound(w_bits: np.ndarray, scale: np.ndarray) -> np.ndarray:
    """Per-element bound on |w - deq(q(w))| (float64), from the steps: the
    integer grid has spacing `scale`, every value of the widened range lies
    within half a spacing of a grid point inside [0, 15] (the end points sit
    at most half a spacing beyond the grid, since |zp - (-lo/scale)| <= 1/2),
    the binary32 quotient and range add a few ulps, and the result is rounded
    to fp32 and then to bf16 (half an ulp of 2^-8 relative, plus 2^-24)."""
    x = bf16_to_f32(np.asarray(w_bits).reshape(-1)).astype(np.float64)
    s = np.repeat(np.asarray(scale, dtype=np.float64), U4_BLOCK)
    grid = s * (0.5 + 2.0 ** -18)
    return grid + (np.abs(x) + grid) * (2.0 ** -8 + 2.0 ** -23)


# --------------------------------------------------------------------------
# Q8_0
# --------------------------------------------------------------------------
def q8_quantize(w_bits: np.ndarray):
    """bf16 weight bits (numel % 64 == 0) -> (q int8[numel], d16 float16[numel/32]),
    flat block order."""
    x = _blocks(w_bits, Q8_BLOCK)
    absmax = np.max(np.abs(x), axis=1).astype(np.float32)
    d = np.divide(absmax, np.float32(127.0), dtype=np.float32)
    d16 = d.astype(np.float16)                      # round to nearest even
    if not np.all(np.isfinite(d16)):
        raise ValueError("block scale overflows fp16: outside the contract")
    df = d16.astype(np.float32)
    safe = np.where(df == 0, np.float32(1), df).astype(np.float32)
    qv = np.rint(np.divide(x, safe[:, None], dtype=np.float32))
    qv = np.where((df == 0)[:, None], 0.0, qv)
    return np.clip(qv, -127, 127).astype(np.int8).reshape(-1), d16


def q8_dequantize(q, d16) -> np.ndarray:
    """-> bf16 bits (flat): bf16_rne(fp32(d16) * q)."""
    qf = np.asarray(q, dtype=np.int8).astype(np.float32).reshape(-1, Q8_BLOCK)
    prod = (qf * np.asarray(d16, dtype=np.float16).astype(np.float32)[:, None]).astype(np.float32)
    return f32_to_bf16_rne(prod.reshape(-1))


def q8_error_bound(w_bits: np.ndarray, d16: np.ndarray) -> np.ndarray:
    """Per-element bound: half a grid step (plus a few ulps for the binary32
    quotient) while |x| <= 127.5 d16; beyond the last grid point (a block whose
    scale rounded down in fp16, which only the subnormal range can push that
    far) the distance to 127 d16; then the bf16 rounding of the result."""
    x = bf16_to_f32(np.asarray(w_bits).reshape(-1)).astype(np.float64)
    d = np.repeat(np.asarray(d16, dtype=np.float16).astype(np.float64), Q8_BLOCK)
    grid = np.maximum(d * (0.5 + 2.0 ** -17), np.abs(x) - 127.0 * d)
    return grid + (np.abs(x) + grid) * (2.0 ** -8 + 2.0 ** -23)


# --------------------------------------------------------------------------
# sizes and storage order
# --------------------------------------------------------------------------
def u4_bytes(n: int, k: int) -> tuple[int, int]:
    """(code bytes, fp32 scale + zero-point bytes) of an n x k weight."""
    nb = n * k // U4_BLOCK
    return n * k // 2, 8 * nb


def q8_bytes(n: int, k: int) -> tuple[int, int]:
    """(int8 code bytes, fp16 scale bytes) of an n x k weight."""
    return n * k, 2 * (n * k // Q8_BLOCK)


def u4_to_storage(codes, scale, zp, n: int, k: int):
    """Flat-order uint4 arrays -> (codes uint8[n*k/2], params float32[nunits, 2])
    in storage order."""
    c = blocks_to_storage(np.asarray(codes, dtype=np.uint8).reshape(-1, 32), n, k)
    p = blocks_to_storage(np.stack([np.asarray(scale, np.float32), np.asarray(zp, np.float32)], 1), n, k)
    return c.reshape(-1), p


def q8_to_storage(q, d16, n: int, k: int):
    """Flat-order Q8_0 arrays -> (codes int8[n*k], scales float16[nunits, 2])
    in storage order."""
    c = blocks_to_storage(np.asarray(q, dtype=np.int8).reshape(-1, UNIT), n, k)
    s = blocks_to_storage(np.asarray(d16, dtype=np.float16).reshape(-1, 2), n, k)
    return c.reshape(-1), s


def u4_from_storage(codes, params, n: int, k: int):
    pos = storage_positions(n, k)
    c = np.asarray(codes, dtype=np.uint8).reshape(-1, 32)[pos]
    p = np.asarray(params, dtype=np.float32).reshape(-1, 2)[pos]
    return c.reshape(-1), p[:, 0].copy(), p[:, 1].copy()


def q8_from_storage(codes, scales, n: int, k: int):
    pos = storage_positions(n, k)
    c = np.asarray(codes, dtype=np.int8).reshape(-1, UNIT)[pos]
    s = np.asarray(scales, dtype=np.float16).reshape(-1, 2)[pos]
    return c.reshape(-1), s.reshape(-1)
