"""Oracle: the plain (flat) layout of a packed weight.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).  Plain numpy, no
arithmetic beyond moving bytes.

The pages fix what a packed 4-bit weight holds -- two 4-bit codes per uint8
byte, one constant per block of the flat row-major weight [rkmt §4.2 (4-bit
data in uint8 storage), §1.2 (one scale per 64-block), §2.2 (second-level
constants per group of block scales)] -- but no nibble order and no order of
the blocks in memory.  The library stores its own order (``nf4`` steps 3 and
6, ``formats`` storage); the plain layout is the order a producer that knows
only the pages would write, and the one ``qlora_to_plain`` /
``qlora_from_plain`` convert to and from:

* codes, 4-bit formats: the row-major element stream, two codes per byte,
  byte j = code(2j) | code(2j+1) << 4 (the even element in the low nibble --
  the reading that keeps element order in byte order; the pages are silent).
* codes, Q8_0: byte e = the int8 value of element e, row-major.
* block constants in flat block order, block b = row * (k / block) + kb:
  NF4 with double quantization -- ``qscale[b]`` (8 bits) and ``step[g]`` per
  group of 256 flat blocks (already flat in the library layout); NF4 without
  it -- ``step[b]`` the fp32 absmax; uint4 -- ``step[2b], step[2b+1]`` the fp32
  (scale, zero-point) of 64-block b; Q8_0 -- ``qscale`` bytes [2b, 2b+2) the
  little-endian fp16 scale of 32-block b.

The arrays have the same sizes in both layouts; only the order of their bytes
differs.
"""
from __future__ import annotations

import numpy as np

from . import formats as F
from . import nf4


def pack_plain(code: np.ndarray) -> np.ndarray:
    """Element codes (flat, even count) -> bytes, byte j = code(2j) | code(2j+1) << 4."""
    c = np.asarray(code, dtype=np.uint8).reshape(-1, 2)
    return (c[:, 0] | (c[:, 1] << 4)).astype(np.uint8)


def unpack_plain(codes: np.ndarray) -> np.ndarray:
    b = np.asarray(codes, dtype=np.uint8).reshape(-1)
    out = np.empty((b.size, 2), dtype=np.uint8)
    out[:, 0] = b & 0x0F
    out[:, 1] = b >> 4
    return out.reshape(-1)


def nf4_plain(codes, scales, step=None):
    """The oracle's flat-order NF4 arrays (``nf4.quantize``: word-layout code
    bytes, 8-bit block scales and group constants; or ``nf4.quantize_nodq``:
    codes and fp32 absmax, step None) -> plain (codes, qscale, step): qscale
    None without double quantization, the absmax then in step."""
    c = pack_plain(nf4.unpack(codes))
    if step is None:
        return c, None, np.asarray(scales, dtype=np.float32).copy()
    return c, np.asarray(scales, dtype=np.uint8).copy(), np.asarray(step, dtype=np.float32).copy()


def u4_plain(codes, scale, zp):
    """``formats.u4_quantize`` output -> plain (codes, step[2b] = scale, step[2b+1] = zp)."""
    c = pack_plain(nf4.unpack(codes))
    st = np.stack([np.asarray(scale, np.float32), np.asarray(zp, np.float32)], axis=1).reshape(-1)
    return c, st


def q8_plain(q, d16):
    """``formats.q8_quantize`` output -> plain (codes bytes, scale bytes)."""
    c = np.asarray(q, dtype=np.int8).view(np.uint8).copy()
    s = np.asarray(d16, dtype=np.float16).astype("<f2").view(np.uint8).copy()
    return c, s


def nf4_storage(codes, scales, step, n: int, k: int, block: int = nf4.BLOCK):
    """The same flat-order NF4 arrays -> the library layout (codes, qscale, step)."""
    cs = nf4.blocks_to_storage(np.asarray(codes, dtype=np.uint8).reshape(-1, 32), n, k).reshape(-1)
    if step is None:
        return cs, None, nf4.scales_to_storage(np.asarray(scales, dtype=np.float32), n, k, block)
    return cs, nf4.scales_to_storage(np.asarray(scales, dtype=np.uint8), n, k, block), \
        np.asarray(step, dtype=np.float32).copy()


def u4_storage(codes, scale, zp, n: int, k: int):
    c, p = F.u4_to_storage(codes, scale, zp, n, k)
    return c, np.asarray(p, dtype=np.float32).reshape(-1)


def q8_storage(q, d16, n: int, k: int):
    c, s = F.q8_to_storage(q, d16, n, k)
    return c.view(np.uint8), np.asarray(s, dtype=np.float16).astype("<f2").view(np.uint8).reshape(-1)
