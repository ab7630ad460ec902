// Shared device helpers of the HIP path (gfx950 only).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kernels.h"

#define QL_DEV __device__ __forceinline__

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

namespace ql {

constexpr int kBlock = 64;    // weights per first-level block (and per storage unit)
constexpr int kGroup = 256;   // block scales per second-level group
constexpr int kWave = 64;

// Per-unit storage of each weight format (WFmt, kernels.h): each 64-weight
// unit (one row, 64 consecutive k) is stored at the NF4 block position
// (blk_pos); per unit:
//   kFmtNf4Dq  32 code bytes, an 8-bit scale; an fp32 constant per 256 units
//   kFmtNf4    32 code bytes, the fp32 absmax
//   kFmtU4     32 code bytes (uint4, NF4 packing), fp32 scale and zero-point
//   kFmtQ8     64 int8 bytes, two fp16 scales (elements 0-31, 32-63)
//   kFmtNf4DqF16  as kFmtNf4Dq; the dequantized weight is fp16
// NF4 at block 32 keeps two scales per unit (at 2p, 2p + 1), at block 128 one
// scale per two units of a row, stored in the same row-group order over the
// k/128 block columns.
template <int FMT>
struct FmtInfo {
  static constexpr bool nf4 = FMT != kFmtU4 && FMT != kFmtQ8;        // decodes through the codebook
  static constexpr bool dq = FMT == kFmtNf4Dq || FMT == kFmtNf4Dq32 || FMT == kFmtNf4Dq128 ||
                             FMT == kFmtNf4DqF16;
  static constexpr bool f16 = FMT == kFmtNf4DqF16;                   // fp16 compute type
  static constexpr int block = (FMT == kFmtNf4Dq32 || FMT == kFmtNf4_32)    ? 32
                               : (FMT == kFmtNf4Dq128 || FMT == kFmtNf4_128) ? 128
                                                                             : 64;
  static constexpr int code_bytes = FMT == kFmtQ8 ? 64 : 32;         // per unit
  // bytes of one scale entry: 8-bit scale, fp32 absmax, uint4 pair, Q8_0 pair
  static constexpr int param_bytes = dq ? 1 : (FMT == kFmtU4 ? 8 : 4);
};

// D[16x16] += A[16x32] * B[32x16], bf16 (F16: fp16) operands, fp32 accumulate.
// Lane l holds A[l%16][8(l/16) .. +7], B[8(l/16) .. +7][l%16] and
// D[4(l/16) .. +3][l%16] (layout measured on gfx950; the same for both types).
template <bool F16 = false>
QL_DEV f32x4_t mfma16x16x32(const u32x4_t a, const u32x4_t b, f32x4_t c) {
  if constexpr (F16)
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, a),
                                                  __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

// Global-memory view of a generic pointer.  Pointers loaded from memory
// (job tables) are generic to the compiler, which then emits flat loads; flat
// loads count in both the vector-memory and the LDS wait counters, so an LDS
// wait would also wait for them.
#define QL_GLOBAL __attribute__((address_space(1)))
#define QL_LDS __attribute__((address_space(3)))

// Raw buffer resource over `bytes` bytes from `base` (stride 0; loads past
// the end return zeros).  Built in scalar registers when `base` is uniform.
QL_DEV __amdgpu_buffer_rsrc_t buf_rsrc(const void* base, uint32_t bytes = 0x7FFFFFFFu) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                          0x00020000);
}
// Byte count of a buffer resource, clamped to the 31-bit range that every
// buffer offset here stays in.
QL_DEV uint32_t rsrc_bytes(int64_t b) { return (uint32_t)(b < 0x7FFFFFFF ? b : 0x7FFFFFFF); }
template <typename T>
QL_DEV const QL_GLOBAL T* gptr(const T* p) {
  return (const QL_GLOBAL T*)p;
}
template <typename T>
QL_DEV QL_GLOBAL T* gptr_w(T* p) {
  return (QL_GLOBAL T*)p;
}

QL_DEV uint32_t perm(uint32_t s0, uint32_t s1, uint32_t sel) {
  return __builtin_amdgcn_perm(s0, s1, sel);
}

typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// Two fp32 -> packed bf16 pair, round to nearest even, in one
// v_cvt_pk_bf16_f32.
QL_DEV uint32_t pack_bf16x2(float lo, float hi) {
  const bf16x2_t v = __builtin_convertvector(f32x2_t{lo, hi}, bf16x2_t);
  return __builtin_bit_cast(uint32_t, v);
}

QL_DEV uint16_t to_bf16(float x) { return __builtin_bit_cast(uint16_t, (__bf16)x); }
QL_DEV float bf16_lo(uint32_t v) { return __builtin_bit_cast(float, v << 16); }
QL_DEV float bf16_hi(uint32_t v) { return __builtin_bit_cast(float, v & 0xFFFF0000u); }

// The 16-bit compute type: bf16, or IEEE fp16 when F16.  Conversions from
// fp32 round to nearest even (fp16 subnormals kept, overflow to infinity);
// widening is exact.
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
template <bool F16>
QL_DEV uint32_t pack16x2(float lo, float hi) {
  if constexpr (F16)
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{lo, hi}, f16x2_t));
  else
    return pack_bf16x2(lo, hi);
}
template <bool F16>
QL_DEV uint16_t to16(float x) {
  if constexpr (F16)
    return __builtin_bit_cast(uint16_t, (_Float16)x);
  else
    return to_bf16(x);
}
template <bool F16>
QL_DEV float w16(uint32_t bits16) {   // the low 16 bits hold the value
  if constexpr (F16)
    return (float)__builtin_bit_cast(_Float16, (uint16_t)bits16);
  else
    return __builtin_bit_cast(float, bits16 << 16);
}
template <bool F16>
QL_DEV float lo16(uint32_t v) { return F16 ? w16<true>(v & 0xFFFFu) : bf16_lo(v); }
template <bool F16>
QL_DEV float hi16(uint32_t v) { return F16 ? w16<true>(v >> 16) : bf16_hi(v); }

// Per-block lookup table of the 16 dequantized 16-bit values, kept as byte
// planes so that a 4-bit code selects its byte with v_perm_b32:
//   lo[i] byte b = low byte of E[4i+b], hi[i] byte b = high byte of E[4i+b],
//   E[c] = rne(level[c] * s) in bf16, or fp16 for the F16 builders
//   (s = qscale * step of the block).
struct Lut {
  uint32_t lo[4], hi[4];
};

template <bool F16 = false>
QL_DEV Lut make_lut(const float* lv, float s) {
  uint32_t d[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) d[i] = pack16x2<F16>(lv[2 * i] * s, lv[2 * i + 1] * s);
  Lut t;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    t.lo[i] = perm(d[2 * i + 1], d[2 * i], 0x06040200u);
    t.hi[i] = perm(d[2 * i + 1], d[2 * i], 0x07050301u);
  }
  return t;
}

// Lookup table built by the four lanes of a DPP quad that share one block:
// lane q (= lane & 3) computes entries 4q..4q+3 and the planes lo[q], hi[q];
// quad broadcasts hand every lane all four planes.
QL_DEV uint32_t quad_bcast(uint32_t v, int j) {
  switch (j) {   // dpp quad_perm [j, j, j, j]
    case 0: return __builtin_amdgcn_mov_dpp(v, 0x00, 0xF, 0xF, false);
    case 1: return __builtin_amdgcn_mov_dpp(v, 0x55, 0xF, 0xF, false);
    case 2: return __builtin_amdgcn_mov_dpp(v, 0xAA, 0xF, 0xF, false);
    default: return __builtin_amdgcn_mov_dpp(v, 0xFF, 0xF, 0xF, false);
  }
}

// lvq[i] = level[4q + i] for this lane's quad position q.
template <bool F16 = false>
QL_DEV Lut make_lut_quad(const float* lvq, float s) {
  const uint32_t d0 = pack16x2<F16>(lvq[0] * s, lvq[1] * s);
  const uint32_t d1 = pack16x2<F16>(lvq[2] * s, lvq[3] * s);
  const uint32_t lo = perm(d1, d0, 0x06040200u), hi = perm(d1, d0, 0x07050301u);
  Lut t;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    t.lo[j] = quad_bcast(lo, j);
    t.hi[j] = quad_bcast(hi, j);
  }
  return t;
}

// Decode one packed word (elements 8w .. 8w+7: byte j = code j | code j+4 << 4)
// into 8 bf16 values in element order, as 4 packed pairs.  Each byte plane is
// looked up twice (entries 0-7 and 8-15, selected by the low three code
// bits), then a third v_perm picks, per byte, the lookup that matches code
// bit 3 (selector j or j+4).
// d = (a & m) | c in one v_and_or_b32: a VOP3 instruction takes no literal
// operand on this target and reads at most one scalar register, so the mask
// comes in a scalar register and the constant in a vector register.
QL_DEV uint32_t and_or(uint32_t a, uint32_t m, uint32_t c) {
  uint32_t d;
  asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(d) : "v"(a), "s"(m), "v"(c));
  return d;
}

QL_DEV u32x4_t decode8(const Lut& t, uint32_t x) {
  const uint32_t sa = x & 0x07070707u;                            // codes 0..3, low bits
  const uint32_t sb = (x >> 4) & 0x07070707u;                     // codes 4..7
  const uint32_t ka = and_or(x >> 1, 0x04040404u, 0x03020100u);   // bit 3 of codes 0..3
  const uint32_t kb = and_or(x >> 5, 0x04040404u, 0x03020100u);   // bit 3 of codes 4..7
  const uint32_t loa = perm(perm(t.lo[3], t.lo[2], sa), perm(t.lo[1], t.lo[0], sa), ka);
  const uint32_t hia = perm(perm(t.hi[3], t.hi[2], sa), perm(t.hi[1], t.hi[0], sa), ka);
  const uint32_t lob = perm(perm(t.lo[3], t.lo[2], sb), perm(t.lo[1], t.lo[0], sb), kb);
  const uint32_t hib = perm(perm(t.hi[3], t.hi[2], sb), perm(t.hi[1], t.hi[0], sb), kb);
  u32x4_t o;
  o[0] = perm(hia, loa, 0x05010400u);
  o[1] = perm(hia, loa, 0x07030602u);
  o[2] = perm(hib, lob, 0x05010400u);
  o[3] = perm(hib, lob, 0x07030602u);
  return o;
}

// Lookup table for block-32 NF4: the two lanes of each half of a DPP quad
// share a scale s (lanes 0, 1 the unit's first 32 weights, lanes 2, 3 the
// rest); lane q computes entries 8 (q & 1) .. +7 (lv8[i] = level[8 (q & 1) +
// i]) and the pair exchanges its planes with quad_perm [0,0,2,2] / [1,1,3,3].
template <bool F16 = false>
QL_DEV Lut make_lut_pair(const float* lv8, float s) {
  uint32_t d[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) d[i] = pack16x2<F16>(lv8[2 * i] * s, lv8[2 * i + 1] * s);
  const uint32_t lo0 = perm(d[1], d[0], 0x06040200u), hi0 = perm(d[1], d[0], 0x07050301u);
  const uint32_t lo1 = perm(d[3], d[2], 0x06040200u), hi1 = perm(d[3], d[2], 0x07050301u);
  Lut t;
  t.lo[0] = __builtin_amdgcn_mov_dpp(lo0, 0xA0, 0xF, 0xF, false);
  t.lo[1] = __builtin_amdgcn_mov_dpp(lo1, 0xA0, 0xF, 0xF, false);
  t.lo[2] = __builtin_amdgcn_mov_dpp(lo0, 0xF5, 0xF, 0xF, false);
  t.lo[3] = __builtin_amdgcn_mov_dpp(lo1, 0xF5, 0xF, 0xF, false);
  t.hi[0] = __builtin_amdgcn_mov_dpp(hi0, 0xA0, 0xF, 0xF, false);
  t.hi[1] = __builtin_amdgcn_mov_dpp(hi1, 0xA0, 0xF, 0xF, false);
  t.hi[2] = __builtin_amdgcn_mov_dpp(hi0, 0xF5, 0xF, 0xF, false);
  t.hi[3] = __builtin_amdgcn_mov_dpp(hi1, 0xF5, 0xF, 0xF, false);
  return t;
}

// Q8_0: four int8 values (one packed word, element order) times the block
// scale d, as two packed bf16 pairs.  Each byte is biased to unsigned
// (q + 128, converted exactly by v_cvt_f32_ubyte) and fma(q + 128, d, -128 d)
// forms q * d exactly (11 + 8 significant bits fit binary32), then one
// rounding to bf16.
QL_DEV u32x2_t decode_q8x4(uint32_t x, float d) {
  const uint32_t u = x ^ 0x80808080u;
  const float nb = -128.0f * d;
  const float f0 = __builtin_fmaf((float)(u & 0xFFu), d, nb);
  const float f1 = __builtin_fmaf((float)((u >> 8) & 0xFFu), d, nb);
  const float f2 = __builtin_fmaf((float)((u >> 16) & 0xFFu), d, nb);
  const float f3 = __builtin_fmaf((float)(u >> 24), d, nb);
  return u32x2_t{pack_bf16x2(f0, f1), pack_bf16x2(f2, f3)};
}

// 8 consecutive Q8_0 elements (two packed words) -> 4 packed bf16 pairs, in
// the element order decode8 produces.
QL_DEV u32x4_t decode_q8x8(uint32_t w0, uint32_t w1, float d) {
  const u32x2_t a = decode_q8x4(w0, d), b = decode_q8x4(w1, d);
  return u32x4_t{a[0], a[1], b[0], b[1]};
}

// ds_read_b64_tr_b16 of an LDS address: in each 16-lane group, lane i gets
// 4 consecutive 16-bit values of column i of the 4 x 16 block whose rows the
// group's lanes address (lane j: row j / 4, columns 4 (j % 4) .. + 3).
QL_DEV u32x2_t ds_tr16(const uint16_t* p) {
  const s16x4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((QL_LDS s16x4_t*)(p));
  return __builtin_bit_cast(u32x2_t, v);
}

// Eight 16-bit elements row[c .. c+7] as 4 packed pairs: one 16-byte load
// (vec: in range and 16-byte aligned), else element loads with zeros past C.
QL_DEV u32x4_t load_act8(const uint16_t* row, int64_t c, int64_t C, bool vec) {
  if (vec) return *reinterpret_cast<const u32x4_t*>(row + c);
  uint32_t h[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) h[e] = (c + e < C) ? row[c + e] : 0u;
  return u32x4_t{h[0] | h[1] << 16, h[2] | h[3] << 16, h[4] | h[5] << 16, h[6] | h[7] << 16};
}

// fp16 bits -> fp32 (exact)
QL_DEV float half_bits_to_float(uint32_t h) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)h);
}

// Storage position of the 64-block (n, kb) of an N-row weight with nkb blocks
// per row: rows are taken in groups of 16 and inside a group the blocks are
// ordered by k-block, then by row, so the blocks that 16 consecutive rows
// hold at one k-block are contiguous (512 code bytes, 16 scale bytes).  Both
// the codes (32 bytes per block) and the 8-bit scales use this order; the
// fp32 second-level constants are indexed by the flat block n * nkb + kb.
QL_DEV int64_t blk_pos(int64_t n, int64_t kb, int64_t N, int64_t nkb) {
  const int64_t g0 = n & ~int64_t(15);
  const int64_t R = min(int64_t(16), N - g0);
  return g0 * nkb + kb * R + (n - g0);
}

// Block scale s' = fp32(qscale * step): one rounding, as the format defines.
// b is the flat block index, p its storage position.
QL_DEV float block_scale(const uint8_t* qscale, const float* step, int64_t b, int64_t p) {
  return (float)qscale[p] * step[b / kGroup];
}

// s_waitcnt with only vmcnt constrained (gfx9 encoding: vmcnt in bits 3:0 and
// 15:14, expcnt 6:4, lgkmcnt 11:8).
#define QL_VMCNT(n) __builtin_amdgcn_s_waitcnt(((n) & 0xF) | ((((n) >> 4) & 3) << 14) | 0x0F70)
#define QL_LGKMCNT0() __builtin_amdgcn_s_waitcnt(0xC07F)

QL_DEV float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}

QL_DEV float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

}  // namespace ql
