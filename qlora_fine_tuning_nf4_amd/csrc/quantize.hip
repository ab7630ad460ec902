// Block-wise NF4 quantization with double quantization of the block scales,
// the alternate block formats (asymmetric uint4, Q8_0), and the dense
// dequantization used for checking and adapter merging.
//
// Format (news.rkmt.cn/news/4821 §1.2, §1.3, §2.2, §2.3; zky001 section 5.8
// "NF4" and "double quantization"): 64-element blocks scaled by their absmax,
// 4-bit NF4 codes, block absmax quantized to 8 bits in groups of 256 blocks
// with one fp32 constant per group.
#include "common.h"
#include "kernels.h"

#include <algorithm>

namespace ql {

// Encode table: v in [-1, 1] goes to bin n = rint(32 v + 32) in [0, 64];
// bin n covers [(n - 32.5) / 32, (n - 31.5) / 32].  Widened by 2^-10 on both
// sides, a bin holds at most one decision midpoint (they are more than 0.07
// apart), so code = #{k : v > mid_k} = base_n + (v > m_n), with base_n the
// number of midpoints below the widened bin and m_n the midpoint inside it
// (+inf if none).  The widening covers the rounding of the bin index.  Few
// bins keep the lookups mostly broadcast reads (weights crowd the centre).
constexpr int kEncBins = 65;
constexpr float kEncMagic = 12582912.0f;           // 1.5 * 2^23: rounds to integers in the mantissa

QL_DEV void build_encode_table(const float* mid, float2* tab, int tid, int nthreads) {
  for (int i = tid; i < kEncBins; i += nthreads) {
    const float lo = ((float)i - 32.5f) * (1.0f / 32.0f) - (1.0f / 1024.0f);
    const float hi = ((float)i - 31.5f) * (1.0f / 32.0f) + (1.0f / 1024.0f);
    int base = 0;
    float m = __builtin_huge_valf();
    for (int k = 0; k < 15; ++k) {
      if (mid[k] < lo) ++base;
      else if (mid[k] <= hi) m = mid[k];
    }
    tab[i] = make_float2(m, __builtin_bit_cast(float, base));
  }
}

// 8 weights (one 16-byte piece of a block) -> one packed word, given the
// block absmax am.  The quotient v = fp32(w / am) is formed as
// q0 = fp32(w * r), e = w - q0 * am (exact, fma), v = fp32(q0 + e * r) with r
// ~ 1/am: for bf16 w and am (8-bit significands) the exact quotient p/q is a
// short dyadic or at least 2^-33 (relative) away from every binary32 rounding
// boundary (a boundary is an odd multiple of 2^-25 at that scale, so the gap
// is at least 1/(q 2^25)); for fp16 (11-bit significands) at least 2^-36;
// while q0 + e * r is within ~2^-46 of it, so v equals the correctly rounded
// binary32 division bit for bit.  The argument needs r and q0 to be normal
// numbers, so the block is first scaled by a power of two (which changes no
// quotient): absmax below 2^-100 by 2^100, so that 1/am stays finite, and
// absmax at or above 2^64 by 2^-64, so that 1/am is not a subnormal (which
// the reciprocal would lose or flush to zero for am >= 2^126).  Scaling down
// is exact for every element whose quotient is at least 2^-100 or so; smaller
// elements may round or flush, but any quotient below the first midpoints
// around zero (|v| < 0.03) encodes as the zero level either way.
QL_DEV uint32_t encode8(const float (&xin)[8], float am, const float2* tab) {
  const bool tiny = am < 0x1p-100f;
  const bool huge = am >= 0x1p64f;
  const float sc = tiny ? 0x1p100f : (huge ? 0x1p-64f : 1.0f);
  const float a = am * sc;
  const float r = am > 0.f ? __builtin_amdgcn_rcpf(a) : 0.f;
  uint32_t word = 0;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const float x = xin[j] * sc;
    const float q0 = x * r;
    const float e = __builtin_fmaf(-q0, a, x);
    const float v = __builtin_fmaf(e, r, q0);
    const int n = __builtin_bit_cast(int, __builtin_fmaf(v, 32.0f, kEncMagic + 32.0f)) -
                  __builtin_bit_cast(int, kEncMagic);
    const float2 t = tab[n];
    const uint32_t c = (uint32_t)__builtin_bit_cast(int, t.y) + (v > t.x ? 1u : 0u);
    word |= c << (j < 4 ? 8 * j : 8 * (j - 4) + 4);
  }
  return word;
}

// One workgroup per group of 256 blocks (BS weights each; 16384 weights, 32
// KiB of bf16 at BS = 64) at a time, walking groups with the grid as stride;
// the next group's loads are issued before the current one is encoded.  Lane
// l reads 16 bytes (8 weights) of block l / LB (LB = BS / 8 lanes per block),
// so one wave load is 1 KiB contiguous.  The block absmax is a max over the
// LB lanes of the block; encoding needs only the block's own absmax, so codes
// are written in the same pass and the group max is taken afterwards from
// LDS.  Codes keep the 64-weight unit layout whatever the block: the lane's
// word is word w of unit (row, u) with 64 u + 8 w its first element.  Scale
// entries: block 64 at the unit's storage position, block 32 at 2 p + half,
// block 128 at the row-group position over the k/128 block columns.  Without
// double quantization (DQ false) the block absmax itself is stored, fp32, in
// `step`, and `qscale` is unused.  F16: the weight is fp16 instead of bf16
// (both widen to fp32 exactly, after which the steps are the same).
template <bool DQ, int BS, bool F16 = false>
__global__ __launch_bounds__(256) void k_quant_nf4_dq(const uint16_t* __restrict__ W,
                                                      const float* __restrict__ codebook,
                                                      uint8_t* __restrict__ codes,
                                                      uint8_t* __restrict__ qscale,
                                                      float* __restrict__ step, int64_t N,
                                                      int64_t nkb) {
  constexpr int LB = BS / 8;                 // lanes per block
  constexpr int BPW = 64 / LB;               // blocks per wave load
  constexpr int BPI = 4 * BPW;               // blocks per workgroup step
  constexpr int NIT = kGroup / BPI;          // steps per group (= LB)
  __shared__ float s_absmax[kGroup];
  __shared__ float s_red[4];
  __shared__ float2 s_tab[kEncBins];
  // block counts fit 32 bits (the ABI keeps n * k / BS below 2^32), so block
  // coordinates use 32-bit division
  const uint32_t ukbB = (uint32_t)(nkb * 64 / BS);   // blocks per row
  const uint32_t nblocks = (uint32_t)(N * ukbB);
  const uint32_t ngroups = (nblocks + kGroup - 1) / kGroup;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lb0 = wave * BPW + lane / LB;
  const int lw = lane % LB;                  // the lane's 8-weight piece of its block

  {
    float mid[15];
#pragma unroll
    for (int i = 0; i < 15; ++i) mid[i] = codebook[16 + i];
    build_encode_table(mid, s_tab, tid, 256);
  }

  // the NIT 16-byte loads of this lane for group grp (a short last group
  // re-reads its last block; those lanes are not stored)
  auto load_group = [&](uint32_t grp, u32x4_t (&r)[NIT]) {
    const uint32_t blk0 = grp * kGroup;
    const int nb = (int)min(kGroup, nblocks - blk0);
#pragma unroll
    for (int it = 0; it < NIT; ++it) {
      const int lb = min(it * BPI + lb0, nb - 1);
      // the weight is read exactly once: non-temporal loads keep it from
      // displacing the code and scale lines that the L2 merges for writing
      r[it] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(W + ((int64_t)blk0 + lb) * BS + lw * 8));
    }
  };
  // storage entry of the scale of block (row, kb)
  auto scale_pos = [&](uint32_t row, uint32_t kb) -> int64_t {
    if (BS == 64) return blk_pos(row, kb, N, nkb);
    if (BS == 32) return 2 * blk_pos(row, kb >> 1, N, nkb) + (kb & 1);
    return blk_pos(row, kb, N, nkb / 2);
  };

  auto do_group = [&](uint32_t grp, const u32x4_t (&cur)[NIT]) {
    const uint32_t blk0 = grp * kGroup;
    const int nb = (int)min(kGroup, nblocks - blk0);
    // (row, block column) of this lane's block, advanced by BPI blocks per step
    uint32_t row = (blk0 + lb0) / ukbB;
    uint32_t kb = (blk0 + lb0) - row * ukbB;
#pragma unroll
    for (int it = 0; it < NIT; ++it) {
      const int lb = it * BPI + lb0;                    // local block index
      float x[8];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        x[2 * j] = lo16<F16>(cur[it][j]);
        x[2 * j + 1] = hi16<F16>(cur[it][j]);
      }
      float am = 0.f;
#pragma unroll
      for (int j = 0; j < 8; ++j) am = fmaxf(am, fabsf(x[j]));
#pragma unroll
      for (int o = 1; o < LB; o <<= 1) am = fmaxf(am, __shfl_xor(am, o));
      const uint32_t word = encode8(x, am, s_tab);
      if (lb < nb) {
        const uint32_t e0 = kb * BS + lw * 8;           // first element within the row
        const int64_t p = blk_pos(row, e0 >> 6, N, nkb);
        reinterpret_cast<uint32_t*>(codes)[p * 8 + ((e0 & 63) >> 3)] = word;
        if (lw == 0) {
          if (DQ)
            s_absmax[lb] = am;
          else
            step[scale_pos(row, kb)] = am;
        }
      }
      kb += BPI;
      while (kb >= ukbB) {
        kb -= ukbB;
        ++row;
      }
    }
    if (!DQ) return;
    __syncthreads();
    const float a = tid < nb ? s_absmax[tid] : 0.f;
    const float wm = wave_max(a);
    if (lane == 0) s_red[wave] = wm;
    __syncthreads();
    const float c2 = fmaxf(fmaxf(s_red[0], s_red[1]), fmaxf(s_red[2], s_red[3]));
    const float st = c2 / 255.0f;
    if (tid < nb) {
      const float q = st == 0.f ? 0.f : fminf(rintf(a / st), 255.f);
      const uint32_t b = blk0 + tid, br = b / ukbB;
      qscale[scale_pos(br, b - br * ukbB)] = (uint8_t)q;
    }
    if (tid == 0) step[grp] = st;
    __syncthreads();   // s_absmax and s_red are reused by the next group
  };

  // Workgroup ids are dealt to the 8 XCDs round robin; renumber them so that
  // consecutive groups run on one XCD: the rows of a 16-row storage group are
  // then written through one L2, which merges the 32-byte block writes of
  // neighbouring rows into whole lines.  (The grid is a multiple of 8.)
  const uint32_t per_xcd = gridDim.x / 8;
  const uint32_t lwg = (blockIdx.x & 7) * per_xcd + (blockIdx.x >> 3);
  // ping-pong between two register sets (no copies of in-flight loads)
  u32x4_t ra[NIT], rb[NIT];
  uint32_t grp = lwg;
  if (grp < ngroups) load_group(grp, ra);
  __syncthreads();   // encode table ready
  while (grp < ngroups) {
    if (grp + gridDim.x < ngroups) load_group(grp + gridDim.x, rb);
    do_group(grp, ra);
    grp += gridDim.x;
    if (grp >= ngroups) break;
    if (grp + gridDim.x < ngroups) load_group(grp + gridDim.x, ra);
    do_group(grp, rb);
    grp += gridDim.x;
  }
}

// Asymmetric uint4 (news.rkmt.cn/news/4821 §1.3, §2.1; kwkr.cn/news/627310
// §2.1): per 64-block, the range widened to hold 0, scale = (hi - lo) / 15,
// zero-point = rint(-lo / scale) in [0, 15] (an fp32 integer value, never
// -0), q = clamp(rint(x / scale) + zp, 0, 15); an all-zero block gets scale
// 0, zp 0 and codes 0.  The zero-point is taken from the range with the real
// scale, -lo * 15 / (hi - lo) in binary64 (the reading under which kwkr §2.1's
// INT8 example gives its printed zero-point 128); the other divisions are the
// correctly rounded binary32 ones.
// Eight lanes per 64-weight unit (16-byte loads, eight weights each), one
// unit per lane group; codes packed as the NF4 codes, (scale, zp) at the
// unit's storage position.
__global__ __launch_bounds__(256) void k_quant_u4(const uint16_t* __restrict__ W,
                                                  uint8_t* __restrict__ codes,
                                                  float* __restrict__ params, int64_t N,
                                                  int64_t nkb) {
  const uint32_t nunits = (uint32_t)(N * nkb), ukb = (uint32_t)nkb;
  const int lane8 = threadIdx.x & 7;
  const uint32_t u = blockIdx.x * 32u + (threadIdx.x >> 3);
  if (u >= nunits) return;   // whole lane groups leave together
  const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(W + (int64_t)u * kBlock + lane8 * 8));
  float x[8];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    x[2 * j] = bf16_lo(v[j]);
    x[2 * j + 1] = bf16_hi(v[j]);
  }
  float lo = 0.f, hi = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    lo = fminf(lo, x[j]);
    hi = fmaxf(hi, x[j]);
  }
#pragma unroll
  for (int o = 1; o < 8; o <<= 1) {
    lo = fminf(lo, __shfl_xor(lo, o));
    hi = fmaxf(hi, __shfl_xor(hi, o));
  }
  const float sc = (hi - lo) / 15.0f;
  const bool live = sc > 0.f;
  // binary64: 15 * lo is exact, the subtraction and the division round once
  const double zd = rint((-(double)lo * 15.0) / ((double)hi - (double)lo));
  const int zp = live ? (int)fmin(fmax(zd, 0.0), 15.0) : 0;
  uint32_t word = 0;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int q = live ? min(max((int)rintf(x[j] / sc) + zp, 0), 15) : 0;
    word |= (uint32_t)q << (j < 4 ? 8 * j : 8 * (j - 4) + 4);
  }
  const uint32_t row = u / ukb;
  const int64_t p = blk_pos(row, u - row * ukb, N, nkb);
  reinterpret_cast<uint32_t*>(codes)[p * 8 + lane8] = word;
  if (lane8 == 0) reinterpret_cast<float2*>(params)[p] = make_float2(live ? sc : 0.f, (float)zp);
}

// Q8_0 (www.cf-1.com/news/5705389 §1.1, §2.2; kwkr.cn/news/627310 §2.1): per
// 32-block, d16 = fp16_rne(fp32(absmax / 127)), q = clamp(rint(x / d16), -127,
// 127), 0 when d16 is 0.  Eight lanes per 64-weight unit, four per block;
// 64 int8 codes and the two fp16 scales at the unit's storage position.
__global__ __launch_bounds__(256) void k_quant_q8(const uint16_t* __restrict__ W,
                                                  uint8_t* __restrict__ codes,
                                                  uint8_t* __restrict__ scales, int64_t N,
                                                  int64_t nkb) {
  const uint32_t nunits = (uint32_t)(N * nkb), ukb = (uint32_t)nkb;
  const int lane8 = threadIdx.x & 7;
  const uint32_t u = blockIdx.x * 32u + (threadIdx.x >> 3);
  if (u >= nunits) return;
  const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(W + (int64_t)u * kBlock + lane8 * 8));
  float x[8];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    x[2 * j] = bf16_lo(v[j]);
    x[2 * j + 1] = bf16_hi(v[j]);
  }
  float am = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j) am = fmaxf(am, fabsf(x[j]));
  am = fmaxf(am, __shfl_xor(am, 1));
  am = fmaxf(am, __shfl_xor(am, 2));
  const _Float16 h = (_Float16)(am / 127.0f);
  const float d = (float)h;
  uint32_t b[2] = {0u, 0u};
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int q = d != 0.f ? min(max((int)rintf(x[j] / d), -127), 127) : 0;
    b[j >> 2] |= ((uint32_t)q & 0xFFu) << (8 * (j & 3));
  }
  const uint32_t row = u / ukb;
  const int64_t p = blk_pos(row, u - row * ukb, N, nkb);
  *reinterpret_cast<u32x2_t*>(codes + p * 64 + lane8 * 8) = u32x2_t{b[0], b[1]};
  if ((lane8 & 3) == 0)
    reinterpret_cast<uint16_t*>(scales)[p * 2 + (lane8 >> 2)] = __builtin_bit_cast(uint16_t, h);
}

// Dense dequantization: one thread per 64-weight unit, 8 x 16-byte stores.
// The 4-bit formats go through a per-block table (NF4: level[c] times the
// block scale; uint4: (c - zp) times the scale), Q8_0 bytes are scaled
// directly.
template <int FMT>
__global__ __launch_bounds__(256) void k_dequant(Nf4View w, const float* __restrict__ codebook,
                                                 uint16_t* __restrict__ out) {
  const int64_t N = w.n, nkb = w.k / kBlock, nblocks = N * nkb;
  __shared__ float s_lv[16];
  if (FmtInfo<FMT>::nf4 && threadIdx.x < 16) s_lv[threadIdx.x] = codebook[threadIdx.x];
  __syncthreads();
  const int64_t b = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= nblocks) return;
  const int64_t p = blk_pos(b / nkb, b % nkb, N, nkb);
  u32x4_t* dst = reinterpret_cast<u32x4_t*>(out + b * kBlock);
  if constexpr (FMT == kFmtQ8) {
    const uint16_t* sc = reinterpret_cast<const uint16_t*>(w.qscale) + p * 2;
    const float d0 = half_bits_to_float(sc[0]), d1 = half_bits_to_float(sc[1]);
    const u32x4_t* src = reinterpret_cast<const u32x4_t*>(w.codes + p * 64);
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      const u32x4_t c = src[h];
      dst[2 * h] = decode_q8x8(c[0], c[1], h < 2 ? d0 : d1);
      dst[2 * h + 1] = decode_q8x8(c[2], c[3], h < 2 ? d0 : d1);
    }
  } else {
    float lv[16];
    float s = 0.f;
    if constexpr (FMT == kFmtU4) {
      const float2 sz = reinterpret_cast<const float2*>(w.step)[p];
      const int zp = (int)sz.y;   // c - zp is formed exactly as an integer (c == zp gives +0)
#pragma unroll
      for (int i = 0; i < 16; ++i) lv[i] = (float)(i - zp);
      s = sz.x;
    } else {
#pragma unroll
      for (int i = 0; i < 16; ++i) lv[i] = s_lv[i];
    }
    // the scale of each half of the unit (the same unless the block is 32)
    float sh[2];
    if constexpr (FMT == kFmtU4) {
      sh[0] = sh[1] = s;
    } else {
      constexpr int BS = FmtInfo<FMT>::block;
      const int64_t row = b / nkb, kb = b - row * nkb;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        int64_t e, fb;   // scale entry, flat block
        if (BS == 64) {
          e = p;
          fb = b;
        } else if (BS == 32) {
          e = 2 * p + h;
          fb = 2 * b + h;
        } else {
          e = blk_pos(row, kb >> 1, N, nkb / 2);
          fb = row * (nkb / 2) + (kb >> 1);
        }
        sh[h] = FmtInfo<FMT>::dq ? (float)w.qscale[e] * w.step[fb / kGroup] : w.step[e];
      }
    }
    const u32x4_t* src = reinterpret_cast<const u32x4_t*>(w.codes + p * 32);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const Lut t = make_lut<FmtInfo<FMT>::f16>(lv, sh[h]);
      const u32x4_t c = src[h];
#pragma unroll
      for (int j = 0; j < 4; ++j) dst[h * 4 + j] = decode8(t, c[j]);
    }
  }
}

// Adapter merge (www.lqnn.cn/news/228537 §3.3: dequantize, add the low-rank
// branch at high precision, quantize again), in place on the dequantized
// weight W [N x K] (bf16, or fp16 when F16, as are A and B):
//   merged[n][k] = rne16(fp32(w + fp32(s * acc))),
//   acc = sum_j B[n][j] A[j][k]  in binary32, in rank order (16-bit products are exact).
// A thread owns 8 consecutive k of one row: A[j][k .. k+7] as one 16-byte load
// per rank, B[n][j] as a scalar shared by the row's threads.  Contraction of
// the multiply-add into an fma is switched off: the steps round as written.
template <bool F16>
__global__ __launch_bounds__(256) void k_merge(uint16_t* __restrict__ W, const uint16_t* __restrict__ A,
                                               const uint16_t* __restrict__ B, int64_t N, int64_t K,
                                               int r, float s) {
#pragma clang fp contract(off)
  const int64_t pieces = N * (K / 8);
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= pieces) return;
  const int64_t n = idx / (K / 8), k = (idx - n * (K / 8)) * 8;
  float acc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = 0.f;
  for (int j = 0; j < r; ++j) {
    const float b = w16<F16>(B[n * r + j]);
    const u32x4_t a = *reinterpret_cast<const u32x4_t*>(A + (int64_t)j * K + k);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      acc[2 * e] = acc[2 * e] + b * lo16<F16>(a[e]);
      acc[2 * e + 1] = acc[2 * e + 1] + b * hi16<F16>(a[e]);
    }
  }
  u32x4_t* wp = reinterpret_cast<u32x4_t*>(W + n * K + k);
  const u32x4_t w = *wp;
  u32x4_t o;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const float t0 = s * acc[2 * e], t1 = s * acc[2 * e + 1];
    o[e] = pack16x2<F16>(lo16<F16>(w[e]) + t0, hi16<F16>(w[e]) + t1);
  }
  *wp = o;
}

hipError_t launch_merge(uint16_t* W, const uint16_t* A, const uint16_t* B, int64_t n, int64_t k, int r,
                        float s, bool f16, hipStream_t st) {
  const int64_t pieces = n * (k / 8);
  const dim3 grid((unsigned)((pieces + 255) / 256));
  if (f16)
    hipLaunchKernelGGL(k_merge<true>, grid, dim3(256), 0, st, W, A, B, n, k, r, s);
  else
    hipLaunchKernelGGL(k_merge<false>, grid, dim3(256), 0, st, W, A, B, n, k, r, s);
  return hipGetLastError();
}

hipError_t launch_quantize(const uint16_t* W, const float* codebook, uint8_t* codes,
                           uint8_t* qscale, float* step, int64_t n, int64_t k, int fmt,
                           hipStream_t s) {
  const int64_t nkb = k / kBlock, nunits = n * nkb;
  const dim3 ugrid((unsigned)((nunits + 31) / 32));                         // 32 units per workgroup
  // NF4: persistent workgroups (each walks groups of 256 blocks of the
  // format's block size with a stride of the grid), a few per CU so loads of
  // the next group overlap the current one; a multiple of 8
  const int bs = fmt == kFmtNf4Dq32 || fmt == kFmtNf4_32 ? 32 : (fmt == kFmtNf4Dq128 || fmt == kFmtNf4_128 ? 128 : 64);
  const int64_t ngB = (n * k / bs + kGroup - 1) / kGroup;
  const dim3 ggrid((unsigned)std::min<int64_t>((ngB + 7) / 8 * 8, 256 * 8));
#define QL_QNF4(DQ, BS, ...) \
  hipLaunchKernelGGL((k_quant_nf4_dq<DQ, BS, ##__VA_ARGS__>), ggrid, dim3(256), 0, s, W, codebook, codes, qscale, step, n, nkb)
  switch (fmt) {
    case kFmtNf4Dq: QL_QNF4(true, 64); break;
    case kFmtNf4DqF16: QL_QNF4(true, 64, true); break;
    case kFmtNf4: QL_QNF4(false, 64); break;
    case kFmtNf4Dq32: QL_QNF4(true, 32); break;
    case kFmtNf4_32: QL_QNF4(false, 32); break;
    case kFmtNf4Dq128: QL_QNF4(true, 128); break;
    case kFmtNf4_128: QL_QNF4(false, 128); break;
    case kFmtU4:
      hipLaunchKernelGGL(k_quant_u4, ugrid, dim3(256), 0, s, W, codes, step, n, nkb);
      break;
    default:
      hipLaunchKernelGGL(k_quant_q8, ugrid, dim3(256), 0, s, W, codes, qscale, n, nkb);
      break;
  }
#undef QL_QNF4
  return hipGetLastError();
}

hipError_t launch_dequant(const Nf4View& w, const float* codebook, uint16_t* out, hipStream_t s) {
  const int64_t nblocks = w.n * (w.k / kBlock);
  const dim3 grid((unsigned)((nblocks + 255) / 256));
#define QL_DQ(F) hipLaunchKernelGGL(k_dequant<F>, grid, dim3(256), 0, s, w, codebook, out)
  switch (w.fmt) {
    case kFmtNf4Dq: QL_DQ(kFmtNf4Dq); break;
    case kFmtNf4: QL_DQ(kFmtNf4); break;
    case kFmtU4: QL_DQ(kFmtU4); break;
    case kFmtQ8: QL_DQ(kFmtQ8); break;
    case kFmtNf4Dq32: QL_DQ(kFmtNf4Dq32); break;
    case kFmtNf4_32: QL_DQ(kFmtNf4_32); break;
    case kFmtNf4Dq128: QL_DQ(kFmtNf4Dq128); break;
    case kFmtNf4DqF16: QL_DQ(kFmtNf4DqF16); break;
    default: QL_DQ(kFmtNf4_128); break;
  }
#undef QL_DQ
  return hipGetLastError();
}

}  // namespace ql
