// Block-wise NF4 quantization with double quantization of the block scales,
// and the dense dequantization used for checking and adapter merging.
//
// Format (news.rkmt.cn/news/4821 §1.2, §1.3, §2.2, §2.3; zky001 section 5.8
// "NF4" and "double quantization"): 64-element blocks scaled by their absmax,
// 4-bit NF4 codes, block absmax quantized to 8 bits in groups of 256 blocks
// with one fp32 constant per group.
#include "common.h"
#include "kernels.h"

namespace ql {

// Encode table: v in [-1, 1] falls in bin floor(256 v + 256) (clamped to
// 511); bin i covers [-1 + i/256, -1 + (i+1)/256).  Widened by 2^-10 on both
// sides, each bin holds at most one decision midpoint (they are more than
// 0.05 apart), so code = #{k : v > mid_k} = base_i + (v > m_i), with base_i
// the number of midpoints below the widened bin and m_i the midpoint inside
// it (+inf if none).  The widening covers the rounding of the bin index.
constexpr int kEncBins = 512;

QL_DEV void build_encode_table(const float* mid, float2* tab, int tid, int nthreads) {
  for (int i = tid; i < kEncBins; i += nthreads) {
    const float lo = -1.0f + (float)i * (1.0f / 256.0f) - (1.0f / 1024.0f);
    const float hi = -1.0f + (float)(i + 1) * (1.0f / 256.0f) + (1.0f / 1024.0f);
    int base = 0;
    float m = __builtin_huge_valf();
    for (int k = 0; k < 15; ++k) {
      if (mid[k] < lo) ++base;
      else if (mid[k] <= hi) m = mid[k];
    }
    tab[i] = make_float2(m, __builtin_bit_cast(float, base));
  }
}

// One workgroup per group of 256 blocks (16384 weights, 32 KiB of bf16).
// Each wave handles 8 blocks per iteration: lane l reads 16 bytes (8 weights)
// of block l/8, so one wave load is 1 KiB contiguous.  The block absmax is a
// max over the 8 lanes of the block; encoding needs only the block's own
// absmax, so codes are written in the same pass and the group max is taken
// afterwards from LDS.
//
// Quotient: v = fp32(w / absmax) is formed as fp32(w * r) in binary64 with r
// = 1/absmax refined to binary64 accuracy.  For bf16 w and absmax (8-bit
// significands) the exact quotient is either a short dyadic (no fp32 rounding
// tie possible) or at least 2^-33 (relative) away from every fp32 rounding
// boundary, far more than the binary64 error, so this equals the correctly
// rounded binary32 division bit for bit.
__global__ __launch_bounds__(256) void k_quant_nf4_dq(const uint16_t* __restrict__ W,
                                                      const float* __restrict__ codebook,
                                                      uint8_t* __restrict__ codes,
                                                      uint8_t* __restrict__ qscale,
                                                      float* __restrict__ step, int64_t N,
                                                      int64_t nkb) {
  __shared__ float s_absmax[kGroup];
  __shared__ float s_red[4];
  __shared__ float2 s_tab[kEncBins];
  const int64_t nblocks = N * nkb;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t blk0 = (int64_t)blockIdx.x * kGroup;
  const int nb = (int)min<int64_t>(kGroup, nblocks - blk0);

  {
    float mid[15];
#pragma unroll
    for (int i = 0; i < 15; ++i) mid[i] = codebook[16 + i];
    build_encode_table(mid, s_tab, tid, 256);
  }
  __syncthreads();

  // (row, k-block) of this lane's block, advanced by 32 blocks per iteration
  // without a division
  const int lb0 = wave * 8 + (lane >> 3);
  int64_t row = (blk0 + lb0) / nkb;
  int64_t kb = (blk0 + lb0) - row * nkb;
#pragma unroll 2
  for (int it = 0; it < kGroup / 32; ++it) {
    const int lb = it * 32 + lb0;                      // local block index
    const bool valid = lb < nb;
    u32x4_t raw = {0u, 0u, 0u, 0u};
    if (valid)
      raw = *reinterpret_cast<const u32x4_t*>(W + (blk0 + lb) * kBlock + (lane & 7) * 8);
    float x[8];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      x[2 * j] = bf16_lo(raw[j]);
      x[2 * j + 1] = bf16_hi(raw[j]);
    }
    float am = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) am = fmaxf(am, fabsf(x[j]));
    am = fmaxf(am, __shfl_xor(am, 1));
    am = fmaxf(am, __shfl_xor(am, 2));
    am = fmaxf(am, __shfl_xor(am, 4));
    // 1/absmax in binary64: hardware reciprocal plus one Newton step (0 for
    // an all-zero block, which then encodes as the zero level)
    double r = 0.0;
    if (am > 0.f) {
      const double a = (double)am;
      r = __builtin_amdgcn_rcp(a);
      r = __builtin_fma(r, __builtin_fma(-a, r, 1.0), r);
    }
    uint32_t word = 0;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float v = (float)((double)x[j] * r);
      const int bin = min((int)__builtin_fmaf(v, 256.0f, 256.0f), kEncBins - 1);
      const float2 e = s_tab[bin];
      const uint32_t c = (uint32_t)__builtin_bit_cast(int, e.y) + (v > e.x ? 1u : 0u);
      word |= c << (j < 4 ? 8 * j : 8 * (j - 4) + 4);
    }
    if (valid) {
      const int64_t p = blk_pos(row, kb, N, nkb);
      reinterpret_cast<uint32_t*>(codes)[p * 8 + (lane & 7)] = word;
      if ((lane & 7) == 0) s_absmax[lb] = am;
    }
    kb += 32;
    while (kb >= nkb) {
      kb -= nkb;
      ++row;
    }
  }
  __syncthreads();
  const float a = tid < nb ? s_absmax[tid] : 0.f;
  const float wm = wave_max(a);
  if (lane == 0) s_red[wave] = wm;
  __syncthreads();
  const float c2 = fmaxf(fmaxf(s_red[0], s_red[1]), fmaxf(s_red[2], s_red[3]));
  const float st = c2 / 255.0f;
  if (tid < nb) {
    const float q = st == 0.f ? 0.f : fminf(rintf(a / st), 255.f);
    const int64_t b = blk0 + tid;
    qscale[blk_pos(b / nkb, b % nkb, N, nkb)] = (uint8_t)q;
  }
  if (tid == 0) step[blockIdx.x] = st;
}

// Dense dequantization: one thread per 64-block, 8 x 16-byte stores.
__global__ __launch_bounds__(256) void k_dequant(const uint8_t* __restrict__ codes,
                                                 const uint8_t* __restrict__ qscale,
                                                 const float* __restrict__ step,
                                                 const float* __restrict__ codebook,
                                                 uint16_t* __restrict__ out, int64_t N,
                                                 int64_t nkb) {
  const int64_t nblocks = N * nkb;
  __shared__ float s_lv[16];
  if (threadIdx.x < 16) s_lv[threadIdx.x] = codebook[threadIdx.x];
  __syncthreads();
  float lv[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) lv[i] = s_lv[i];
  const int64_t b = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= nblocks) return;
  const int64_t p = blk_pos(b / nkb, b % nkb, N, nkb);
  const Lut t = make_lut(lv, block_scale(qscale, step, b, p));
  const u32x4_t* src = reinterpret_cast<const u32x4_t*>(codes + p * 32);
  u32x4_t* dst = reinterpret_cast<u32x4_t*>(out + b * kBlock);
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const u32x4_t w = src[h];
#pragma unroll
    for (int j = 0; j < 4; ++j) dst[h * 4 + j] = decode8(t, w[j]);
  }
}

hipError_t launch_quantize(const uint16_t* W, const float* codebook, uint8_t* codes,
                           uint8_t* qscale, float* step, int64_t n, int64_t k, hipStream_t s) {
  const int64_t nkb = k / kBlock, ngroups = (n * nkb + kGroup - 1) / kGroup;
  hipLaunchKernelGGL(k_quant_nf4_dq, dim3((unsigned)ngroups), dim3(256), 0, s, W, codebook, codes,
                     qscale, step, n, nkb);
  return hipGetLastError();
}

hipError_t launch_dequant(const uint8_t* codes, const uint8_t* qscale, const float* step,
                          const float* codebook, uint16_t* out, int64_t n, int64_t k, hipStream_t s) {
  const int64_t nkb = k / kBlock, nblocks = n * nkb;
  hipLaunchKernelGGL(k_dequant, dim3((unsigned)((nblocks + 255) / 256)), dim3(256), 0, s, codes,
                     qscale, step, codebook, out, n, nkb);
  return hipGetLastError();
}

}  // namespace ql
