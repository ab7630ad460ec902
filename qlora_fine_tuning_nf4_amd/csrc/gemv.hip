// Forward base product of the quantized linear, Y = X deq(W)^T (+ LoRA term),
// with the 4-bit weight dequantized to bf16 inside the kernels and never
// written to global memory (www.cf-1.com/news/5705389 §2.2 and §4.2: block
// dequantization inside the GEMM, results kept in registers / shared memory;
// www.lqnn.cn/news/228537 §3.3 and zky001 section 5.8: dequantize to 16 bits
// for the product, then discard).
//
// Small-M forward (the large-M GEMMs are in gemm.hip) and the split-K reduce.
//  * k_gemv_fwd  -- small M (<= 64): a wave owns 16 weight rows and streams
//    their packed bytes; each lane decodes a whole 64-block (one lookup table
//    per block) and feeds eight MFMAs whose 32-wide contraction spans four
//    different blocks; the activation fragments are read straight from L2.
#include "common.h"
#include "kernels.h"

namespace ql {

QL_DEV float lora_dot(const LoraTerm& L, int64_t m, int64_t c) {
  float acc = 0.f;
  const float* lr = L.L + m * L.r;
  const uint16_t* rr = L.R + c * L.rs_c;
  for (int j = 0; j < L.r; ++j) acc += lr[j] * __builtin_bit_cast(float, (uint32_t)rr[j * L.rs_j] << 16);
  return acc;
}

QL_DEV void store_out(void* out, bool bf16, int64_t idx, float v) {
  if (bf16)
    reinterpret_cast<uint16_t*>(out)[idx] = to_bf16(v);
  else
    reinterpret_cast<float*>(out)[idx] = v;
}

template <int MT>
__global__ __launch_bounds__(256) void k_gemv_fwd(const uint16_t* __restrict__ X, Nf4View w,
                                                  const float* __restrict__ codebook, int64_t M,
                                                  LoraTerm lora, void* __restrict__ Y, int y_bf16,
                                                  float* __restrict__ part, int ksplit,
                                                  int quads_per_split) {
  __shared__ float s_lv[16];
  __shared__ f32x4_t s_red[3][MT][64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t N = w.n, K = w.k, nkb = K / kBlock, nquads = (nkb + 3) / 4;
  const int64_t n = (int64_t)blockIdx.x * 16 + (lane & 15);
  const int g = lane >> 4;
  const int split = blockIdx.y;
  const int64_t q0 = (int64_t)split * quads_per_split;
  const int64_t q1 = min(nquads, q0 + quads_per_split);
  if (tid < 16) s_lv[tid] = codebook[tid];
  __syncthreads();
  float lv[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) lv[i] = s_lv[i];

  f32x4_t acc[MT];
#pragma unroll
  for (int t = 0; t < MT; ++t) acc[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  for (int64_t q = q0 + wave; q < q1; q += 4) {
    const int64_t kb = 4 * q + g;
    u32x4_t c0 = {0u, 0u, 0u, 0u}, c1 = {0u, 0u, 0u, 0u};
    float sc = 0.f;
    if (n < N && kb < nkb) {
      const int64_t b = n * nkb + kb;
      const u32x4_t* src = reinterpret_cast<const u32x4_t*>(w.codes + b * 32);
      c0 = src[0];
      c1 = src[1];
      sc = block_scale(w.qscale, w.step, b);
    }
    const Lut t = make_lut(lv, sc);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const u32x4_t bf = decode8(t, i < 4 ? c0[i] : c1[i - 4]);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const int64_t m = mt * 16 + (lane & 15);
        u32x4_t af = {0u, 0u, 0u, 0u};
        if (m < M && kb < nkb) af = *reinterpret_cast<const u32x4_t*>(X + m * K + kb * kBlock + i * 8);
        acc[mt] = mfma16x16x32(af, bf, acc[mt]);
      }
    }
  }
  if (wave > 0)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) s_red[wave - 1][mt][lane] = acc[mt];
  __syncthreads();
  if (wave != 0) return;
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    f32x4_t v = acc[mt];
    v += s_red[0][mt][lane];
    v += s_red[1][mt][lane];
    v += s_red[2][mt][lane];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int64_t m = mt * 16 + g * 4 + e;
      if (m < M && n < N) {
        float y = v[e];
        if (ksplit > 1) {
          part[((int64_t)split * M + m) * N + n] = y;
        } else {
          if (lora.r > 0) y += lora.scaling * lora_dot(lora, m, n);
          store_out(Y, y_bf16, m * N + n, y);
        }
      }
    }
  }
}

__global__ __launch_bounds__(256) void k_reduce(const float* __restrict__ part, int nsplit, int64_t M,
                                                int64_t C, LoraTerm lora, void* __restrict__ out,
                                                int out_bf16) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= M * C) return;
  float v = 0.f;
  for (int s = 0; s < nsplit; ++s) v += part[(int64_t)s * M * C + idx];
  if (lora.r > 0) v += lora.scaling * lora_dot(lora, idx / C, idx % C);
  store_out(out, out_bf16, idx, v);
}

hipError_t launch_gemv_fwd(const Nf4View& w, const float* codebook, const uint16_t* X, int64_t M,
                           const LoraTerm& lora, void* Y, bool y_bf16, float* part, int ksplit,
                           hipStream_t s) {
  const int64_t nquads = (w.k / kBlock + 3) / 4;
  const int per = (int)((nquads + ksplit - 1) / ksplit);
  dim3 grid((unsigned)((w.n + 15) / 16), (unsigned)ksplit);
  const int mt = (int)((M + 15) / 16);
#define QL_GEMV(MT)                                                                             \
  hipLaunchKernelGGL(k_gemv_fwd<MT>, grid, dim3(256), 0, s, X, w, codebook, M, lora, Y,        \
                     (int)y_bf16, part, ksplit, per)
  switch (mt) {
    case 1: QL_GEMV(1); break;
    case 2: QL_GEMV(2); break;
    case 3: QL_GEMV(3); break;
    default: QL_GEMV(4); break;
  }
#undef QL_GEMV
  return hipGetLastError();
}

hipError_t launch_reduce(const float* part, int nsplit, int64_t M, int64_t C, const LoraTerm& lora,
                         void* out, bool out_bf16, hipStream_t s) {
  const int64_t total = M * C;
  hipLaunchKernelGGL(k_reduce, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s, part, nsplit,
                     M, C, lora, out, (int)out_bf16);
  return hipGetLastError();
}

}  // namespace ql
