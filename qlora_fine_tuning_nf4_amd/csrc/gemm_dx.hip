// Input gradient through the frozen quantized weight, dX = dY deq(W) (+ LoRA
// term) (www.cf-1.com/news/5705389 §2.1: the gradient with respect to x is
// dL/dy times W0^T, itself a quantized matrix product).
//
// W is [N x K] with its 64-blocks along K, but here the contraction runs over
// N, so each MFMA B operand needs 8 consecutive rows of one column.  The tile
// is decoded into LDS in its natural [n][k] layout (16-byte stores, same
// decoder as the forward) and read back column-wise with gfx950's transposing
// LDS load ds_read_b64_tr_b16: within a 16-lane group, lane 4q+p addresses row
// q, columns 4p..4p+3, and lane i receives column i of rows 0..3.
#include "common.h"
#include "kernels.h"

namespace ql {

constexpr int DBM = 128, DBK = 128, DBN = 128, DLD = DBN + 8;

QL_DEV float lora_dot_dx(const LoraTerm& L, int64_t m, int64_t c) {
  float acc = 0.f;
  const float* lr = L.L + m * L.r;
  const uint16_t* rr = L.R + c * L.rs_c;
  for (int j = 0; j < L.r; ++j) acc += lr[j] * __builtin_bit_cast(float, (uint32_t)rr[j * L.rs_j] << 16);
  return acc;
}

QL_DEV u32x2_t tr16(const uint16_t* p) {
  const s16x4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) s16x4_t*)(p));
  return __builtin_bit_cast(u32x2_t, v);
}

// dY rows may be unaligned (n % 8 != 0): element loads then.
QL_DEV u32x4_t load_row8(const uint16_t* row, int64_t c, int64_t C, bool vec) {
  if (vec && c + 8 <= C) return *reinterpret_cast<const u32x4_t*>(row + c);
  uint32_t h[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) h[e] = (c + e < C) ? row[c + e] : 0u;
  return u32x4_t{h[0] | h[1] << 16, h[2] | h[3] << 16, h[4] | h[5] << 16, h[6] | h[7] << 16};
}

__global__ __launch_bounds__(256) void k_gemm_dx(const uint16_t* __restrict__ dY, Nf4View w,
                                                 const float* __restrict__ codebook, int64_t M,
                                                 LoraTerm lora, void* __restrict__ dX, int dx_bf16,
                                                 float* __restrict__ part, int nsplit,
                                                 int steps_per_split) {
  __shared__ __attribute__((aligned(16))) uint16_t sA[DBM * DLD];   // dY tile [m][n]
  __shared__ __attribute__((aligned(16))) uint16_t sW[DBN * DLD];   // W tile  [n][k]
  __shared__ float s_lv[16];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t N = w.n, K = w.k, nkb = K / kBlock;
  const int64_t k0 = (int64_t)blockIdx.x * DBK, m0 = (int64_t)blockIdx.y * DBM;
  const int split = blockIdx.z;
  const int nsteps = (int)((N + DBN - 1) / DBN);
  const int s_begin = split * steps_per_split;
  const int s_end = min(nsteps, s_begin + steps_per_split);
  const bool vec = (N % 8) == 0;
  if (tid < 16) s_lv[tid] = codebook[tid];
  __syncthreads();
  float lv[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) lv[i] = s_lv[i];

  u32x4_t ar[8];
  u32x4_t wc0, wc1;
  float wsc;
  const int wrow = tid >> 1, whalf = tid & 1;
  auto load = [&](int st) {
    const int64_t nb = (int64_t)st * DBN;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int c = tid + 256 * i, row = c >> 4, col = (c & 15) * 8;
      const int64_t m = m0 + row;
      ar[i] = (m < M) ? load_row8(dY + m * N, nb + col, N, vec) : u32x4_t{0u, 0u, 0u, 0u};
    }
    const int64_t n = nb + wrow, kb = k0 / kBlock + whalf;
    if (n < N && kb < nkb) {
      const int64_t b = n * nkb + kb;
      const u32x4_t* src = reinterpret_cast<const u32x4_t*>(w.codes + b * 32);
      wc0 = src[0];
      wc1 = src[1];
      wsc = block_scale(w.qscale, w.step, b);
    } else {
      wc0 = u32x4_t{0u, 0u, 0u, 0u};
      wc1 = wc0;
      wsc = 0.f;
    }
  };

  f32x4_t acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  const int wm = wave & 1, wk = wave >> 1;
  const int fr = lane & 15, fg = lane >> 4;
  const int tq = (lane & 15) >> 2, tp = lane & 3;   // transposed-read addressing
  if (s_begin < s_end) load(s_begin);
  for (int st = s_begin; st < s_end; ++st) {
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int c = tid + 256 * i, row = c >> 4, col = (c & 15) * 8;
      *reinterpret_cast<u32x4_t*>(sA + row * DLD + col) = ar[i];
    }
    {
      const Lut t = make_lut(lv, wsc);
      u32x4_t* dst = reinterpret_cast<u32x4_t*>(sW + wrow * DLD + whalf * 64);
#pragma unroll
      for (int j = 0; j < 4; ++j) dst[j] = decode8(t, wc0[j]);
#pragma unroll
      for (int j = 0; j < 4; ++j) dst[4 + j] = decode8(t, wc1[j]);
    }
    __syncthreads();
    if (st + 1 < s_end) load(st + 1);
#pragma unroll
    for (int nn = 0; nn < DBN / 32; ++nn) {
      u32x4_t a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        a[i] = *reinterpret_cast<const u32x4_t*>(sA + (wm * 64 + i * 16 + fr) * DLD + nn * 32 + fg * 8);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int row = nn * 32 + fg * 8 + tq;
        const int col = wk * 64 + j * 16 + tp * 4;
        const u32x2_t lo = tr16(sW + row * DLD + col);
        const u32x2_t hi = tr16(sW + (row + 4) * DLD + col);
        b[j] = u32x4_t{lo[0], lo[1], hi[0], hi[1]};
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = mfma16x16x32(a[i], b[j], acc[i][j]);
    }
  }

#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int64_t m = m0 + wm * 64 + i * 16 + fg * 4 + e;
        const int64_t k = k0 + wk * 64 + j * 16 + fr;
        if (m < M && k < K) {
          float v = acc[i][j][e];
          if (nsplit > 1) {
            part[((int64_t)split * M + m) * K + k] = v;
          } else {
            if (lora.r > 0) v += lora.scaling * lora_dot_dx(lora, m, k);
            if (dx_bf16)
              reinterpret_cast<uint16_t*>(dX)[m * K + k] = to_bf16(v);
            else
              reinterpret_cast<float*>(dX)[m * K + k] = v;
          }
        }
      }
}

hipError_t launch_gemm_dx(const Nf4View& w, const float* codebook, const uint16_t* dY, int64_t M,
                          const LoraTerm& lora, void* dX, bool dx_bf16, float* part, int nsplit,
                          hipStream_t s) {
  const int nsteps = (int)((w.n + DBN - 1) / DBN);
  const int per = (nsteps + nsplit - 1) / nsplit;
  dim3 grid((unsigned)((w.k + DBK - 1) / DBK), (unsigned)((M + DBM - 1) / DBM), (unsigned)nsplit);
  hipLaunchKernelGGL(k_gemm_dx, grid, dim3(256), 0, s, dY, w, codebook, M, lora, dX, (int)dx_bf16,
                     part, nsplit, per);
  return hipGetLastError();
}

}  // namespace ql
