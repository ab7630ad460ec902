// LoRA branch pieces (www.lqnn.cn/news/228537 §3.2; www.cf-1.com/news/5705389
// §2.1, §3.2): the rank-r projections T = X A^T and U = dY B, and the adapter
// weight gradients dA = s U^T X and dB = s dY^T T.  T and U stay fp32.
#include "common.h"
#include "kernels.h"

namespace ql {

QL_DEV u32x4_t load8_guard(const uint16_t* row, int64_t c, int64_t C, bool vec) {
  if (vec && c + 8 <= C) return *reinterpret_cast<const u32x4_t*>(row + c);
  uint32_t h[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) h[e] = (c + e < C) ? row[c + e] : 0u;
  return u32x4_t{h[0] | h[1] << 16, h[2] | h[3] << 16, h[4] | h[5] << 16, h[6] | h[7] << 16};
}

// out[m][j] = sum_c P[m][c] Q[j][c]: a 16 x 16 output tile per workgroup, the
// four waves take interleaved 32-wide slices of the contraction and are summed
// in a fixed order through LDS.  bf16 products are exact; sums are fp32.
__global__ __launch_bounds__(256) void k_rowdot(const uint16_t* __restrict__ P,
                                                const uint16_t* __restrict__ Q, int64_t M,
                                                int64_t C, int r, float* __restrict__ out) {
  __shared__ f32x4_t s_red[3][64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t m = (int64_t)blockIdx.x * 16 + (lane & 15);
  const int64_t j = (int64_t)blockIdx.y * 16 + (lane & 15);
  const int g = lane >> 4;
  const bool vec = (C % 8) == 0;
  f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
  for (int64_t c0 = wave * 32; c0 < C; c0 += 128) {
    const int64_t c = c0 + g * 8;
    const u32x4_t a = m < M ? load8_guard(P + m * C, c, C, vec) : u32x4_t{0u, 0u, 0u, 0u};
    const u32x4_t b = j < r ? load8_guard(Q + j * C, c, C, vec) : u32x4_t{0u, 0u, 0u, 0u};
    acc = mfma16x16x32(a, b, acc);
  }
  if (wave > 0) s_red[wave - 1][lane] = acc;
  __syncthreads();
  if (wave != 0) return;
  acc += s_red[0][lane];
  acc += s_red[1][lane];
  acc += s_red[2][lane];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int64_t mm = (int64_t)blockIdx.x * 16 + g * 4 + e;
    if (mm < M && j < r) out[mm * r + j] = acc[e];
  }
}

__global__ void k_transpose_bf16(const uint16_t* __restrict__ Q, int64_t N, int r,
                                 uint16_t* __restrict__ Qt) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= N * r) return;
  const int64_t n = idx / r, j = idx % r;
  Qt[j * N + n] = Q[idx];
}

// Partial weight gradient over a slice of rows m:
//   part[split][j][c] = sum_{m in slice} Q[m][j] * P[m][c]
// Each thread owns two adjacent columns c and eight ranks j (blockIdx.z).
__global__ __launch_bounds__(256) void k_wgrad(const uint16_t* __restrict__ P,
                                               const float* __restrict__ Q, int64_t M, int64_t C,
                                               int r, float scaling, float* __restrict__ out,
                                               int transpose_out, float* __restrict__ part,
                                               int msplit, int rows_per_split) {
  const int64_t c = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 2;
  const int split = blockIdx.y;
  const int j0 = blockIdx.z * 8;
  const int64_t mb = (int64_t)split * rows_per_split;
  const int64_t me = min(M, mb + rows_per_split);
  const bool pair = (C % 2) == 0 && c + 1 < C;
  float acc0[8], acc1[8];
#pragma unroll
  for (int t = 0; t < 8; ++t) acc0[t] = acc1[t] = 0.f;
  if (c < C) {
    for (int64_t m = mb; m < me; ++m) {
      float p0, p1;
      if (pair) {
        const uint32_t v = *reinterpret_cast<const uint32_t*>(P + m * C + c);
        p0 = bf16_lo(v);
        p1 = bf16_hi(v);
      } else {
        p0 = __builtin_bit_cast(float, (uint32_t)P[m * C + c] << 16);
        p1 = c + 1 < C ? __builtin_bit_cast(float, (uint32_t)P[m * C + c + 1] << 16) : 0.f;
      }
      const float* q = Q + m * r + j0;
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        if (j0 + t < r) {
          const float qv = q[t];
          acc0[t] += qv * p0;
          acc1[t] += qv * p1;
        }
      }
    }
  }
  if (c >= C) return;
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    const int j = j0 + t;
    if (j >= r) break;
    if (msplit > 1) {
      float* dst = part + ((int64_t)split * r + j) * C + c;
      dst[0] = acc0[t];
      if (c + 1 < C) dst[1] = acc1[t];
    } else if (transpose_out) {
      out[c * r + j] = scaling * acc0[t];
      if (c + 1 < C) out[(c + 1) * r + j] = scaling * acc1[t];
    } else {
      out[(int64_t)j * C + c] = scaling * acc0[t];
      if (c + 1 < C) out[(int64_t)j * C + c + 1] = scaling * acc1[t];
    }
  }
}

__global__ __launch_bounds__(256) void k_wgrad_reduce(const float* __restrict__ part, int msplit,
                                                      int64_t C, int r, float scaling,
                                                      float* __restrict__ out, int transpose_out) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;   // = j * C + c
  if (idx >= (int64_t)r * C) return;
  float v = 0.f;
  for (int s = 0; s < msplit; ++s) v += part[(int64_t)s * r * C + idx];
  const int64_t j = idx / C, c = idx % C;
  if (transpose_out)
    out[c * r + j] = scaling * v;
  else
    out[idx] = scaling * v;
}

hipError_t launch_rowdot(const uint16_t* P, const uint16_t* Q, int64_t M, int64_t C, int r,
                         float* out, hipStream_t s) {
  dim3 grid((unsigned)((M + 15) / 16), (unsigned)((r + 15) / 16));
  hipLaunchKernelGGL(k_rowdot, grid, dim3(256), 0, s, P, Q, M, C, r, out);
  return hipGetLastError();
}

hipError_t launch_transpose_bf16(const uint16_t* Q, int64_t N, int r, uint16_t* Qt, hipStream_t s) {
  const int64_t total = N * r;
  hipLaunchKernelGGL(k_transpose_bf16, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s, Q, N,
                     r, Qt);
  return hipGetLastError();
}

hipError_t launch_wgrad(const uint16_t* P, const float* Q, int64_t M, int64_t C, int r,
                        float scaling, float* out, bool transpose_out, float* part, int msplit,
                        hipStream_t s) {
  const int rows = (int)((M + msplit - 1) / msplit);
  dim3 grid((unsigned)((C + 511) / 512), (unsigned)msplit, (unsigned)((r + 7) / 8));
  hipLaunchKernelGGL(k_wgrad, grid, dim3(256), 0, s, P, Q, M, C, r, scaling, out,
                     (int)transpose_out, part, msplit, rows);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || msplit == 1) return e;
  const int64_t total = (int64_t)r * C;
  hipLaunchKernelGGL(k_wgrad_reduce, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s, part,
                     msplit, C, r, scaling, out, (int)transpose_out);
  return hipGetLastError();
}

}  // namespace ql
