// LoRA branch pieces (www.lqnn.cn/news/228537 §3.2; www.cf-1.com/news/5705389
// §2.1, §3.2): the rank-r projections T = X A^T and U = dY B, and the adapter
// weight gradients dA = s U^T X and dB = s dY^T T.  T and U stay fp32.
#include "common.h"
#include "kernels.h"

namespace ql {

QL_DEV u32x4_t load8_guard(const uint16_t* row, int64_t c, int64_t C, bool vec) {
  if (vec && c + 8 <= C) return *reinterpret_cast<const u32x4_t*>(row + c);
  if (c >= C) return u32x4_t{0u, 0u, 0u, 0u};
  uint32_t h[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) h[e] = (c + e < C) ? row[c + e] : 0u;
  return u32x4_t{h[0] | h[1] << 16, h[2] | h[3] << 16, h[4] | h[5] << 16, h[6] | h[7] << 16};
}

// out[m][j] = sum_c P[m][c] Q[j][c]: an output tile of `rows` (16, or 8 so
// that a few thousand rows still spread over every compute unit) x 16 ranks
// per workgroup of 16 waves; wave w takes the 32-wide contraction slices w,
// w+16, ... and keeps four independent accumulators (four loads in flight);
// the 16 partial tiles are summed in a fixed order through LDS.  bf16
// products are exact, sums fp32.
constexpr int RD_WAVES = 16;
template <bool GROUPED>
__global__ __launch_bounds__(1024) void k_rowdot(const uint16_t* __restrict__ P,
                                                 const uint16_t* __restrict__ Q, int64_t M,
                                                 int64_t C, int r, float* __restrict__ out,
                                                 const RowdotJob* __restrict__ jobs, int rows) {
  if constexpr (GROUPED) {
    const RowdotJob& J = jobs[blockIdx.z];
    P = J.P;
    Q = J.Q;
    out = J.out;
    C = J.C;
    r = J.r;
    if ((int)blockIdx.y * 16 >= r) return;
  }
  __shared__ f32x4_t s_red[RD_WAVES][64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t m = (int64_t)blockIdx.x * rows + (lane & 15);
  const int64_t j = (int64_t)blockIdx.y * 16 + (lane & 15);
  const int g = lane >> 4;
  const bool vec = (C % 8) == 0;
  const bool mok = (lane & 15) < rows && m < M, jok = j < r;
  f32x4_t acc[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) acc[u] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  const int64_t stride = 32 * RD_WAVES;
  for (int64_t c0 = wave * 32; c0 < C; c0 += 4 * stride) {
    u32x4_t a[4], b[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int64_t c = c0 + u * stride + g * 8;
      a[u] = mok ? load8_guard(P + m * C, c, C, vec) : u32x4_t{0u, 0u, 0u, 0u};
      b[u] = jok ? load8_guard(Q + j * C, c, C, vec) : u32x4_t{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) acc[u] = mfma16x16x32(a[u], b[u], acc[u]);
  }
  s_red[wave][lane] = (acc[0] + acc[1]) + (acc[2] + acc[3]);
  __syncthreads();
  if (wave != 0) return;
  f32x4_t v = s_red[0][lane];
  for (int w = 1; w < RD_WAVES; ++w) v += s_red[w][lane];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int64_t mm = (int64_t)blockIdx.x * rows + g * 4 + e;
    if (g * 4 + e < rows && mm < M && jok) out[mm * r + j] = v[e];
  }
}

// Qt[j][n] = Q[n][j]; thread (j, n) with n fastest, so the writes coalesce
// (N * r < 2^31).
__global__ void k_transpose_bf16(const uint16_t* __restrict__ Q, int N, int r,
                                 uint16_t* __restrict__ Qt) {
  const int n = (int)blockIdx.x * 256 + (int)threadIdx.x, j = (int)blockIdx.y;
  if (n < N) Qt[(int64_t)j * N + n] = Q[(int64_t)n * r + j];
}

// Partial weight gradient over a slice of WG_ROWS rows m:
//   part[split][j][c] = sum_{m in slice} Q[m][j] * P[m][c]
// A workgroup owns 128 columns (two per lane) and eight ranks j (blockIdx.z);
// the slice's Q values (128 rows x 8 ranks) are staged in LDS and read back as
// broadcasts; wave w takes rows [32w, 32w+32) with all 32 P loads issued
// before the FMAs, and the four wave partials are summed through LDS in a
// fixed order.
constexpr int WG_ROWS = 128;
__global__ __launch_bounds__(256) void k_wgrad(const uint16_t* __restrict__ P,
                                               const float* __restrict__ Q, int64_t M, int64_t C,
                                               int r, float scaling, float* __restrict__ out,
                                               int transpose_out, float* __restrict__ part,
                                               int msplit, int rows_per_split) {
  __shared__ float s_red[3][8][128];
  __shared__ __attribute__((aligned(16))) float sQ[WG_ROWS][8];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int cl = lane * 2;                                  // local column pair
  const int64_t c = (int64_t)blockIdx.x * 128 + cl;
  const int split = blockIdx.y;
  const int j0 = blockIdx.z * 8;
  const int64_t mb = (int64_t)split * rows_per_split + wave * 32;
  {
    // 1024 values, 4 per thread: row tid/2, ranks 4*(tid&1) .. +3
    const int row = tid >> 1, jq = (tid & 1) * 4;
    const int64_t m = (int64_t)split * rows_per_split + row;
#pragma unroll
    for (int e = 0; e < 4; ++e)
      sQ[row][jq + e] = (m < M && j0 + jq + e < r) ? Q[m * r + j0 + jq + e] : 0.f;
  }
  const bool pair = (C % 2) == 0 && c + 1 < C;
  float acc0[8], acc1[8];
#pragma unroll
  for (int t = 0; t < 8; ++t) acc0[t] = acc1[t] = 0.f;
  uint32_t pv[32];
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    const int64_t m = mb + i;
    uint32_t v = 0;
    if (m < M && c < C) {
      if (pair)
        v = *reinterpret_cast<const uint32_t*>(P + m * C + c);
      else
        v = (uint32_t)P[m * C + c] | (c + 1 < C ? (uint32_t)P[m * C + c + 1] << 16 : 0u);
    }
    pv[i] = v;
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    const float p0 = bf16_lo(pv[i]), p1 = bf16_hi(pv[i]);
    const f32x4_t qa = *reinterpret_cast<const f32x4_t*>(&sQ[wave * 32 + i][0]);
    const f32x4_t qb = *reinterpret_cast<const f32x4_t*>(&sQ[wave * 32 + i][4]);
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      acc0[t] += qa[t] * p0;
      acc1[t] += qa[t] * p1;
      acc0[4 + t] += qb[t] * p0;
      acc1[4 + t] += qb[t] * p1;
    }
  }
  if (wave > 0) {
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      s_red[wave - 1][t][cl] = acc0[t];
      s_red[wave - 1][t][cl + 1] = acc1[t];
    }
  }
  __syncthreads();
  if (wave != 0 || c >= C) return;
#pragma unroll
  for (int w = 0; w < 3; ++w)
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      acc0[t] += s_red[w][t][cl];
      acc1[t] += s_red[w][t][cl + 1];
    }
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
  // partials added in split order; eight loads in flight at a time
  const int64_t stride = (int64_t)r * C;
  float v = 0.f;
  int s = 0;
  for (; s + 8 <= msplit; s += 8) {
    float t[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) t[u] = part[(int64_t)(s + u) * stride + idx];
#pragma unroll
    for (int u = 0; u < 8; ++u) v += t[u];
  }
  for (; s < msplit; ++s) v += part[(int64_t)s * stride + idx];
  const int64_t j = idx / C, c = idx % C;
  if (transpose_out)
    out[c * r + j] = scaling * v;
  else
    out[idx] = scaling * v;
}

hipError_t launch_rowdot(const uint16_t* P, const uint16_t* Q, int64_t M, int64_t C, int r,
                         float* out, hipStream_t s) {
  // 8-row tiles when 16-row tiles would leave compute units idle
  const int rows = ((M + 15) / 16) * ((r + 15) / 16) < 512 ? 8 : 16;
  dim3 grid((unsigned)((M + rows - 1) / rows), (unsigned)((r + 15) / 16));
  hipLaunchKernelGGL(k_rowdot<false>, grid, dim3(64 * RD_WAVES), 0, s, P, Q, M, C, r, out,
                     nullptr, rows);
  return hipGetLastError();
}

hipError_t launch_rowdot_grouped(const RowdotJob* jobs, int njobs, int64_t M, int max_r,
                                 hipStream_t s) {
  dim3 grid((unsigned)((M + 15) / 16), (unsigned)((max_r + 15) / 16), (unsigned)njobs);
  hipLaunchKernelGGL(k_rowdot<true>, grid, dim3(64 * RD_WAVES), 0, s, nullptr, nullptr, M,
                     int64_t(0), 0, nullptr, jobs, 16);
  return hipGetLastError();
}

hipError_t launch_transpose_bf16(const uint16_t* Q, int64_t N, int r, uint16_t* Qt, hipStream_t s) {
  hipLaunchKernelGGL(k_transpose_bf16, dim3((unsigned)((N + 255) / 256), (unsigned)r), dim3(256), 0,
                     s, Q, (int)N, r, Qt);
  return hipGetLastError();
}

hipError_t launch_wgrad(const uint16_t* P, const float* Q, int64_t M, int64_t C, int r,
                        float scaling, float* out, bool transpose_out, float* part, int msplit,
                        hipStream_t s) {
  const int rows = WG_ROWS;   // msplit == ceil(M / WG_ROWS), chosen by the caller
  dim3 grid((unsigned)((C + 127) / 128), (unsigned)msplit, (unsigned)((r + 7) / 8));
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
