// Measured ceilings of the part, reported beside the data-sheet peaks: a
// streaming read of a large buffer (two access orders), a device copy, and a
// loop of independent bf16 MFMA 32x32x16 chains.  Measurement probes for the
// benchmark, built as their own library (libqlora_peaks.so); not part of the
// linear layer's path.  Every kernel stays inside the buffers it is given.
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/qlora_peaks.h"

namespace {

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));

constexpr int kThreads = 256;
constexpr int kReadBlocks = 4096;
constexpr int kMfmaBlocks = 1024;   // 4 workgroups of 4 waves per CU: 4 waves per SIMD

// The folded value is stored only if it equals a value the inputs never
// produce, so the loads cannot be dropped and nothing is written in practice.
__device__ __forceinline__ void keep(float v, float* sink) {
  if (v == 1.2345678e-30f) sink[0] = v;
}

// Grid-stride: consecutive threads read consecutive 16-byte pieces.
__global__ __launch_bounds__(kThreads) void k_read_strided(const u32x4_t* __restrict__ p, int64_t n,
                                                           float* sink) {
  uint32_t x = 0;
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n; i += (int64_t)gridDim.x * kThreads) {
    const u32x4_t v = __builtin_nontemporal_load(p + i);
    x ^= v[0] ^ v[1] ^ v[2] ^ v[3];
  }
  keep(__uint_as_float(x), sink);
}

// Each workgroup reads its own contiguous range, four pieces per thread in
// flight.
__global__ __launch_bounds__(kThreads) void k_read_ranges(const u32x4_t* __restrict__ p, int64_t n,
                                                          float* sink) {
  const int64_t per = (n + gridDim.x - 1) / gridDim.x;
  const int64_t b = (int64_t)blockIdx.x * per, e = b + per < n ? b + per : n;
  uint32_t x = 0;
  for (int64_t i = b + threadIdx.x; i < e; i += 4 * kThreads) {
    u32x4_t v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int64_t j = i + u * kThreads;
      v[u] = j < e ? __builtin_nontemporal_load(p + j) : u32x4_t{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) x ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
  }
  keep(__uint_as_float(x), sink);
}

__global__ __launch_bounds__(kThreads) void k_copy(const u32x4_t* __restrict__ s, u32x4_t* __restrict__ d,
                                                   int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n; i += (int64_t)gridDim.x * kThreads)
    __builtin_nontemporal_store(__builtin_nontemporal_load(s + i), d + i);
}

// Eight independent accumulation chains per wave (with four waves per SIMD
// enough to keep the matrix pipe busy; one wave alone, or four chains,
// measured 4-20 % less); operands from registers.
constexpr int kChains = 8;
__global__ __launch_bounds__(kThreads) void k_mfma(int iters, float* sink) {
  const int lane = threadIdx.x & 63;
  bf16x8_t a, b;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    a[e] = (__bf16)(0.001f * (float)((lane + e) & 7));
    b[e] = (__bf16)(0.001f * (float)((lane * 3 + e) & 7));
  }
  f32x16_t c[kChains];
#pragma unroll
  for (int j = 0; j < kChains; ++j) c[j] = f32x16_t{};
  for (int i = 0; i < iters; ++i)
#pragma unroll
    for (int j = 0; j < kChains; ++j) c[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c[j], 0, 0, 0);
  float v = 0.f;
#pragma unroll
  for (int j = 0; j < kChains; ++j)
#pragma unroll
    for (int i = 0; i < 16; ++i) v += c[j][i];
  keep(v, sink);
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

}  // namespace

extern "C" {

int qlora_peak_read(const void* buf, size_t bytes, int contiguous, float* sink, void* stream) {
  if (!buf || !sink) return 1;
  if (bytes == 0 || bytes % 16 != 0 || !aligned16(buf)) return 2;
  const int64_t n = (int64_t)(bytes / 16);
  if (contiguous)
    hipLaunchKernelGGL(k_read_ranges, dim3(kReadBlocks), dim3(kThreads), 0, (hipStream_t)stream,
                       static_cast<const u32x4_t*>(buf), n, sink);
  else
    hipLaunchKernelGGL(k_read_strided, dim3(kReadBlocks), dim3(kThreads), 0, (hipStream_t)stream,
                       static_cast<const u32x4_t*>(buf), n, sink);
  return hipGetLastError() == hipSuccess ? 0 : 3;
}

int qlora_peak_copy(const void* src, void* dst, size_t bytes, void* stream) {
  if (!src || !dst) return 1;
  if (bytes == 0 || bytes % 16 != 0 || !aligned16(src) || !aligned16(dst)) return 2;
  const uintptr_t s = (uintptr_t)src, d = (uintptr_t)dst;
  if (s < d + bytes && d < s + bytes) return 2;   // overlapping buffers
  hipLaunchKernelGGL(k_copy, dim3(kReadBlocks), dim3(kThreads), 0, (hipStream_t)stream,
                     static_cast<const u32x4_t*>(src), static_cast<u32x4_t*>(dst), (int64_t)(bytes / 16));
  return hipGetLastError() == hipSuccess ? 0 : 3;
}

int qlora_peak_mfma(int iters, float* sink, void* stream) {
  if (!sink) return 1;
  if (iters < 1) return 2;
  hipLaunchKernelGGL(k_mfma, dim3(kMfmaBlocks), dim3(kThreads), 0, (hipStream_t)stream, iters, sink);
  return hipGetLastError() == hipSuccess ? 0 : 3;
}

double qlora_peak_mfma_flops(int iters) {
  // workgroups x waves x iterations x chains x 2*32*32*16
  return (double)kMfmaBlocks * (kThreads / 64) * (double)iters * kChains * 2.0 * 32 * 32 * 16;
}

}  // extern "C"
