// Conversion of a packed weight between the library's layout and the plain
// flat layout (news.rkmt.cn/news/4821 §4.2: 4-bit codes two per uint8 byte;
// §1.2, §2.2: one constant per block and per group of block constants).
//
// Library layout: 64-weight units (one row, 64 consecutive k) in 16-row
// groups, k-block-major inside a group; inside a unit's 32 code bytes the
// 4-byte word w holds elements 8w..8w+7, byte j = code(8w+j) | code(8w+j+4) << 4.
// Plain layout: units and block constants in flat row-major order, byte j of
// the code stream = code(2j) | code(2j+1) << 4.  Both layouts hold a word's
// eight elements in the same four bytes, so each word converts on its own.
#include "common.h"

#include <algorithm>

#include "kernels.h"

namespace ql {

// nibble position of element e (0..7) of a library word
QL_DEV int lib_nibble(int e) { return e < 4 ? 2 * e : 2 * e - 7; }

QL_DEV uint32_t word_to_plain(uint32_t w) {
  uint32_t p = 0;
#pragma unroll
  for (int e = 0; e < 8; ++e) p |= ((w >> (4 * lib_nibble(e))) & 0xFu) << (4 * e);
  return p;
}

QL_DEV uint32_t word_from_plain(uint32_t p) {
  uint32_t w = 0;
#pragma unroll
  for (int e = 0; e < 8; ++e) w |= ((p >> (4 * e)) & 0xFu) << (4 * lib_nibble(e));
  return w;
}

// Unit (row, kb) of a k-block grid nkb wide: its library position.
QL_DEV int64_t lib_position(int64_t row, int64_t kb, int64_t n, int64_t nkb) {
  const int64_t g0 = row & ~int64_t(15);
  const int64_t R = min(int64_t(16), n - g0);
  return g0 * nkb + kb * R + (row - g0);
}

// One thread per 64-weight unit (grid-stride): its code bytes and its block
// constants move between the unit's flat index f and its library position
// p; the threads below the number of second-level groups also copy the group
// constants, which are flat in both layouts.
__global__ __launch_bounds__(256) void k_relayout(const uint8_t* __restrict__ sc,
                                                  const uint8_t* __restrict__ sq,
                                                  const float* __restrict__ ss,
                                                  uint8_t* __restrict__ dc, uint8_t* __restrict__ dq,
                                                  float* __restrict__ ds, int64_t n, int64_t k,
                                                  int fmt, int to_plain) {
  const int64_t nkb = k / 64, units = n * nkb;
  const int64_t t0 = (int64_t)blockIdx.x * 256 + threadIdx.x, stride = (int64_t)gridDim.x * 256;
  const bool dq2 = fmt == kFmtNf4Dq || fmt == kFmtNf4Dq32 || fmt == kFmtNf4Dq128 ||
                   fmt == kFmtNf4DqF16;
  for (int64_t f = t0; f < units; f += stride) {
    const int64_t row = f / nkb, kb = f - row * nkb;
    const int64_t p = lib_position(row, kb, n, nkb);
    const int64_t si = to_plain ? p : f, di = to_plain ? f : p;
    if (fmt == kFmtQ8) {   // 64 int8 codes in element order in both layouts
      const u32x4_t* s4 = reinterpret_cast<const u32x4_t*>(sc + 64 * si);
      u32x4_t* d4 = reinterpret_cast<u32x4_t*>(dc + 64 * di);
#pragma unroll
      for (int i = 0; i < 4; ++i) d4[i] = s4[i];
      reinterpret_cast<uint32_t*>(dq)[di] = reinterpret_cast<const uint32_t*>(sq)[si];
      continue;
    }
    const u32x4_t* s4 = reinterpret_cast<const u32x4_t*>(sc + 32 * si);
    u32x4_t* d4 = reinterpret_cast<u32x4_t*>(dc + 32 * di);
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      u32x4_t v = s4[i];
#pragma unroll
      for (int j = 0; j < 4; ++j) v[j] = to_plain ? word_to_plain(v[j]) : word_from_plain(v[j]);
      d4[i] = v;
    }
    switch (fmt) {
      case kFmtNf4Dq:
      case kFmtNf4DqF16: dq[di] = sq[si]; break;
      case kFmtNf4Dq32: dq[2 * di] = sq[2 * si]; dq[2 * di + 1] = sq[2 * si + 1]; break;
      case kFmtNf4: ds[di] = ss[si]; break;
      case kFmtNf4_32:
      case kFmtU4: ds[2 * di] = ss[2 * si]; ds[2 * di + 1] = ss[2 * si + 1]; break;
      case kFmtNf4Dq128:
      case kFmtNf4_128:
        if ((kb & 1) == 0) {   // one constant per unit pair, on a k/128 block grid
          const int64_t kb2 = kb >> 1, nkb2 = nkb >> 1;
          const int64_t p2 = lib_position(row, kb2, n, nkb2), f2 = row * nkb2 + kb2;
          const int64_t s2 = to_plain ? p2 : f2, d2 = to_plain ? f2 : p2;
          if (fmt == kFmtNf4Dq128) dq[d2] = sq[s2];
          else ds[d2] = ss[s2];
        }
        break;
      default: break;
    }
  }
  if (dq2) {
    const int64_t block = fmt == kFmtNf4Dq32 ? 32 : (fmt == kFmtNf4Dq128 ? 128 : 64);
    const int64_t groups = (n * k / block + 255) / 256;
    for (int64_t g = t0; g < groups; g += stride) ds[g] = ss[g];
  }
}

hipError_t launch_relayout(const uint8_t* sc, const uint8_t* sq, const float* ss, uint8_t* dc,
                           uint8_t* dq, float* ds, int64_t n, int64_t k, int fmt, bool to_plain,
                           hipStream_t s) {
  const int64_t units = n * (k / 64);
  const int64_t blocks = std::min<int64_t>((units + 255) / 256, 8192);
  hipLaunchKernelGGL(k_relayout, dim3((unsigned)std::max<int64_t>(blocks, 1)), dim3(256), 0, s, sc, sq,
                     ss, dc, dq, ds, n, k, fmt, (int)to_plain);
  return hipGetLastError();
}

}  // namespace ql
