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
//    different blocks.  The next block's codes, scale and activation
//    fragments are loaded while the current one is decoded.  One launch can
//    cover a list of independent projections (grouped form).
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

// Per-lane work unit of the streaming forward: lane (n = l % 16, g = l / 16)
// of a wave owns the 64-block (n, 4q + g) of quad q: its 32 code bytes, its
// scale, and the activation fragments X[m][64(4q + g) + 8i .. +8], i = 0..7,
// for the 16-row groups of M.  The eight MFMA 16x16x32 steps of a quad
// contract, for each i, word i of the four blocks of the quad.
template <int MT, bool PREX>
struct GemvUnit {
  u32x4_t c0, c1;          // packed words 0-3 and 4-7 of the block
  uint32_t qbyte;
  float step;
  bool ok;
  u32x4_t x[PREX ? MT : 1][8];
};

template <int MT, bool GROUPED>
__global__ __launch_bounds__(256) void k_gemv_fwd(GemvJob job1, const GemvJob* __restrict__ jobs,
                                                  int njobs, const float* __restrict__ codebook,
                                                  int ksplit, int quads_per_split) {
  constexpr bool PREX = MT <= 2;   // activation fragments prefetched with the codes
  __shared__ f32x4_t s_red[3][MT][64];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  int64_t rg = blockIdx.x;
  GemvJob J;
  if constexpr (GROUPED) {
    // the job whose row-group range holds this workgroup (uniform search)
    int lo = 0, hi = njobs - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (jobs[mid].rg_begin <= rg) lo = mid; else hi = mid - 1;
    }
    J = jobs[lo];
    rg -= J.rg_begin;
  } else {
    J = job1;
  }
  const Nf4View& w = J.w;
  const int64_t N = w.n, K = w.k, M = J.M;
  const int nkb = (int)(K / kBlock), nquads = (nkb + 3) / 4;   // loop indices stay 32-bit (SALU)
  const int64_t n = rg * 16 + (lane & 15);
  const bool nok = n < N;
  const int64_t nn = nok ? n : N - 1;
  const int g = lane >> 4;
  const int split = blockIdx.y;
  const int q0 = split * quads_per_split;
  const int q1 = min(nquads, q0 + quads_per_split);

  float lv[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) lv[i] = codebook[i];

  // rows of M past the end are loaded from row M-1 (their outputs are dropped)
  const uint16_t* xrow[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) xrow[mt] = J.X + min((int64_t)(mt * 16 + (lane & 15)), M - 1) * K;

  using U = GemvUnit<MT, PREX>;
  // storage position of (nn, kb): the 16 rows of this row group are
  // contiguous at each k-block, so lane l of a unit reads bytes [32l, 32l+32)
  // of a 2 KiB run (full row group)
  const int64_t g0 = nn & ~int64_t(15);
  const int64_t R = min(int64_t(16), N - g0);
  const int64_t p0 = g0 * nkb + (nn - g0);
  auto load = [&](int q, U& u) {
    const int kb = 4 * q + g;
    u.ok = nok && kb < nkb;
    const int kbc = min(kb, nkb - 1);
    const int64_t b = nn * nkb + kbc;
    const int64_t p = p0 + kbc * R;
    const u32x4_t* src = reinterpret_cast<const u32x4_t*>(w.codes + p * 32);
    u.c0 = src[0];
    u.c1 = src[1];
    u.qbyte = w.qscale[p];
    u.step = w.step[b >> 8];
    if constexpr (PREX) {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int i = 0; i < 8; ++i)
          u.x[mt][i] = *reinterpret_cast<const u32x4_t*>(xrow[mt] + (int64_t)kbc * kBlock + i * 8);
    }
  };

  f32x4_t acc[MT][2];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) acc[mt][0] = acc[mt][1] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  auto compute = [&](int q, const U& u) {
    const float sc = u.ok ? (float)u.qbyte * u.step : 0.f;
    const Lut t = make_lut(lv, sc);
    const int kbc = min(4 * q + g, nkb - 1);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const u32x4_t bf = decode8(t, i < 4 ? u.c0[i] : u.c1[i - 4]);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        u32x4_t af;
        if constexpr (PREX)
          af = u.x[mt][i];
        else
          af = *reinterpret_cast<const u32x4_t*>(xrow[mt] + (int64_t)kbc * kBlock + i * 8);
        acc[mt][i & 1] = mfma16x16x32(af, bf, acc[mt][i & 1]);
      }
    }
  };

  // quads q0 + wave + 4j of this split, one unit ahead: the loads of the
  // next unit are issued (and kept, by the scheduling fences) before the
  // current unit is decoded, whose own loads are then the only ones waited for
  constexpr int NLOAD = 4 + (PREX ? 8 * MT : 0);   // vector loads per unit
  const int qlast = q1 - 1;
  int q = q0 + wave;
  if (q < q1) {
    U u0, u1;
    load(q, u0);
    for (;;) {
      load(min(q + 4, qlast), u1);
      __builtin_amdgcn_sched_barrier(0);
      QL_VMCNT(NLOAD);
      __builtin_amdgcn_sched_barrier(0);
      compute(q, u0);
      __builtin_amdgcn_sched_barrier(0);
      q += 4;
      if (q >= q1) break;
      load(min(q + 4, qlast), u0);
      __builtin_amdgcn_sched_barrier(0);
      QL_VMCNT(NLOAD);
      __builtin_amdgcn_sched_barrier(0);
      compute(q, u1);
      __builtin_amdgcn_sched_barrier(0);
      q += 4;
      if (q >= q1) break;
    }
  }

  f32x4_t tot[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) tot[mt] = acc[mt][0] + acc[mt][1];
  if (wave > 0)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) s_red[wave - 1][mt][lane] = tot[mt];
  __syncthreads();
  if (wave != 0) return;
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    f32x4_t v = tot[mt];
    v += s_red[0][mt][lane];
    v += s_red[1][mt][lane];
    v += s_red[2][mt][lane];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int64_t m = mt * 16 + g * 4 + e;
      if (m < M && nok) {
        float y = v[e];
        if (ksplit > 1) {
          J.part[((int64_t)split * M + m) * N + n] = y;
        } else {
          if (J.lora.r > 0) y += J.lora.scaling * lora_dot(J.lora, m, n);
          store_out(J.Y, J.y_bf16, m * N + n, y);
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
  const GemvJob job{X, w, lora, Y, part, M, (int)y_bf16, 0};
  dim3 grid((unsigned)((w.n + 15) / 16), (unsigned)ksplit);
  const int mt = (int)((M + 15) / 16);
#define QL_GEMV(MT)                                                                             \
  hipLaunchKernelGGL((k_gemv_fwd<MT, false>), grid, dim3(256), 0, s, job, nullptr, 0, codebook, \
                     ksplit, per)
  switch (mt) {
    case 1: QL_GEMV(1); break;
    case 2: QL_GEMV(2); break;
    case 3: QL_GEMV(3); break;
    default: QL_GEMV(4); break;
  }
#undef QL_GEMV
  return hipGetLastError();
}

hipError_t launch_gemv_grouped(const GemvJob* jobs, int njobs, int64_t row_groups, int64_t M,
                               const float* codebook, int64_t max_quads, hipStream_t s) {
  dim3 grid((unsigned)row_groups, 1);
  const int mt = (int)((M + 15) / 16);
  const GemvJob none{};
#define QL_GEMV(MT)                                                                           \
  hipLaunchKernelGGL((k_gemv_fwd<MT, true>), grid, dim3(256), 0, s, none, jobs, njobs,        \
                     codebook, 1, (int)max_quads)
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
