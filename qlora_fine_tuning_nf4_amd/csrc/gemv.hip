// Forward base product of the quantized linear, Y = X deq(W)^T (+ LoRA term),
// with the packed weight dequantized to bf16 inside the kernels and never
// written to global memory (www.cf-1.com/news/5705389 §2.2 and §4.2: block
// dequantization inside the GEMM, results kept in registers / shared memory;
// www.lqnn.cn/news/228537 §3.3 and zky001 section 5.8: dequantize to 16 bits
// for the product, then discard).
//
// Small-M forward (the large-M GEMMs are in gemm.hip) and the split-K reduce.
//  * k_gemv_fwd  -- small M (<= 32): a wave owns 16 weight rows and streams
//    their packed bytes; each lane decodes a whole 64-weight unit (one lookup
//    table per 4-bit block; Q8_0 bytes times their fp16 scale) and feeds
//    eight MFMAs whose 32-wide contraction spans four different units.  The next block's codes, scale and activation
//    fragments are loaded while the current one is decoded.  One launch can
//    cover a list of independent projections (grouped form).
#include "common.h"
#include "kernels.h"

#include <algorithm>
#include <type_traits>

namespace ql {

// R and 16-bit outputs: fp16 when F16, else bf16
template <bool F16>
QL_DEV float lora_dot(const LoraTerm& L, int64_t m, int64_t c) {
  float acc = 0.f;
  const float* lr = L.L + m * L.r;
  const uint16_t* rr = L.R + c * L.rs_c;
  for (int j = 0; j < L.r; ++j) acc += lr[j] * w16<F16>(rr[j * L.rs_j]);
  return acc;
}

template <bool F16>
QL_DEV void store_out(void* out, bool out16, int64_t idx, float v) {
  if (out16)
    gptr_w(reinterpret_cast<uint16_t*>(out))[idx] = to16<F16>(v);
  else
    gptr_w(reinterpret_cast<float*>(out))[idx] = v;
}

// LoRA term of one output: scaling * sum_j L[m][j] R[c][j], with 16-byte loads
// when the rank and the pointers allow it.
template <bool F16>
QL_DEV float lora_dot_v(const LoraTerm& L, int64_t m, int64_t c, bool vec) {
  const QL_GLOBAL float* lr = gptr(L.L + m * L.r);
  const QL_GLOBAL uint16_t* rr = gptr(L.R + c * L.rs_c);
  float acc = 0.f;
  int j = 0;
  if (vec) {
    for (; j + 8 <= L.r; j += 8) {
      const u32x4_t bv = *reinterpret_cast<const QL_GLOBAL u32x4_t*>(rr + j);
      const f32x4_t t0 = *reinterpret_cast<const QL_GLOBAL f32x4_t*>(lr + j);
      const f32x4_t t1 = *reinterpret_cast<const QL_GLOBAL f32x4_t*>(lr + j + 4);
      acc += t0[0] * lo16<F16>(bv[0]) + t0[1] * hi16<F16>(bv[0]) + t0[2] * lo16<F16>(bv[1]) +
             t0[3] * hi16<F16>(bv[1]) + t1[0] * lo16<F16>(bv[2]) + t1[1] * hi16<F16>(bv[2]) +
             t1[2] * lo16<F16>(bv[3]) + t1[3] * hi16<F16>(bv[3]);
    }
  }
  for (; j < L.r; ++j) acc += lr[j] * w16<F16>(rr[j]);
  return acc;
}

// rsrc_bytes for a wave-uniform, non-negative count, on the scalar unit:
// this part has no scalar 64-bit ordered compare, and in C the clamp becomes
// a vector-ALU 64-bit compare once per quad (any bit at or above bit 31 means
// the count exceeds the clamp).
QL_DEV uint32_t rsrc_bytes_u(int64_t b) {
  uint32_t r;
  uint64_t t;
  asm("s_lshr_b64 %1, %2, 31\n\t"
      "s_cmp_lg_u64 %1, 0\n\t"
      "s_cselect_b32 %0, 0x7fffffff, %3"
      : "=s"(r), "=&s"(t)
      : "s"(b), "s"((uint32_t)b)
      : "scc");
  return r;
}

// Streaming forward, small M.  A workgroup of 4 waves owns 64 weight rows
// (wave w: the 16-row group 4 * blockIdx.x + w) and walks the quads (4
// blocks = 256 k) of its split in step.  Per quad, lane l (n = l % 16,
// g = l / 16) decodes the 64-block (n, 4q + g): 32 code bytes read as part of
// one coalesced 2 KiB run (tiled storage order), one lookup table, eight
// decoded words; MFMA 16x16x32 step i contracts word i of the four blocks.
// The activation chunk X[0..M)[256q, 256q + 256) goes global -> LDS once per
// workgroup with the LDS DMA (rows XOR-swizzled in 16-byte units so the
// fragment reads of 16 different rows hit 16 different bank groups) and is
// read from there by all four waves.  Three-deep rings (LDS chunks, code
// registers) keep the loads of quad q+2 in flight while quad q is computed;
// one barrier per quad.
template <int FMT>
struct GemvRaw {
  u32x4_t c[FMT == kFmtQ8 ? 4 : 2];   // the lane's unit: 32 code bytes, or 64 int8 values
  uint32_t qbyte;   // NF4 with double quantization: the 8-bit scale; Q8_0: the two fp16 scales
  float step;       // NF4: the group's fp32 constant, or the block absmax; uint4: the scale
  float zp;         // uint4: the zero-point; NF4 single level at block 32: the second half's absmax
};

constexpr int GV_CHUNK_BYTES = 512;   // one row of an activation chunk: 256 bf16

// XPW: activation-chunk DMA instructions per wave and quad (8 * XPW chunk
// rows: XPW = 1 for M <= 8, 2 for M <= 16, 4 for M <= 32).
// Waves per SIMD the small-M forward is held to: four for one 16-row tile (its
// registers fit 128 without spilling, where the unconstrained build takes 132
// and runs three), except for the formats that would spill (Q8_0, block 32).
template <int MT, int FMT>
constexpr int gv_waves() { return MT == 1 && FMT != kFmtQ8 && FMT != kFmtNf4Dq32 && FMT != kFmtNf4_32 ? 4 : 1; }

template <int MT, int XPW, bool GROUPED, int FMT>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(gv_waves<MT, FMT>()))) void k_gemv_fwd(GemvJob job1, const GemvJob* __restrict__ jobs,
                                                  int njobs, const float* __restrict__ codebook,
                                                  int ksplit, int quads_per_split) {
  constexpr int XROWS = 8 * XPW;                           // rows of a chunk stage
  constexpr int XSTAGE = XROWS * GV_CHUNK_BYTES / 2;       // bf16 elements per stage
  // three separate chunk stages: distinct LDS objects let the compiler see
  // that the DMA into one stage does not feed the reads of another
  __shared__ __attribute__((aligned(16))) uint16_t sX0[XSTAGE];
  __shared__ __attribute__((aligned(16))) uint16_t sX1[XSTAGE];
  __shared__ __attribute__((aligned(16))) uint16_t sX2[XSTAGE];
  auto stage_ptr = [&](int st) { return st == 0 ? sX0 : (st == 1 ? sX1 : sX2); };
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  int64_t wg = blockIdx.x;
  GemvJob J;
  if constexpr (GROUPED) {
    // the job whose workgroup range holds this workgroup (uniform search)
    int lo = 0, hi = njobs - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (jobs[mid].rg_begin <= wg) lo = mid; else hi = mid - 1;
    }
    J = jobs[lo];
    wg -= J.rg_begin;
  } else {
    J = job1;
  }
  const Nf4View& w = J.w;
  const int64_t N = w.n, K = w.k, M = J.M;
  const int nkb = (int)(K / kBlock), nquads = (nkb + 3) / 4;
  const int64_t g0 = (wg * 4 + wave) * 16;                 // this wave's row group
  const int64_t n = g0 + (lane & 15);
  const bool nok = n < N;
  // rows past N read (and discard) the last row; its group gives the layout
  const int64_t nn = min(n, N - 1);
  const int64_t gg = min(g0, (N - 1) & ~int64_t(15));      // = nn & ~15, uniform
  const int64_t R = min(int64_t(16), N - gg);              // rows of the group
  const int g = lane >> 4;
  const int split = blockIdx.y;
  const int q0 = split * quads_per_split;
  const int q1 = min(nquads, q0 + quads_per_split);

  using FI = FmtInfo<FMT>;
  constexpr int CB = FI::code_bytes, NC = CB / 16;   // code bytes per unit, 16-byte loads
  // the 16 levels are the same in every lane: scalar registers
  float lv[16];
#pragma unroll
  for (int i = 0; i < 16; ++i)
    lv[i] = FI::nf4 ? __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(
                                                   __builtin_bit_cast(int, gptr(codebook)[i])))
                    : 0.f;

  // DMA of an activation chunk: instruction j covers chunk rows 2j, 2j+1;
  // instruction j is issued by wave j % 4.  Lane l writes LDS bytes
  // [16l, 16l + 16) of the instruction's 1 KiB: row 2j + l / 32, physical
  // 16-byte column l % 32, which holds logical column (l % 32) ^ (row % 16).
  // Every wave issues XPW DMA instructions per chunk (a compile-time count,
  // so the waits below are exact): instruction j = wave + 4t covers chunk
  // rows 2j, 2j+1; rows past M re-read row M-1 (their products are dropped).
  // All loads are buffer loads from a per-quad base in scalar registers with
  // a fixed per-lane offset.  A ragged last quad (k % 256 != 0) reads, past
  // the row end, the next row or zeros past the end of the buffer; those
  // values meet blocks whose scale is forced to zero.
  // XPW <= 4; a fixed-size array (one sized by the template parameter, used as
  // a buffer-load offset, made the host pass drop the kernel stubs)
  uint32_t x_vo[4] = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int t = 0; t < XPW; ++t) {
    const int j = wave + 4 * t;
    const int row = 2 * j + (lane >> 5);
    const int col = (lane & 31) ^ (row & 15);
    x_vo[t] = (uint32_t)((min((int64_t)row, M - 1) * K + 8 * col) * 2);
  }
  const uint32_t x_bytes = (uint32_t)(M * K * 2);
  auto load_x = [&](int q, int stage) {
    const uint32_t off = (uint32_t)min(q, nquads - 1) * 512u;   // first k of the quad, bytes
    const auto rs = buf_rsrc(reinterpret_cast<const uint8_t*>(J.X) + off, x_bytes - off);
#pragma unroll
    for (int t = 0; t < XPW; ++t) {
      const int j = wave + 4 * t;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (QL_LDS void*)(stage_ptr(stage) + j * 512), 16,
                                               x_vo[t], 0, 0, 0);
    }
  };
  // unit (nn, 4q + g) sits at storage position gg * nkb + 4q * R + (g * R + nn - gg)
  const uint32_t w_lane = (uint32_t)(g * R + (nn - gg));
  const int64_t nblk = N * nkb;
  // NF4 scale entries: block 64 at the unit's position, block 32 the pair at
  // 2p, 2p + 1, block 128 at (nn, 2q + g/2) in the row-group order over the
  // k/128 columns (nkb2); the second-level constant of flat block b is
  // step[b / 256]
  constexpr int BS = FI::block;
  const int64_t nkb2 = nkb / 2;
  const int64_t nsc = N * K / BS;                               // scale entries
  const uint32_t w_lane2 = (uint32_t)((g >> 1) * R + (nn - gg));
  const uint32_t b_lane = (uint32_t)(BS == 64 ? nn * nkb + g : (BS == 32 ? 2 * (nn * nkb + g) : nn * nkb2 + (g >> 1)));
  const auto step_rsrc = buf_rsrc(w.step, (uint32_t)(((nsc + kGroup - 1) / kGroup) * 4));
  // per-unit data at the storage position: CB code bytes, then the 8-bit
  // scale(s) (double quantization), the fp32 absmax(es), the uint4 scale and
  // zero-point, or the two Q8_0 scales
  auto load_w = [&](int q, GemvRaw<FMT>& u) {
    const int qc = min(q, nquads - 1);
    const int64_t ub = gg * nkb + (int64_t)4 * qc * R;
    const auto rc = buf_rsrc(w.codes + ub * CB, rsrc_bytes_u((nblk - ub) * CB));
#pragma unroll
    for (int j = 0; j < NC; ++j)
      u.c[j] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rc, w_lane * CB + 16 * j, 0, 0));
    // scale entry base (uniform) and this lane's entry offset
    const int64_t sb = BS == 64 ? ub : (BS == 32 ? 2 * ub : gg * nkb2 + (int64_t)2 * qc * R);
    const uint32_t so = BS == 64 ? w_lane : (BS == 32 ? 2 * w_lane : w_lane2);
    const uint32_t bq = BS == 64 ? 4u * qc : (BS == 32 ? 8u * qc : 2u * qc);   // flat block advance
    if constexpr (FI::nf4 && FI::dq) {
      const auto rq = buf_rsrc(w.qscale + sb, rsrc_bytes_u(nsc - sb));
      u.qbyte = BS == 32 ? (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(rq, so, 0, 0)
                         : (uint32_t)__builtin_amdgcn_raw_buffer_load_b8(rq, so, 0, 0);
      u.step = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                             step_rsrc, ((b_lane + bq) >> 8) * 4, 0, 0));
    } else if constexpr (FI::nf4) {
      const auto rs = buf_rsrc(w.step + sb, rsrc_bytes_u((nsc - sb) * 4));
      u.qbyte = 1u;
      u.step = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rs, so * 4, 0, 0));
      if constexpr (BS == 32)
        u.zp = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rs, so * 4 + 4, 0, 0));
    } else if constexpr (FMT == kFmtU4) {
      // two dword loads: a 64-bit buffer load whose halves are bit-cast to
      // float is shrunk to one dword by this compiler, both halves then
      // holding the scale
      const auto prs = buf_rsrc(w.step + 2 * ub, rsrc_bytes_u((nblk - ub) * 8));
      u.step = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(prs, w_lane * 8, 0, 0));
      u.zp = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(prs, w_lane * 8 + 4, 0, 0));
    } else {
      u.qbyte = __builtin_amdgcn_raw_buffer_load_b32(buf_rsrc(w.qscale + 4 * ub, rsrc_bytes_u((nblk - ub) * 4)),
                                                     w_lane * 4, 0, 0);
    }
  };

  f32x4_t acc[MT][2];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) acc[mt][0] = acc[mt][1] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  auto compute = [&](int q, int stage, const GemvRaw<FMT>& u) {
    // Blocks past the row end exist only in a ragged last quad (k % 256 !=
    // 0): their scale is forced to zero there.  Rows past N read the last
    // row (finite values) and their outputs are never stored.
    const bool ok = (nkb & 3) == 0 || q < nquads - 1 || 4 * q + g < nkb;
    const uint16_t* sx = stage_ptr(stage);
    u32x4_t af[MT][8];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const int row = (int)min((int64_t)(16 * mt + (lane & 15)), M - 1);
#pragma unroll
      for (int i = 0; i < 8; ++i)
        af[mt][i] = *reinterpret_cast<const u32x4_t*>(sx + row * 256 + ((8 * g + i) ^ (row & 15)) * 8);
    }
    __builtin_amdgcn_sched_barrier(0);   // the fragment reads go out before the decode
    if constexpr (FMT == kFmtQ8) {
      // elements 8i .. 8i+7 are bytes 8i .. 8i+7: words 2i, 2i+1 of the unit
      const float d0 = ok ? half_bits_to_float(u.qbyte & 0xFFFFu) : 0.f;
      const float d1 = ok ? half_bits_to_float(u.qbyte >> 16) : 0.f;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const u32x4_t& cw = u.c[i >> 1];
        const u32x4_t bf = decode_q8x8(cw[2 * (i & 1)], cw[2 * (i & 1) + 1], i < 4 ? d0 : d1);
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) acc[mt][i & 1] = mfma16x16x32<FI::f16>(af[mt][i], bf, acc[mt][i & 1]);
      }
    } else {
      float lvu[16];   // table levels: NF4 levels, or c - zp for uint4
      float scr;
      if constexpr (FMT == kFmtU4) {
        const int zp = (int)u.zp;   // c - zp formed as an integer: +0 at c == zp
#pragma unroll
        for (int i = 0; i < 16; ++i) lvu[i] = (float)(i - zp);
        scr = u.step;
      } else {
#pragma unroll
        for (int i = 0; i < 16; ++i) lvu[i] = lv[i];
        scr = (float)(u.qbyte & 0xFFu) * u.step;
      }
      const Lut t = make_lut<FI::f16>(lvu, ok ? scr : 0.f);
      if constexpr (BS == 32) {
        // words 4-7 are the second 32-weight block: its own scale and table
        const float scr1 = FI::dq ? (float)(u.qbyte >> 8) * u.step : u.zp;
        const Lut t1 = make_lut(lvu, ok ? scr1 : 0.f);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const u32x4_t bf = decode8(i < 4 ? t : t1, u.c[i >> 2][i & 3]);
#pragma unroll
          for (int mt = 0; mt < MT; ++mt) acc[mt][i & 1] = mfma16x16x32<FI::f16>(af[mt][i], bf, acc[mt][i & 1]);
        }
      } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const u32x4_t bf = decode8(t, u.c[i >> 2][i & 3]);
#pragma unroll
          for (int mt = 0; mt < MT; ++mt) acc[mt][i & 1] = mfma16x16x32<FI::f16>(af[mt][i], bf, acc[mt][i & 1]);
        }
      }
    }
  };

  // wait for this wave's loads of quad q (everything but the loads issued in
  // the following iteration: NC code loads, one or two parameter loads and
  // XPW chunk loads), then barrier.  The uint4 pair and the block-32 absmax
  // pair count as one load: the backend may merge their two dword loads, and
  // where it does not, the count only waits for one load of the next quad as
  // well.
  auto wait_q = [&]() {
    QL_VMCNT(NC + (FI::dq ? 2 : 1) + XPW);
    QL_LGKMCNT0();
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  };

  if (q0 < q1) {
    GemvRaw<FMT> rw[3];
    load_w(q0, rw[0]);
    load_x(q0, 0);
    load_w(q0 + 1, rw[1]);
    load_x(q0 + 1, 1);
    auto step = [&](int q, auto PHc) {
      constexpr int PH = decltype(PHc)::value;
      wait_q();
      __builtin_amdgcn_sched_barrier(0);
      load_w(q + 2, rw[(PH + 2) % 3]);
      load_x(q + 2, (PH + 2) % 3);
      __builtin_amdgcn_sched_barrier(0);
      compute(q, PH, rw[PH]);
      __builtin_amdgcn_sched_barrier(0);
    };
    using P0 = std::integral_constant<int, 0>;
    using P1 = std::integral_constant<int, 1>;
    using P2 = std::integral_constant<int, 2>;
    int q = q0;
    for (; q + 2 < q1; q += 3) {
      step(q, P0{});
      step(q + 1, P1{});
      step(q + 2, P2{});
    }
    if (q < q1) step(q, P0{});
    if (q + 1 < q1) step(q + 1, P1{});
  }

  const bool lvec = J.lora.r % 8 == 0 && (reinterpret_cast<uintptr_t>(J.lora.R) & 15) == 0 &&
                    (reinterpret_cast<uintptr_t>(J.lora.L) & 15) == 0 && J.lora.rs_j == 1 &&
                    J.lora.rs_c == J.lora.r;
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const f32x4_t v = acc[mt][0] + acc[mt][1];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int64_t m = mt * 16 + g * 4 + e;
      if (m < M && nok) {
        float y = v[e];
        if (ksplit > 1) {
          gptr_w(J.part)[((int64_t)split * M + m) * N + n] = y;
        } else {
          if (J.lora.r > 0) y += J.lora.scaling * lora_dot_v<FI::f16>(J.lora, m, n, lvec);
          store_out<FI::f16>(J.Y, J.y16, m * N + n, y);
        }
      }
    }
  }
}

// Streaming input gradient, small M: dX[m][k] = sum_n dY[m][n] deq(W)[n][k]
// (www.cf-1.com/news/5705389 §2.1: the gradient passes through the frozen
// quantized matrix).  A workgroup of 4 waves owns one 64-wide k-block kb and
// one split of the rows; per iteration wave w decodes rows [nb + 64 w, +64)
// at kb, one 64-weight unit per lane (lane = row), into its own LDS tile
// [64 n][72], and reads it back with ds_read_b64_tr_b16, which hands each
// lane 4 consecutive rows of one column: the MFMA 16x16x32 operand
// W^T[16 k][32 n].  The contraction over n runs inside the wave (no barrier
// until the end); the four waves' sums are added through LDS once, and the
// splits over n through k_reduce.  Per lane and iteration the loads are the
// unit's code bytes, its scale entry and the dY fragments of its 64 rows
// (dY[m][nb .. +64), 16-byte pieces, from L2): a three-deep ring keeps the
// loads of two iterations in flight.
constexpr int GDX_LDW = 72;   // LDS pitch of a wave tile (16-bit elements)

template <int FMT, int MT>
struct GdxRaw {
  u32x4_t c[FMT == kFmtQ8 ? 4 : 2];
  uint32_t qbyte;
  float step, zp;
  u32x4_t y[MT][2];   // dY fragments: row tile mt, row half h of the 64
};

template <int MT, int FMT>
__global__ __launch_bounds__(256) void k_gemv_dx(const uint16_t* __restrict__ dY, Nf4View w,
                                                 const float* __restrict__ codebook, int64_t M,
                                                 LoraTerm lora, void* __restrict__ out, int out16,
                                                 float* __restrict__ part, int iters) {
  __shared__ __attribute__((aligned(16))) uint16_t sT[4 * 64 * GDX_LDW];
  using FI = FmtInfo<FMT>;
  constexpr int CB = FI::code_bytes, NC = CB / 16, BS = FI::block;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t N = w.n, K = w.k, nkb = K / kBlock, nkb2 = nkb / 2;
  const int64_t kb = blockIdx.x;
  const int split = blockIdx.y, nsplit = gridDim.y;
  const int64_t n_begin = (int64_t)split * iters * 256;          // first row of the split
  const int i16 = lane & 15, G16 = lane >> 4;
  uint16_t* const sw = sT + wave * 64 * GDX_LDW;

  float lv[16];   // the same in every lane: scalar registers
#pragma unroll
  for (int i = 0; i < 16; ++i)
    lv[i] = FI::nf4 ? __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(
                                                   __builtin_bit_cast(int, gptr(codebook)[i])))
                    : 0.f;

  const int64_t nsc = N * K / BS;
  const auto step_rsrc = buf_rsrc(w.step, (uint32_t)(((nsc + kGroup - 1) / kGroup) * 4));
  const bool yvec = (N & 7) == 0;   // 16-byte dY pieces inside the rows
  const auto y_rsrc = buf_rsrc(dY, (uint32_t)(M * N * 2));
  // Unit (n, kb) sits at storage position gg * nkb + kb * R + (n - gg), gg =
  // n & ~15, R = min(16, N - gg); positions are taken relative to the first
  // row nb of the wave's 64 (a multiple of 16).  Rows past N get an offset
  // past any resource: the hardware returns zeros, hence a zero scale.
  constexpr uint32_t kOut = 0x80000000u;
  auto load = [&](int it, GdxRaw<FMT, MT>& u) {
    const int64_t nb = n_begin + (int64_t)min(it, iters - 1) * 256 + 64 * wave;
    const int64_t n = nb + lane, gg = n & ~int64_t(15);
    const bool ok = n < N;
    const int64_t R = min(int64_t(16), N - gg);
    const uint32_t rel = (uint32_t)((gg - nb) * nkb + kb * R + (n - gg));
    const int64_t base = nb * nkb;   // position of (nb, 0)
    const auto rc = buf_rsrc(w.codes + base * CB);
    const uint32_t co = ok ? rel * CB : kOut;
#pragma unroll
    for (int j = 0; j < NC; ++j)
      u.c[j] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rc, co + 16 * j, 0, 0));
    if constexpr (FI::nf4) {
      // scale entry: block 64 at the position, block 32 the pair at 2p, 2p+1,
      // block 128 at (n, kb / 2) in the row-group order over k/128 columns
      const int64_t sbase = BS == 64 ? base : (BS == 32 ? 2 * base : nb * nkb2);
      const uint32_t srel = BS == 64 ? rel : (BS == 32 ? 2 * rel
                                              : (uint32_t)((gg - nb) * nkb2 + (kb >> 1) * R + (n - gg)));
      if constexpr (FI::dq) {
        const auto rq = buf_rsrc(w.qscale + sbase);
        u.qbyte = BS == 32 ? (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(rq, ok ? srel : kOut, 0, 0)
                           : (uint32_t)__builtin_amdgcn_raw_buffer_load_b8(rq, ok ? srel : kOut, 0, 0);
        // flat block index of the unit's (first) block, for its group constant
        const int64_t b = BS == 64 ? n * nkb + kb : (BS == 32 ? 2 * (n * nkb + kb) : n * nkb2 + (kb >> 1));
        u.step = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                               step_rsrc, ok ? (uint32_t)(b >> 8) * 4 : kOut, 0, 0));
      } else {
        const auto rs = buf_rsrc(w.step + sbase);
        u.qbyte = 1u;
        u.step = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rs, ok ? srel * 4 : kOut, 0, 0));
        if constexpr (BS == 32)
          u.zp = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rs, ok ? srel * 4 + 4 : kOut, 0, 0));
      }
    } else if constexpr (FMT == kFmtU4) {
      const auto prs = buf_rsrc(w.step + 2 * base);
      u.step = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(prs, ok ? rel * 8 : kOut, 0, 0));
      u.zp = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(prs, ok ? rel * 8 + 4 : kOut, 0, 0));
    } else {
      u.qbyte = __builtin_amdgcn_raw_buffer_load_b32(buf_rsrc(w.qscale + 4 * base), ok ? rel * 4 : kOut, 0, 0);
    }
    // dY fragments: lane (i16, G16) holds dY[16 mt + i16][nb + 32 h + 8 G16 .. +7]
    // (rows past M re-read row M-1, whose products are dropped; columns past
    // N are zeros)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const int64_t m = min((int64_t)(16 * mt + i16), M - 1);
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int64_t c = nb + 32 * h + 8 * G16;
        if (yvec) {
          u.y[mt][h] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(
                                                       y_rsrc, c < N ? (uint32_t)((m * N + c) * 2) : kOut, 0, 0));
        } else {
          u.y[mt][h] = load_act8(dY + m * N, c, N, false);
        }
      }
    }
  };
  // vector-memory loads per iteration (the uint4 pair and the block-32
  // absmax pair counted once: the backend may merge them; a count below the
  // real one only waits longer)
  constexpr int kLoads = NC + (FI::dq ? 2 : 1) + 2 * MT;

  f32x4_t acc[4][MT];
#pragma unroll
  for (int kt = 0; kt < 4; ++kt)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[kt][mt] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  auto compute = [&](const GdxRaw<FMT, MT>& u) {
    // decode the lane's unit into row `lane` of the wave tile: word i holds
    // elements 8i .. 8i+7
    auto put = [&](int i, const u32x4_t& v) {
      *reinterpret_cast<u32x4_t*>(sw + lane * GDX_LDW + 8 * i) = v;
    };
    if constexpr (FMT == kFmtQ8) {
      const float d0 = half_bits_to_float(u.qbyte & 0xFFFFu), d1 = half_bits_to_float(u.qbyte >> 16);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const u32x4_t& cw = u.c[i >> 1];
        put(i, decode_q8x8(cw[2 * (i & 1)], cw[2 * (i & 1) + 1], i < 4 ? d0 : d1));
      }
    } else {
      float lvu[16];
      float scr;
      if constexpr (FMT == kFmtU4) {
        const int zp = (int)u.zp;
#pragma unroll
        for (int i = 0; i < 16; ++i) lvu[i] = (float)(i - zp);
        scr = u.step;
      } else {
#pragma unroll
        for (int i = 0; i < 16; ++i) lvu[i] = lv[i];
        scr = (float)(u.qbyte & 0xFFu) * u.step;
      }
      const Lut t = make_lut<FI::f16>(lvu, scr);
      if constexpr (BS == 32) {
        const float scr1 = FI::dq ? (float)(u.qbyte >> 8) * u.step : u.zp;
        const Lut t1 = make_lut(lvu, scr1);
#pragma unroll
        for (int i = 0; i < 8; ++i) put(i, decode8(i < 4 ? t : t1, u.c[i >> 2][i & 3]));
      } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) put(i, decode8(t, u.c[i >> 2][i & 3]));
      }
    }
    // contraction over the 64 rows: row half h, k tile kt.  (The LDS
    // operations of a wave execute in order: these reads see the writes
    // above, and the next iteration's writes follow these reads.)
#pragma unroll
    for (int h = 0; h < 2; ++h) {
#pragma unroll
      for (int kt = 0; kt < 4; ++kt) {
        const uint16_t* p = sw + (32 * h + 8 * G16 + (i16 >> 2)) * GDX_LDW + 16 * kt + 4 * (i16 & 3);
        const u32x2_t lo = ds_tr16(p), hi = ds_tr16(p + 4 * GDX_LDW);
        const u32x4_t a = u32x4_t{lo[0], lo[1], hi[0], hi[1]};
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) acc[kt][mt] = mfma16x16x32<FI::f16>(a, u.y[mt][h], acc[kt][mt]);
      }
    }
  };

  {
    GdxRaw<FMT, MT> rw[3];
    load(0, rw[0]);
    load(1, rw[1]);
    auto step = [&](int it, auto PHc) {
      constexpr int PH = decltype(PHc)::value;
      load(it + 2, rw[(PH + 2) % 3]);
      QL_VMCNT(2 * kLoads);   // iteration it's loads have landed
      compute(rw[PH]);
    };
    using P0 = std::integral_constant<int, 0>;
    using P1 = std::integral_constant<int, 1>;
    using P2 = std::integral_constant<int, 2>;
    int it = 0;
    for (; it + 2 < iters; it += 3) {
      step(it, P0{});
      step(it + 1, P1{});
      step(it + 2, P2{});
    }
    if (it < iters) step(it, P0{});
    if (it + 1 < iters) step(it + 1, P1{});
  }

  // the four waves' sums through LDS (the tiles are free once every wave is
  // past its last reads): red[wave][kt][mt][lane][e]
  __syncthreads();
  float* red = reinterpret_cast<float*>(sT);
#pragma unroll
  for (int kt = 0; kt < 4; ++kt)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
      *reinterpret_cast<f32x4_t*>(red + (((wave * 4 + kt) * MT + mt) * 64 + lane) * 4) = acc[kt][mt];
  __syncthreads();
  // thread t: outputs idx = t + 256 j over (m, k) = (idx / 64, idx % 64)
#pragma unroll
  for (int j = 0; j < 4 * MT; ++j) {
    const int idx = tid + 256 * j;
    const int m = idx >> 6, kl = idx & 63;
    const int kt = kl >> 4, e = kl & 3, ln = 16 * ((kl & 15) >> 2) + (m & 15), mt = m >> 4;
    float v = 0.f;
#pragma unroll
    for (int wv = 0; wv < 4; ++wv) v += red[(((wv * 4 + kt) * MT + mt) * 64 + ln) * 4 + e];
    const int64_t k = kb * kBlock + kl;
    if (m < M) {
      if (nsplit > 1) {
        part[((int64_t)split * M + m) * K + k] = v;
      } else {
        if (lora.r > 0) v += lora.scaling * lora_dot<FI::f16>(lora, m, k);
        store_out<FI::f16>(out, out16, m * K + k, v);
      }
    }
  }
}

template <bool F16>
__global__ __launch_bounds__(256) void k_reduce(const float* __restrict__ part, int nsplit, int64_t M,
                                                int64_t C, LoraTerm lora, void* __restrict__ out,
                                                int out16) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= M * C) return;
  float v = 0.f;
  for (int s = 0; s < nsplit; ++s) v += part[(int64_t)s * M * C + idx];
  if (lora.r > 0) v += lora.scaling * lora_dot<F16>(lora, idx / C, idx % C);
  store_out<F16>(out, out16, idx, v);
}

template <int MT, int XPW, bool GROUPED>
static void gemv_launch(int fmt, dim3 grid, hipStream_t s, const GemvJob& job1, const GemvJob* jobs,
                        int njobs, const float* codebook, int ksplit, int per) {
#define QL_GEMV(F)                                                                              \
  hipLaunchKernelGGL((k_gemv_fwd<MT, XPW, GROUPED, F>), grid, dim3(256), 0, s, job1, jobs, njobs, \
                     codebook, ksplit, per)
  switch (fmt) {
    case kFmtNf4Dq: QL_GEMV(kFmtNf4Dq); break;
    case kFmtNf4: QL_GEMV(kFmtNf4); break;
    case kFmtU4: QL_GEMV(kFmtU4); break;
    case kFmtQ8: QL_GEMV(kFmtQ8); break;
    case kFmtNf4Dq32: QL_GEMV(kFmtNf4Dq32); break;
    case kFmtNf4_32: QL_GEMV(kFmtNf4_32); break;
    case kFmtNf4Dq128: QL_GEMV(kFmtNf4Dq128); break;
    case kFmtNf4DqF16: QL_GEMV(kFmtNf4DqF16); break;
    default: QL_GEMV(kFmtNf4_128); break;
  }
#undef QL_GEMV
}

template <bool GROUPED>
static void gemv_launch_m(int64_t M, int fmt, dim3 grid, hipStream_t s, const GemvJob& job1,
                          const GemvJob* jobs, int njobs, const float* codebook, int ksplit, int per) {
  // M <= 32, checked by the caller
  if (M <= 8) gemv_launch<1, 1, GROUPED>(fmt, grid, s, job1, jobs, njobs, codebook, ksplit, per);
  else if (M <= 16) gemv_launch<1, 2, GROUPED>(fmt, grid, s, job1, jobs, njobs, codebook, ksplit, per);
  else gemv_launch<2, 4, GROUPED>(fmt, grid, s, job1, jobs, njobs, codebook, ksplit, per);
}

hipError_t launch_gemv_fwd(const Nf4View& w, const float* codebook, const uint16_t* X, int64_t M,
                           const LoraTerm& lora, void* Y, bool y16, float* part, int ksplit,
                           hipStream_t s) {
  const int64_t nquads = (w.k / kBlock + 3) / 4;
  const int per = (int)((nquads + ksplit - 1) / ksplit);
  const GemvJob job{X, w, lora, Y, part, M, (int)y16, 0};
  const dim3 grid((unsigned)((w.n + 63) / 64), (unsigned)ksplit);
  gemv_launch_m<false>(M, w.fmt, grid, s, job, nullptr, 0, codebook, ksplit, per);
  return hipGetLastError();
}

hipError_t launch_gemv_grouped(const GemvJob* jobs, int njobs, int64_t row_groups, int64_t M,
                               const float* codebook, int64_t max_quads, int fmt, hipStream_t s) {
  const dim3 grid((unsigned)row_groups, 1);
  const GemvJob none{};
  gemv_launch_m<true>(M, fmt, grid, s, none, jobs, njobs, codebook, 1, (int)max_quads);
  return hipGetLastError();
}

template <int MT>
static void gemv_dx_launch(int fmt, dim3 grid, hipStream_t s, const uint16_t* dY, const Nf4View& w,
                           const float* codebook, int64_t M, const LoraTerm& lora, void* out,
                           int out16, float* part, int iters) {
#define QL_GDX(F)                                                                             \
  hipLaunchKernelGGL((k_gemv_dx<MT, F>), grid, dim3(256), 0, s, dY, w, codebook, M, lora, out, \
                     out16, part, iters)
  switch (fmt) {
    case kFmtNf4Dq: QL_GDX(kFmtNf4Dq); break;
    case kFmtNf4: QL_GDX(kFmtNf4); break;
    case kFmtU4: QL_GDX(kFmtU4); break;
    case kFmtQ8: QL_GDX(kFmtQ8); break;
    case kFmtNf4Dq32: QL_GDX(kFmtNf4Dq32); break;
    case kFmtNf4_32: QL_GDX(kFmtNf4_32); break;
    case kFmtNf4Dq128: QL_GDX(kFmtNf4Dq128); break;
    case kFmtNf4DqF16: QL_GDX(kFmtNf4DqF16); break;
    default: QL_GDX(kFmtNf4_128); break;
  }
#undef QL_GDX
}

hipError_t launch_gemv_dx(const Nf4View& w, const float* codebook, const uint16_t* dY, int64_t M,
                          const LoraTerm& lora, void* dX, bool dx16, float* part, int nsplit,
                          hipStream_t s) {
  // M <= 32 and nsplit = gemv_dx_splits(M, n, k), checked by the caller
  const int64_t niter = (w.n + 255) / 256;
  const int iters = (int)((niter + nsplit - 1) / nsplit);
  const dim3 grid((unsigned)(w.k / kBlock), (unsigned)nsplit);
  if (M <= 16)
    gemv_dx_launch<1>(w.fmt, grid, s, dY, w, codebook, M, lora, dX, (int)dx16, part, iters);
  else
    gemv_dx_launch<2>(w.fmt, grid, s, dY, w, codebook, M, lora, dX, (int)dx16, part, iters);
  return hipGetLastError();
}

hipError_t launch_reduce(const float* part, int nsplit, int64_t M, int64_t C, const LoraTerm& lora,
                         void* out, bool out16, bool f16, hipStream_t s) {
  const int64_t total = M * C;
  const dim3 grid((unsigned)((total + 255) / 256));
  if (f16)
    hipLaunchKernelGGL(k_reduce<true>, grid, dim3(256), 0, s, part, nsplit, M, C, lora, out, (int)out16);
  else
    hipLaunchKernelGGL(k_reduce<false>, grid, dim3(256), 0, s, part, nsplit, M, C, lora, out, (int)out16);
  return hipGetLastError();
}

}  // namespace ql
