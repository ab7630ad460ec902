// Fused-dequant MFMA GEMMs of the quantized linear (large-M regime):
//   forward   Y  = X  deq(W)^T (+ LoRA term)    contraction over k
//   backward  dX = dY deq(W)   (+ LoRA term)    contraction over n
// The packed weight (NF4, asymmetric uint4 or Q8_0) is decoded to the 16-bit
// compute type (bf16; fp16 for kFmtNf4DqF16, news.rkmt.cn/news/4821 §3.3) inside
// the kernel and lives only in registers and LDS (www.cf-1.com/news/5705389
// §2.2, §4.2: block dequant in the GEMM's outer loop, results kept in
// registers / shared memory;
// www.lqnn.cn/news/228537 §3.3: dequantize to 16 bits for the product, then
// discard).
//
// gfx950 design:
//  * 256 x 128 output tile per workgroup, 8 waves in two groups of four (one
//    wave of each group per SIMD): wave (g, w) accumulates rows 64w .. +63 x
//    all 128 columns over K-slices 2g, 2g+1 of every step (MFMA 32x32x16,
//    bf16 or fp16 operands, fp32 accumulators); the partner waves swap halves
//    at the end, each finishing a 64 x 64 tile.
//  * The activation operand (X or dY) goes global -> LDS with the gfx950
//    global_load_lds b128 DMA (no registers, each wave load covers 8 whole
//    128-byte row pieces) into a 3-stage ring, two K-steps ahead.  16-byte
//    chunks are XOR-swizzled by row so the MFMA fragment reads are free of
//    bank conflicts.
//  * The weight tile of each K-step (128 x 64 weights = 128 storage units) is
//    decoded by all 512 threads into a double-buffered LDS stage: the four
//    lanes of a DPP quad share a unit and decode 16 weights each; for the
//    4-bit formats they build its 16-entry table together (broadcast with
//    quad_perm), Q8_0 bytes are scaled directly.  Ping-pong: while one
//    group runs the MFMAs of step s the other reads its fragments and decodes
//    its half of step s+1, a barrier between phases; the decode is amortized
//    over 256 output rows.
//  * Forward reads B fragments with ds_read_b128 from the [n][k] stage; the
//    backward contracts over n and reads them with the transposing
//    ds_read_b64_tr_b16 from a [n][k] stage.
//  * Tiles are renumbered so that the workgroups sharing one activation row
//    tile run on the same XCD (workgroup ids are dealt to the 8 XCDs round
//    robin), keeping that tile in the XCD's L2.
#include "common.h"
#include "kernels.h"

#include <type_traits>

namespace ql {

typedef float f32x16_t __attribute__((ext_vector_type(16)));

// D[32x32] += A[32x16] B[16x32]; lane l holds A[l%32][8(l/32)..+7],
// B[8(l/32)..+7][l%32], D[8(i/4) + 4(l/32) + i%4][l%32] for i = 0..15.
template <bool F16>
QL_DEV f32x16_t mfma32(const u32x4_t a, const u32x4_t b, f32x16_t c) {
  if constexpr (F16)
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8_t, a),
                                                  __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

constexpr int GBM = 256, GBN = 128, GBK = 64;

template <bool DX>
struct Geo {
  // LDS stage of one K-step of the weight, bf16, [rows][ld].  Forward:
  // 144-byte rows put the 16 rows of a ds_read_b128 quarter-wave on 16
  // different bank groups.  Backward: 320-byte rows (16 banks apart) keep the
  // 4-row x 32-byte footprints of the two 16-lane groups of a tr16 half-wave
  // read on disjoint banks.
  static constexpr int rows = DX ? GBK : GBN;    // n (dx: contraction) or n (fwd: output)
  static constexpr int cols = DX ? GBN : GBK;    // k
  static constexpr int ld = DX ? cols + 32 : cols + 8;
  static constexpr int stage = rows * ld;
};

QL_DEV u32x4_t load_act8(const uint16_t* row, int64_t c, int64_t C, bool vec) {
  if (vec) return *reinterpret_cast<const u32x4_t*>(row + c);
  uint32_t h[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) h[e] = (c + e < C) ? row[c + e] : 0u;
  return u32x4_t{h[0] | h[1] << 16, h[2] | h[3] << 16, h[4] | h[5] << 16, h[6] | h[7] << 16};
}

QL_DEV u32x2_t ds_tr16(const uint16_t* p) {
  const s16x4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) s16x4_t*)(p));
  return __builtin_bit_cast(u32x2_t, v);
}

// Logical tile of this workgroup: consecutive logical tiles (row-tile major)
// go to the same XCD.
QL_DEV int64_t logical_tile(int64_t id, int64_t total) {
  const int64_t xcd = id & 7, slot = id >> 3;
  const int64_t base = total >> 3, rem = total & 7;
  return xcd * base + (xcd < rem ? xcd : rem) + slot;
}

constexpr int NA = 3;                 // activation stages in the ring
constexpr int A_STAGE = GBM * GBK;     // bf16 elements per activation stage (32 KiB)


// Workgroup barrier for the K loop.  __syncthreads() would add a release
// fence, and with LDS DMA in flight that fence waits for every outstanding
// vector load (vmcnt 0), draining the prefetch pipeline at each step.  Here
// the caller states the vmcnt it needs; this waits for the wave's own LDS
// traffic and the empty asm statements keep the compiler from moving memory
// accesses across the barrier.
QL_DEV void k_barrier() {
  QL_LGKMCNT0();
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Workgroup barrier that waits for nothing: the caller has already waited for
// what it needs.
QL_DEV void k_barrier_issue() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Physical 16-byte chunk of logical chunk c in activation row r of a stage.
QL_DEV int a_chunk(int r, int c) { return c ^ ((r >> 1) & 7); }

template <bool DX, bool VEC, int FMT>
__global__ __launch_bounds__(512, 1) void k_gemm(const uint16_t* __restrict__ act, Nf4View w,
                                                 const float* __restrict__ codebook, int64_t M,
                                                 LoraTerm lora, void* __restrict__ out, int out16,
                                                 float* __restrict__ part, int ksplit,
                                                 int steps_per_split, int64_t mtiles, int64_t otiles) {
  using G = Geo<DX>;
  extern __shared__ __attribute__((aligned(16))) uint16_t sA[];   // [NA][GBM rows][GBK], swizzled
  __shared__ __attribute__((aligned(16))) uint16_t sW[2 * G::stage];   // decoded weight stages
  __shared__ float s_lv[16];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  // wave w: rows [64 (w % 4), +64) of the tile, all 128 columns, the half
  // kk in {2g, 2g+1} of every K-step, g = w / 4 (its group)
  const int wm = wave & 3, grp = wave >> 2;
  const int lr = lane & 31, lg = lane >> 5;
  const int64_t N = w.n, K = w.k, nkb = K / kBlock;
  const int64_t C = DX ? N : K;       // contraction length
  const int64_t O = DX ? K : N;       // output columns

  const int64_t total = mtiles * otiles * ksplit;
  const int64_t L = logical_tile(blockIdx.x, total);
  const int64_t mt_ = L / (otiles * ksplit);
  const int64_t rem_ = L - mt_ * otiles * ksplit;
  const int64_t ot_ = rem_ / ksplit;
  const int split = (int)(rem_ - ot_ * ksplit);
  const int64_t m0 = mt_ * GBM, o0 = ot_ * GBN;

  const int nsteps = (int)((C + GBK - 1) / GBK);
  const int s_begin = split * steps_per_split;
  const int s_end = min(nsteps, s_begin + steps_per_split);

  if (FmtInfo<FMT>::nf4 && tid < 16) s_lv[tid] = codebook[tid];

  // Decode role: group g decodes blocks [64g, 64g+64) of each step's 128; a
  // quad of lanes shares one block, lane q = tid & 3 decodes its elements
  // [16q, 16q+16).
  const int q = tid & 3;
  const int blk = 64 * grp + ((tid & 255) >> 2);
  const int wr = DX ? (blk >> 1) : blk;                     // stage row
  const int wcb = DX ? (blk & 1) : 0;                       // block within the stage row (dx)

  // Activation tile of step st into ring stage `stage`: wave w fills rows
  // [32w, 32w+32) with 4 DMA loads of 8 rows; lane l lands at byte 16l of its
  // load's 1 KiB, i.e. row l/8, physical chunk l%8.  Rows past M are clamped
  // to row M-1 (their products are discarded).  With 16-byte rows (VEC) the
  // loads are buffer loads from a per-step base held in scalar registers and
  // a fixed per-lane offset, so they cost no vector ALU work; a ragged last
  // step clamps each piece into its row instead (columns past the
  // contraction meet zero weights).  Without 16-byte rows the loads go
  // through registers with zero fill and complete before the stores.
  uint32_t a_vo[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int rl = wave * 32 + i * 8 + (lane >> 3);
    a_vo[i] = (uint32_t)(((min(m0 + rl, M - 1) - m0) * C + a_chunk(rl, lane & 7) * 8) * 2);
  }
  const uint16_t* a_tile = act + m0 * C;
  // steps whose 64 columns all lie inside the contraction (the forward's
  // contraction is a whole number of 64-blocks)
  const int full_steps = (int)(C / GBK);
  auto fill_a_one = [&](int64_t c0, uint16_t* base, int i, auto FULLc) {
    uint16_t* dst = base + (wave * 32 + i * 8) * GBK;
    const int rl = wave * 32 + i * 8 + (lane >> 3);
    const int lc = a_chunk(rl, lane & 7);
    if (VEC) {
      if (decltype(FULLc)::value) {
        __builtin_amdgcn_raw_ptr_buffer_load_lds(buf_rsrc(a_tile + c0), (QL_LDS void*)dst, 16,
                                                 a_vo[i], 0, 0, 0);
      } else {
        const int64_t row = min(m0 + rl, M - 1);
        __builtin_amdgcn_global_load_lds(act + row * C + min(c0 + lc * 8, C - 8), (QL_LDS void*)dst,
                                         16, 0, 0);
      }
    } else {
      const int64_t row = min(m0 + rl, M - 1);
      const int64_t c = c0 + lc * 8;
      const u32x4_t v = c < C ? load_act8(act + row * C, c, C, false) : u32x4_t{0u, 0u, 0u, 0u};
      *reinterpret_cast<u32x4_t*>(dst + lane * 8) = v;
    }
  };
  auto fill_a = [&](int st, int stage) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (!DX || st < full_steps)
        fill_a_one((int64_t)st * GBK, sA + stage * A_STAGE, i, std::true_type{});
      else
        fill_a_one((int64_t)st * GBK, sA + stage * A_STAGE, i, std::false_type{});
    }
  };

  struct WRaw {
    u32x4_t codes;    // this lane's 16 weights: words 0-1 (4-bit formats) or 0-3 (Q8_0)
    uint32_t qbyte;   // NF4 with double quantization: the 8-bit scale; Q8_0: the two fp16 scales
    float step;       // NF4: the group's fp32 constant, or the block absmax; uint4: the scale
    float zp;         // uint4: the zero-point
  };
  // This lane's unit at step st.  Storage position (rows in groups of 16,
  // k-block-major inside a group): forward fp0 + st * fR (fixed row; fR = 16
  // except in a partial last group), backward st * 64 * nkb plus a fixed part
  // whenever all 64 rows of the step are present.  Positions are taken
  // relative to a per-step base in scalar registers; units outside the
  // weight get an offset past the buffer end, so the hardware returns zeros
  // (scale 0, hence decoded zeros).  Per-unit data at the storage position:
  // CB code bytes and PB parameter bytes (the 8-bit scale with double
  // quantization, whose fp32 constant of flat block b sits at step[b / 256];
  // the fp32 absmax; the uint4 scale and zero-point; the two Q8_0 scales).
  using FI = FmtInfo<FMT>;
  constexpr uint32_t CB = FI::code_bytes, PB = FI::param_bytes;
  constexpr uint32_t kOut = 0x80000000u;
  // NF4 scale entries: block 64 one per unit (its position), block 32 two
  // per unit (2p + half), block 128 one per unit pair, in the row-group order
  // over the k/128 block columns (nkb2); the second-level constant of flat
  // block b is step[b / 256].
  constexpr int BS = FI::block;
  const int64_t nkb2 = nkb / 2;
  const uint32_t hq = (uint32_t)(q >> 1);   // block 32: the lane's half of its unit
  const int64_t kb_dx = o0 / kBlock + wcb;
  const int64_t fg0 = (o0 + wr) & ~int64_t(15);
  const bool f_ok = (o0 + wr) < N;
  const uint32_t fR = f_ok ? (uint32_t)min(int64_t(16), N - fg0) : 16u;
  const uint32_t f_prel = (uint32_t)((fg0 - o0) * nkb + (o0 + wr - fg0));   // fp0 - o0 * nkb
  const uint32_t f_prel2 = (uint32_t)((fg0 - o0) * nkb2 + (o0 + wr - fg0));
  const bool d_kok = kb_dx < nkb;
  const uint32_t d_prel = (uint32_t)((wr & ~15) * nkb + kb_dx * 16 + (wr & 15));
  const uint32_t d_prel2 = (uint32_t)((wr & ~15) * nkb2 + (kb_dx >> 1) * 16 + (wr & 15));
  auto sent = [&](uint32_t prel, uint32_t prel2) -> uint32_t {   // scale entry of the lane's unit
    return BS == 64 ? prel : (BS == 32 ? 2 * prel + hq : prel2);
  };
  const uint32_t c_vo0 =
      DX ? (d_kok ? d_prel * CB + q * (CB / 4) : kOut) : (f_ok ? f_prel * CB + q * (CB / 4) : kOut);
  const uint32_t p_vo0 =
      DX ? (d_kok ? sent(d_prel, d_prel2) * PB : kOut) : (f_ok ? sent(f_prel, f_prel2) * PB : kOut);
  const uint32_t b_lane = (uint32_t)(BS == 64    ? (DX ? wr * nkb + kb_dx : (o0 + wr) * nkb)
                                     : BS == 32 ? 2 * (DX ? wr * nkb + kb_dx : (o0 + wr) * nkb) + hq
                                                : (DX ? wr * nkb2 + (kb_dx >> 1) : (o0 + wr) * nkb2));
  const auto step_rsrc = buf_rsrc(w.step, (uint32_t)(((N * K / BS + kGroup - 1) / kGroup) * 4));
  auto load_w = [&](int st, WRaw& r) {
    uint32_t cvo, pvo, bidx;
    int64_t pbase;   // storage position of the per-step (backward) or per-tile (forward) base
    int64_t sbase;   // its scale entry
    if (DX) {
      const int64_t n0 = (int64_t)st * GBK;
      pbase = n0 * nkb;
      sbase = BS == 64 ? pbase : (BS == 32 ? 2 * pbase : n0 * nkb2);
      bidx = b_lane + (uint32_t)sbase;
      if (st < full_steps) {
        cvo = c_vo0;
        pvo = p_vo0;
      } else {   // ragged last step: partial group and rows past N
        const int64_t g0 = (wr & ~15), R = min(int64_t(16), N - n0 - g0);
        const bool ok = d_kok && n0 + wr < N;
        const uint32_t prel = (uint32_t)(g0 * nkb + kb_dx * R + (wr & 15));
        const uint32_t prel2 = (uint32_t)(g0 * nkb2 + (kb_dx >> 1) * R + (wr & 15));
        cvo = ok ? prel * CB + q * (CB / 4) : kOut;
        pvo = ok ? sent(prel, prel2) * PB : kOut;
      }
    } else {
      pbase = o0 * nkb;
      sbase = BS == 64 ? pbase : (BS == 32 ? 2 * pbase : o0 * nkb2);
      const uint32_t sinc = BS == 64 ? (uint32_t)st : (BS == 32 ? 2u * st : (uint32_t)st >> 1);
      cvo = c_vo0 + (uint32_t)st * fR * CB;
      pvo = p_vo0 + sinc * fR * PB;
      bidx = b_lane + sinc;
    }
    const auto crs = buf_rsrc(w.codes + pbase * CB);
    if constexpr (FMT == kFmtQ8) {
      r.codes = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(crs, cvo, 0, 0));
      r.qbyte = __builtin_amdgcn_raw_buffer_load_b32(buf_rsrc(w.qscale + pbase * 4), pvo, 0, 0);
    } else {
      const u32x2_t c = __builtin_bit_cast(u32x2_t, __builtin_amdgcn_raw_buffer_load_b64(crs, cvo, 0, 0));
      r.codes = u32x4_t{c[0], c[1], 0u, 0u};
      if constexpr (FI::nf4 && FI::dq) {
        r.qbyte = __builtin_amdgcn_raw_buffer_load_b8(buf_rsrc(w.qscale + sbase), pvo, 0, 0);
        r.step = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(step_rsrc, (bidx >> 8) * 4, 0, 0));
      } else if constexpr (FI::nf4) {
        r.qbyte = 1u;   // scale = 1 * absmax, exact
        r.step = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(buf_rsrc(w.step + sbase), pvo, 0, 0));
      } else {
        // two dword loads (the backend merges them): a 64-bit buffer load
        // whose halves are bit-cast to float is shrunk to one dword by this
        // compiler, both halves then holding the scale
        const auto prs = buf_rsrc(w.step + 2 * pbase);
        r.step = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(prs, pvo, 0, 0));
        r.zp = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(prs, pvo + 4, 0, 0));
      }
    }
  };
  // NF4 levels of this lane's table entries (set once the codebook is in
  // LDS): level[4q + i], or for block 32 level[8 (q & 1) + i]
  float lvq[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  // Decode this lane's 16 weights into the stage: the 4-bit formats through a
  // per-block table built by the quad (entries level[c] * s for NF4,
  // (c - zp) * scale for uint4); Q8_0 bytes times the fp16 scale of the
  // lane's 32-element half.
  auto decode_to = [&](const WRaw& r, u32x4_t* dst) {
    if constexpr (FMT == kFmtQ8) {
      const float d = half_bits_to_float(q >= 2 ? r.qbyte >> 16 : r.qbyte & 0xFFFFu);
      dst[0] = decode_q8x8(r.codes[0], r.codes[1], d);
      dst[1] = decode_q8x8(r.codes[2], r.codes[3], d);
    } else {
      float lvr[4];
      float sc;
      if constexpr (FMT == kFmtU4) {
        const int zp = (int)r.zp;   // c - zp formed as an integer: +0 at c == zp
#pragma unroll
        for (int i = 0; i < 4; ++i) lvr[i] = (float)(4 * q + i - zp);
        sc = r.step;
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) lvr[i] = lvq[i];
        sc = (float)r.qbyte * r.step;
      }
      // block 32: the half-quads hold different scales, so each lane pair
      // builds its own table
      const Lut t = BS == 32 ? make_lut_pair(lvq, sc) : make_lut_quad<FI::f16>(lvr, sc);
      dst[0] = decode8(t, r.codes[0]);
      dst[1] = decode8(t, r.codes[1]);
    }
  };
  auto wdst = [&](int stage) {
    return reinterpret_cast<u32x4_t*>(sW + stage * G::stage + wr * G::ld + wcb * 64 + q * 16);
  };
  // MFMA fragments of this wave for one step: A rows 64 wm + 32 mt, B
  // columns 32 nt, contraction kk = 2g + h (16 wide each)
  auto read_frags = [&](const uint16_t* sa, const uint16_t* sw, u32x4_t (&a)[2][2],
                        u32x4_t (&b)[2][4]) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int kk = 2 * grp + h;
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) {
        const int r = wm * 64 + 32 * mt + lr;
        a[h][mt] = *reinterpret_cast<const u32x4_t*>(sa + r * GBK + a_chunk(r, 2 * kk + lg) * 8);
      }
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        if (DX) {
          const int G16 = lane >> 4, i16 = lane & 15;
          const int row = 16 * kk + 8 * (G16 >> 1) + (i16 >> 2);
          const int col = 32 * nt + 16 * (G16 & 1) + 4 * (i16 & 3);
          const u32x2_t lo = ds_tr16(sw + row * G::ld + col);
          const u32x2_t hi = ds_tr16(sw + (row + 4) * G::ld + col);
          b[h][nt] = u32x4_t{lo[0], lo[1], hi[0], hi[1]};
        } else {
          b[h][nt] = *reinterpret_cast<const u32x4_t*>(sw + (32 * nt + lr) * G::ld + 16 * kk + 8 * lg);
        }
      }
    }
  };

  __syncthreads();
  if constexpr (FmtInfo<FMT>::nf4) {
    if constexpr (FmtInfo<FMT>::block == 32) {
#pragma unroll
      for (int i = 0; i < 8; ++i) lvq[i] = s_lv[8 * (q & 1) + i];
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) lvq[i] = s_lv[4 * q + i];
    }
  }

  f32x16_t acc[2][4];
#pragma unroll
  for (int mt = 0; mt < 2; ++mt)
#pragma unroll
    for (int nt = 0; nt < 4; ++nt)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[mt][nt][i] = 0.f;

  if (s_begin < s_end) {
    const int last = s_end - 1;
    // prologue: decoded weight of s_begin (stage 0), activation tiles of
    // s_begin and s_begin+1, codes of s_begin+1 and s_begin+2
    WRaw rw[3];   // codes of step t in rw[(t - s_begin) % 3]
    {
      WRaw wf;
      load_w(s_begin, wf);
      fill_a(s_begin, 0);
      fill_a(min(s_begin + 1, last), 1);
      load_w(min(s_begin + 1, last), rw[1]);
      load_w(min(s_begin + 2, last), rw[2]);
      __builtin_amdgcn_s_waitcnt(0);       // (prologue only)
      decode_to(wf, wdst(0));
      __syncthreads();
    }
    u32x4_t fa[2][2], fb[2][4];

    // Ping-pong schedule.  Every step t has a memory phase MEM(t) and a
    // matrix phase MMA(t) per wave; group 0 runs MEM(t) while group 1 runs
    // MMA(t-1), then group 0 runs MMA(t) while group 1 runs MEM(t), with a
    // workgroup barrier between phases, so each SIMD (one wave of each group)
    // alternates the matrix cores between its two waves.
    //   MEM(t): read this wave's fragments of step t (A ring stage t%3, W
    //   stage t&1), decode the group's half of W(t+1) into stage (t+1)&1 and
    //   wait for its LDS traffic.
    //   MMA(t): 16 MFMAs (2 K halves x 2 x 4 tiles) from those fragments,
    //   with the DMA of A(t+2) and the codes of W(t+3) issued between them so
    //   that the address and data paths stay busy under the matrix work.
    // A(t+2) is first read by group 0 in MEM(t+2), two phases after group 1
    // issued its rows in MMA(t): every wave waits for all its loads at the
    // end of its next MEM phase.
    auto mem = [&](int st, auto PHc) {
      constexpr int PH = decltype(PHc)::value;   // (st - s_begin) % 3
      const int rel = st - s_begin;
      read_frags(sA + (rel % NA) * A_STAGE, sW + (rel & 1) * G::stage, fa, fb);
      decode_to(rw[(PH + 1) % 3], wdst((rel + 1) & 1));
      QL_LGKMCNT0();
      QL_VMCNT(0);
      __builtin_amdgcn_sched_barrier(0);
      k_barrier_issue();
      __builtin_amdgcn_sched_barrier(0);
    };
    auto mma = [&](int st, auto PHc) {
      constexpr int PH = decltype(PHc)::value;
      const int rel = st - s_begin;
      const int sa = min(st + 2, last);
      const int64_t c0 = (int64_t)sa * GBK;
      uint16_t* abase = sA + ((rel + 2) % NA) * A_STAGE;
      const bool full = !DX || sa < full_steps;
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
          for (int nt = 0; nt < 4; ++nt) {
            acc[mt][nt] = mfma32<FI::f16>(fa[h][mt], fb[h][nt], acc[mt][nt]);
            const int i = (h * 2 + mt) * 4 + nt;
            if (i % 4 == 0) {
              __builtin_amdgcn_sched_barrier(0);
              if (full)
                fill_a_one(c0, abase, i / 4, std::true_type{});
              else
                fill_a_one(c0, abase, i / 4, std::false_type{});
              __builtin_amdgcn_sched_barrier(0);
            }
            if (i == 6) {
              load_w(min(st + 3, last), rw[PH % 3]);
              __builtin_amdgcn_sched_barrier(0);
            }
          }
      __builtin_amdgcn_sched_barrier(0);
      k_barrier_issue();
      __builtin_amdgcn_sched_barrier(0);
    };
    // group 1 starts one phase late
    if (grp == 1) k_barrier_issue();
    using P0 = std::integral_constant<int, 0>;
    using P1 = std::integral_constant<int, 1>;
    using P2 = std::integral_constant<int, 2>;
    int st = s_begin;
    for (; st + 2 < s_end; st += 3) {
      mem(st, P0{});
      mma(st, P0{});
      mem(st + 1, P1{});
      mma(st + 1, P1{});
      mem(st + 2, P2{});
      mma(st + 2, P2{});
    }
    if (st < s_end) {
      mem(st, P0{});
      mma(st, P0{});
    }
    if (st + 1 < s_end) {
      mem(st + 1, P1{});
      mma(st + 1, P1{});
    }
    // group 0 matches group 1's extra barrier
    if (grp == 0) k_barrier_issue();
  }

  // ---- the two groups hold partial sums over complementary K halves of the
  // same 64 x 128 tiles: group 0 finishes columns [0, 64), group 1 columns
  // [64, 128).  Each wave hands the other group's half to its partner wave
  // (same rows) through 16 KiB of LDS: waves 0-5 in the activation ring,
  // waves 6-7 in the weight stages.  The clamped prefetches of the last steps
  // may still be landing in the ring, hence the full wait first.
  QL_VMCNT(0);
  __syncthreads();
  f32x16_t fin[2][2];   // this wave's finished 64 x 64 output tile
  {
    auto region = [&](int v) {
      return v < 6 ? reinterpret_cast<f32x4_t*>(sA) + (size_t)v * 1024
                   : reinterpret_cast<f32x4_t*>(sW) + (size_t)(v - 6) * 1024;
    };
    static_assert(2 * G::stage * sizeof(uint16_t) >= 2 * 16384, "exchange needs 32 KiB of stages");
    static_assert(NA * A_STAGE * sizeof(uint16_t) >= 6 * 16384, "exchange needs 96 KiB of ring");
    // (the accumulators are selected, never indexed by the group, so they
    // stay in registers)
    f32x4_t* mine = region(wave);
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const f32x16_t v = grp == 0 ? acc[mt][2 + j] : acc[mt][j];
#pragma unroll
        for (int e = 0; e < 4; ++e)
          mine[((mt * 2 + j) * 4 + e) * 64 + lane] = f32x4_t{v[4 * e], v[4 * e + 1], v[4 * e + 2], v[4 * e + 3]};
        fin[mt][j] = grp == 0 ? acc[mt][j] : acc[mt][2 + j];
      }
    __syncthreads();
    const f32x4_t* theirs = region(wave ^ 4);
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const f32x4_t v = theirs[((mt * 2 + j) * 4 + e) * 64 + lane];
#pragma unroll
          for (int i = 0; i < 4; ++i) fin[mt][j][4 * e + i] += v[i];
        }
  }
  const int nt0 = grp == 0 ? 0 : 2;   // this wave's output columns: nt0, nt0 + 1

  // ---- epilogue.  LoRA term (ksplit == 1): out += (scaling * L) R^T on the
  // matrix cores, 16 ranks per MFMA step; the fp32 factor scaling * L is
  // split into 16-bit hi + lo parts so the product keeps fp32 accuracy.  The
  // operands of each 16-rank chunk are fetched without branches (indices
  // clamped into the matrices, values past the rank masked to zero), as
  // 16-byte loads where the layout allows, and the next chunk's fetch is
  // issued before the current chunk's MFMAs.
  if (ksplit == 1 && lora.r > 0) {
    const int r = lora.r;
    int64_t orow[2], mrow[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) orow[j] = min(o0 + 32 * (nt0 + j) + lr, O - 1);
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) mrow[mt] = min(m0 + wm * 64 + 32 * mt + lr, M - 1);
    const bool rvec = lora.rs_j == 1 && r % 8 == 0 && (lora.rs_c % 8) == 0 &&
                      (reinterpret_cast<uintptr_t>(lora.R) & 15) == 0;
    const bool lvec = r % 8 == 0 && (reinterpret_cast<uintptr_t>(lora.L) & 15) == 0;
    struct Ops {
      u32x4_t rb[2];      // R[o][jb .. jb+7], 16-bit pairs
      f32x4_t lv[2][2];   // L[m][jb .. jb+7]
    };
    // this lane's ranks of the chunk at j0: jb .. jb+7, jb = j0 + 8 lg
    auto fetch = [&](int j0, Ops& op) {
      const int jb = j0 + 8 * lg;
      const int jc = min(jb, r - 8 > 0 ? r - 8 : 0);   // vector start kept inside the row
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        if (rvec) {
          op.rb[j] = *reinterpret_cast<const u32x4_t*>(lora.R + orow[j] * lora.rs_c + jc);
        } else {
          uint32_t h[8];
#pragma unroll
          for (int e = 0; e < 8; ++e)
            h[e] = lora.R[orow[j] * lora.rs_c + (int64_t)min(jb + e, r - 1) * lora.rs_j];
          op.rb[j] = u32x4_t{h[0] | h[1] << 16, h[2] | h[3] << 16, h[4] | h[5] << 16, h[6] | h[7] << 16};
        }
      }
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) {
        const float* lp = lora.L + mrow[mt] * r;
        if (lvec) {
          op.lv[mt][0] = *reinterpret_cast<const f32x4_t*>(lp + jc);
          op.lv[mt][1] = *reinterpret_cast<const f32x4_t*>(lp + jc + 4);
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e) op.lv[mt][e >> 2][e & 3] = lp[min(jb + e, r - 1)];
        }
      }
    };
    auto apply = [&](int j0, const Ops& op) {
      const int jb = j0 + 8 * lg;
      // ranks past r read a clamped element: zero both factors' share
      u32x4_t rb[2];
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        rb[j] = op.rb[j];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const bool k0 = jb + 2 * e < r, k1 = jb + 2 * e + 1 < r;
          rb[j][e] = (k0 ? rb[j][e] & 0xFFFFu : 0u) | (k1 ? rb[j][e] & 0xFFFF0000u : 0u);
        }
      }
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) {
        float tv[8], lo[8];
#pragma unroll
        for (int e = 0; e < 8; ++e)
          tv[e] = jb + e < r ? lora.scaling * op.lv[mt][e >> 2][e & 3] : 0.f;
        u32x4_t ahi, alo;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          ahi[e] = pack16x2<FI::f16>(tv[2 * e], tv[2 * e + 1]);
          lo[2 * e] = tv[2 * e] - lo16<FI::f16>(ahi[e]);
          lo[2 * e + 1] = tv[2 * e + 1] - hi16<FI::f16>(ahi[e]);
          alo[e] = pack16x2<FI::f16>(lo[2 * e], lo[2 * e + 1]);
        }
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          fin[mt][j] = mfma32<FI::f16>(ahi, rb[j], fin[mt][j]);
          fin[mt][j] = mfma32<FI::f16>(alo, rb[j], fin[mt][j]);
        }
      }
    };
    // two operand sets in turn (a copy of a set still in flight would wait)
    Ops opa, opb;
    fetch(0, opa);
    for (int j0 = 0; j0 < r; j0 += 32) {
      const bool two = j0 + 16 < r;
      if (two) fetch(j0 + 16, opb);
      apply(j0, opa);
      if (two) {
        if (j0 + 32 < r) fetch(j0 + 32, opa);
        apply(j0 + 16, opb);
      }
    }
  }
#pragma unroll
  for (int mt = 0; mt < 2; ++mt)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int64_t m = m0 + wm * 64 + 32 * mt + 8 * (i >> 2) + 4 * lg + (i & 3);
        const int64_t o = o0 + 32 * (nt0 + j) + lr;
        if (m < M && o < O) {
          const float v = fin[mt][j][i];
          if (ksplit > 1)
            part[((int64_t)split * M + m) * O + o] = v;
          else if (out16)
            // written once: non-temporal stores leave the L2 to the operand
            // tiles that the other workgroups reuse
            __builtin_nontemporal_store(to16<FI::f16>(v), reinterpret_cast<uint16_t*>(out) + m * O + o);
          else
            __builtin_nontemporal_store(v, reinterpret_cast<float*>(out) + m * O + o);
        }
      }
}

template <bool DX>
static constexpr size_t smem_bytes() {
  return sizeof(uint16_t) * NA * A_STAGE;   // dynamic part: the activation ring
}

template <bool DX, bool VEC, int FMT>
static hipError_t launch_one(dim3 grid, hipStream_t s, const uint16_t* act, const Nf4View& w,
                             const float* codebook, int64_t M, const LoraTerm& lora, void* out,
                             bool out16, float* part, int ksplit, int per, int64_t mtiles,
                             int64_t otiles) {
  // the dynamic LDS limit of this instantiation, set once per process (a
  // function-local static is initialized exactly once, thread-safely)
  static const hipError_t attr = hipFuncSetAttribute(
      reinterpret_cast<const void*>(&k_gemm<DX, VEC, FMT>), hipFuncAttributeMaxDynamicSharedMemorySize,
      (int)smem_bytes<DX>());
  if (attr != hipSuccess) return attr;
  hipLaunchKernelGGL((k_gemm<DX, VEC, FMT>), grid, dim3(512), smem_bytes<DX>(), s, act, w, codebook,
                     M, lora, out, (int)out16, part, ksplit, per, mtiles, otiles);
  return hipGetLastError();
}

template <bool DX, bool VEC>
static hipError_t launch_fmt(dim3 grid, hipStream_t s, const uint16_t* act, const Nf4View& w,
                             const float* codebook, int64_t M, const LoraTerm& lora, void* out,
                             bool out16, float* part, int ksplit, int per, int64_t mtiles,
                             int64_t otiles) {
#define QL_ONE(F) \
  launch_one<DX, VEC, F>(grid, s, act, w, codebook, M, lora, out, out16, part, ksplit, per, mtiles, otiles)
  switch (w.fmt) {
    case kFmtNf4Dq: return QL_ONE(kFmtNf4Dq);
    case kFmtNf4: return QL_ONE(kFmtNf4);
    case kFmtU4: return QL_ONE(kFmtU4);
    case kFmtQ8: return QL_ONE(kFmtQ8);
    case kFmtNf4Dq32: return QL_ONE(kFmtNf4Dq32);
    case kFmtNf4_32: return QL_ONE(kFmtNf4_32);
    case kFmtNf4Dq128: return QL_ONE(kFmtNf4Dq128);
    case kFmtNf4DqF16: return QL_ONE(kFmtNf4DqF16);
    default: return QL_ONE(kFmtNf4_128);
  }
#undef QL_ONE
}

template <bool DX>
static hipError_t launch(const Nf4View& w, const float* codebook, const uint16_t* act, int64_t M,
                         const LoraTerm& lora, void* out, bool out16, float* part, int ksplit,
                         hipStream_t s) {
  const int64_t C = DX ? w.n : w.k, O = DX ? w.k : w.n;
  const int nsteps = (int)((C + GBK - 1) / GBK);
  const int per = (nsteps + ksplit - 1) / ksplit;
  const int64_t mtiles = (M + GBM - 1) / GBM, otiles = (O + GBN - 1) / GBN;
  const dim3 grid((unsigned)(mtiles * otiles * ksplit));
  // the weight format and 16-byte activation rows select the instantiation
  // (the forward's contraction is a whole number of 64-blocks)
  if constexpr (DX) {
    if (C % 8 != 0)
      return launch_fmt<DX, false>(grid, s, act, w, codebook, M, lora, out, out16, part, ksplit,
                                   per, mtiles, otiles);
  }
  return launch_fmt<DX, true>(grid, s, act, w, codebook, M, lora, out, out16, part, ksplit, per,
                              mtiles, otiles);
}

hipError_t launch_gemm_fwd(const Nf4View& w, const float* codebook, const uint16_t* X, int64_t M,
                           const LoraTerm& lora, void* Y, bool y16, float* part, int ksplit,
                           hipStream_t s) {
  return launch<false>(w, codebook, X, M, lora, Y, y16, part, ksplit, s);
}

hipError_t launch_gemm_dx(const Nf4View& w, const float* codebook, const uint16_t* dY, int64_t M,
                          const LoraTerm& lora, void* dX, bool dx16, float* part, int nsplit,
                          hipStream_t s) {
  return launch<true>(w, codebook, dY, M, lora, dX, dx16, part, nsplit, s);
}

}  // namespace ql
