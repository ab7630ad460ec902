// Fused-dequant MFMA GEMMs of the quantized linear (large-M regime):
//   forward   Y  = X  deq(W)^T (+ LoRA term)    contraction over k
//   backward  dX = dY deq(W)   (+ LoRA term)    contraction over n
// The 4-bit weight is decoded to bf16 inside the kernel and lives only in
// registers and LDS (www.cf-1.com/news/5705389 §2.2, §4.2: block dequant in
// the GEMM's outer loop, results kept in registers / shared memory;
// www.lqnn.cn/news/228537 §3.3: dequantize to 16 bits for the product, then
// discard).
//
// gfx950 design:
//  * 256 x 128 output tile per workgroup, 8 waves (two per SIMD, so one
//    wave's LDS/barrier latency and decode work overlap the other's MFMAs);
//    wave w owns the 64 x 64 sub-tile (w%4, w/4): 2 x 2 MFMA 32x32x16 bf16
//    tiles with fp32 accumulators.
//  * The activation operand (X or dY) goes global -> LDS with the gfx950
//    global_load_lds b128 DMA (no registers, each wave load covers 8 whole
//    128-byte row pieces) into a 3-stage ring, two K-steps ahead.  16-byte
//    chunks are XOR-swizzled by row so the MFMA fragment reads are free of
//    bank conflicts.
//  * The weight tile of each K-step (128 x 64 weights = 128 NF4 blocks) is
//    decoded by all 512 threads into a double-buffered LDS stage: the four
//    lanes of a DPP quad share a block, build its 16-entry table together
//    (broadcast with quad_perm) and decode 16 weights each.  The decode of
//    step s+1 is interleaved with the MFMAs of step s, one barrier per step;
//    it is amortized over 256 output rows.
//  * Forward reads B fragments with ds_read_b128 from the [n][k] stage; the
//    backward contracts over n and reads them with the transposing
//    ds_read_b64_tr_b16 from a [n][k] stage.
//  * Tiles are renumbered so that the workgroups sharing one activation row
//    tile run on the same XCD (workgroup ids are dealt to the 8 XCDs round
//    robin), keeping that tile in the XCD's L2.
#include "common.h"
#include "kernels.h"

namespace ql {

typedef float f32x16_t __attribute__((ext_vector_type(16)));

// D[32x32] += A[32x16] B[16x32]; lane l holds A[l%32][8(l/32)..+7],
// B[8(l/32)..+7][l%32], D[8(i/4) + 4(l/32) + i%4][l%32] for i = 0..15.
QL_DEV f32x16_t mfma32(const u32x4_t a, const u32x4_t b, f32x16_t c) {
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

QL_DEV float lora_dot_g(const LoraTerm& L, int64_t m, int64_t c) {
  float acc = 0.f;
  const float* lr = L.L + m * L.r;
  const uint16_t* rr = L.R + c * L.rs_c;
  for (int j = 0; j < L.r; ++j) acc += lr[j] * __builtin_bit_cast(float, (uint32_t)rr[j * L.rs_j] << 16);
  return acc;
}

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

#ifndef QL_A_DMA
#define QL_A_DMA 1                     // activation tiles by LDS DMA (1) or through registers (0)
#endif
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

// Physical 16-byte chunk of logical chunk c in activation row r of a stage.
QL_DEV int a_chunk(int r, int c) { return c ^ ((r >> 1) & 7); }

template <bool DX, bool VEC>
__global__ __launch_bounds__(512, 1) void k_gemm(const uint16_t* __restrict__ act, Nf4View w,
                                                 const float* __restrict__ codebook, int64_t M,
                                                 LoraTerm lora, void* __restrict__ out, int out_bf16,
                                                 float* __restrict__ part, int ksplit,
                                                 int steps_per_split, int64_t mtiles, int64_t otiles) {
  using G = Geo<DX>;
  extern __shared__ __attribute__((aligned(16))) uint16_t sA[];   // [NA][GBM rows][GBK], swizzled
  __shared__ __attribute__((aligned(16))) uint16_t sW[2 * G::stage];   // decoded weight stages
  __shared__ float s_lv[16];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave & 3, wn = wave >> 2;                  // 64-row block, 64-column half
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

  if (tid < 16) s_lv[tid] = codebook[tid];

  // Decode role (all 512 threads): a quad of lanes shares one of the step's
  // 128 blocks, lane q = tid & 3 decodes its elements [16q, 16q+16).
  const int q = tid & 3;
  const int blk = tid >> 2;
  const int wr = DX ? (blk >> 1) : blk;                     // stage row
  const int wcb = DX ? (blk & 1) : 0;                       // block within the stage row (dx)

  // per-lane source of each of the 4 DMA loads: row base and the largest
  // step offset that keeps the 8-element piece inside the row
  const uint16_t* a_src[4];
  int64_t a_cmax[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int rl = wave * 32 + i * 8 + (lane >> 3);
    const int lc = a_chunk(rl, lane & 7);
    a_src[i] = act + min(m0 + rl, M - 1) * C + lc * 8;
    a_cmax[i] = C - 8 - lc * 8;
  }
  // Activation tile of step st into ring stage `stage`: wave w fills rows
  // [32w, 32w+32) with 4 DMA loads of 8 rows; lane l lands at byte 16l of its
  // load's 1 KiB, i.e. row l/8, physical chunk l%8.  Rows past M and columns
  // past the contraction are clamped (products discarded or against zero
  // weights).
  auto fill_a = [&](int st, int stage) {
    const int64_t c0 = (int64_t)st * GBK;
    uint16_t* base = sA + stage * A_STAGE;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      uint16_t* dst = base + (wave * 32 + i * 8) * GBK;
      if (VEC) {
        __builtin_amdgcn_global_load_lds(a_src[i] + min(c0, a_cmax[i]),
                                         (__attribute__((address_space(3))) void*)dst, 16, 0, 0);
      } else {
        const int rl = wave * 32 + i * 8 + (lane >> 3);
        const int64_t row = min(m0 + rl, M - 1);
        const int64_t c = c0 + a_chunk(rl, lane & 7) * 8;
        const u32x4_t v = c < C ? load_act8(act + row * C, c, C, false) : u32x4_t{0u, 0u, 0u, 0u};
        *reinterpret_cast<u32x4_t*>(dst + lane * 8) = v;
      }
    }
  };
  // register-staged alternative: load (coalesced, same lane mapping) now,
  // store to the ring stage later
  auto load_a_regs = [&](int st, u32x4_t (&r)[4]) {
    const int64_t c0 = (int64_t)st * GBK;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (VEC) {
        r[i] = *reinterpret_cast<const u32x4_t*>(a_src[i] + min(c0, a_cmax[i]));
      } else {
        const int rl = wave * 32 + i * 8 + (lane >> 3);
        const int64_t row = min(m0 + rl, M - 1);
        const int64_t c = c0 + a_chunk(rl, lane & 7) * 8;
        r[i] = c < C ? load_act8(act + row * C, c, C, false) : u32x4_t{0u, 0u, 0u, 0u};
      }
    }
  };
  auto store_a_regs = [&](int stage, const u32x4_t (&r)[4]) {
    uint16_t* base = sA + stage * A_STAGE;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      *reinterpret_cast<u32x4_t*>(base + (wave * 32 + i * 8) * GBK + lane * 8) = r[i];
  };

  struct WRaw {
    u32x2_t codes;    // this lane's two packed words
    uint32_t qbyte;   // the block's 8-bit scale
    float step;
    bool ok;
  };
  // flat index of this lane's block at step st: b0 + st * bstride; its
  // storage position (rows in groups of 16, k-block-major inside a group):
  // forward p0 + st * R (the row is fixed), backward recomputed per step
  const int64_t kb_dx = o0 / kBlock + wcb;
  const int64_t b0 = DX ? (int64_t)wr * nkb + kb_dx : (o0 + wr) * nkb;
  const int64_t bstride = DX ? GBK * nkb : 1;
  const bool w_ok_fixed = DX ? kb_dx < nkb : (o0 + wr) < N;
  const int64_t fg0 = (o0 + wr) & ~int64_t(15);
  const int64_t fR = min(int64_t(16), N - fg0);
  const int64_t fp0 = fg0 * nkb + (o0 + wr - fg0);
  auto load_w = [&](int st, WRaw& r) {
    r.ok = w_ok_fixed && (!DX || (int64_t)st * GBK + wr < N);
    int64_t b = 0, p = 0;
    if (DX) {
      const int64_t n = (int64_t)st * GBK + wr, g0 = n & ~int64_t(15);
      b = r.ok ? b0 + st * bstride : 0;
      p = r.ok ? g0 * nkb + kb_dx * min(int64_t(16), N - g0) + (n - g0) : 0;
    } else {
      b = r.ok ? b0 + st : 0;
      p = r.ok ? fp0 + st * fR : 0;
    }
    r.codes = *reinterpret_cast<const u32x2_t*>(w.codes + p * 32 + q * 8);
    r.qbyte = w.qscale[p];
    r.step = w.step[b >> 8];
  };
  auto scale_of = [](const WRaw& r) {
    return r.ok ? (float)r.qbyte * r.step : 0.f;
  };
  __syncthreads();
  float lvq[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) lvq[i] = s_lv[4 * q + i];

  f32x16_t acc[2][2];
#pragma unroll
  for (int mt = 0; mt < 2; ++mt)
#pragma unroll
    for (int nt = 0; nt < 2; ++nt)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[mt][nt][i] = 0.f;

  auto read_a = [&](const uint16_t* sa, int kk, u32x4_t (&a)[2]) {
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      const int r = wm * 64 + 32 * mt + lr;
      a[mt] = *reinterpret_cast<const u32x4_t*>(sa + r * GBK + a_chunk(r, 2 * kk + lg) * 8);
    }
  };
  auto read_b = [&](const uint16_t* sw, int kk, u32x4_t (&b)[2]) {
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      if (DX) {
        const int G16 = lane >> 4, i16 = lane & 15;
        const int row = 16 * kk + 8 * (G16 >> 1) + (i16 >> 2);
        const int col = wn * 64 + 32 * nt + 16 * (G16 & 1) + 4 * (i16 & 3);
        const u32x2_t lo = ds_tr16(sw + row * G::ld + col);
        const u32x2_t hi = ds_tr16(sw + (row + 4) * G::ld + col);
        b[nt] = u32x4_t{lo[0], lo[1], hi[0], hi[1]};
      } else {
        b[nt] = *reinterpret_cast<const u32x4_t*>(sw + (wn * 64 + 32 * nt + lr) * G::ld + 16 * kk + 8 * lg);
      }
    }
  };
  auto wdst = [&](int stage) {
    return reinterpret_cast<u32x4_t*>(sW + stage * G::stage + wr * G::ld + wcb * 64 + q * 16);
  };

  if (s_begin < s_end) {
    const int last = s_end - 1;
    // prologue: activation stages of steps s_begin, s_begin+1; decoded weight
    // stage 0 of s_begin; codes of s_begin+1 (w0) and s_begin+2 (w1)
    WRaw w0, w1;
    u32x4_t ra0[4], ra1[4];    // register-staged activations (QL_A_DMA == 0)
    {
      WRaw wf;
      load_w(s_begin, wf);
      if (QL_A_DMA) {
        fill_a(s_begin, 0);
        fill_a(min(s_begin + 1, last), 1);
      } else {
        load_a_regs(s_begin, ra0);
        load_a_regs(min(s_begin + 1, last), ra1);
      }
      load_w(min(s_begin + 1, last), w0);
      load_w(min(s_begin + 2, last), w1);
      QL_VMCNT(0);
      if (!QL_A_DMA) {
        store_a_regs(0, ra0);
        store_a_regs(1, ra1);
        load_a_regs(min(s_begin + 2, last), ra0);
      }
      const Lut t = make_lut_quad(lvq, scale_of(wf));
      u32x4_t* dst = wdst(0);
      dst[0] = decode8(t, wf.codes[0]);
      dst[1] = decode8(t, wf.codes[1]);
      __syncthreads();
    }

    // One K-step t: MFMAs on activation stage t%3 and weight stage (t-s)&1.
    // First the activation tile of step t+2 is started (DMA), or, with
    // register staging, the tile of t+2 (loaded a step ago) is stored and the
    // tile of t+3 loaded; then all fragment reads of the step are issued; the
    // decode of the codes of step t+1 (`wd`) into the other weight stage runs
    // between the MFMAs; then `wd` is refilled with the codes of step t+3
    // (consumed two steps later).  Every wave issues the same loads, so the
    // vmcnt values below are exact.
    auto kstep = [&](int st, WRaw& wd, u32x4_t (&ra)[4]) {
      const int rel = st - s_begin;
      const int wstage = rel & 1;
      // `wd` was loaded at the end of step t-2; issued since: the activation
      // loads of step t-1 (4) and the codes of t+2 (3)
      if (VEC) QL_VMCNT(7); else QL_VMCNT(0);
      const float sc = scale_of(wd);
      if (QL_A_DMA) {
        fill_a(min(st + 2, last), (rel + 2) % NA);
      } else {
        store_a_regs((rel + 2) % NA, ra);       // tile of t+2, loaded during step t-1
        load_a_regs(min(st + 3, last), ra);     // tile of t+3
      }
      __builtin_amdgcn_sched_barrier(0);
      const uint16_t* sa = sA + (rel % NA) * A_STAGE;
      const uint16_t* sw = sW + wstage * G::stage;
      u32x4_t a[4][2], b[4][2];
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        read_a(sa, kk, a[kk]);
        read_b(sw, kk, b[kk]);
      }
      // forward: all fragment reads of the step are issued before the first
      // MFMA (the scheduler would otherwise sink each read next to its use and
      // expose the LDS latency at every MFMA pair); measured slower for the
      // transposing reads of the backward, which keep the default order
      if (!DX) __builtin_amdgcn_sched_barrier(0);
      const Lut t = make_lut_quad(lvq, sc);
      u32x4_t* dst = wdst(wstage ^ 1);
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
          for (int nt = 0; nt < 2; ++nt) acc[mt][nt] = mfma32(a[kk][mt], b[kk][nt], acc[mt][nt]);
        if (kk == 1) dst[0] = decode8(t, wd.codes[0]);
        if (kk == 2) dst[1] = decode8(t, wd.codes[1]);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // one MFMA
          __builtin_amdgcn_sched_group_barrier(0x002, 6, 0);   // then up to six VALU
        }
      }
      __builtin_amdgcn_sched_barrier(0);
      load_w(min(st + 3, last), wd);
      // the activation loads of step t+1 were issued a step ago; issued after
      // them: codes of t+2 (3), activation loads of this step (4), codes of
      // t+3 (3).  (Register staging: the loads of t+3 issued this step are
      // stored next step, also waited for here.)
      if (VEC) QL_VMCNT(10); else QL_VMCNT(0);
      k_barrier();
    };

    int st = s_begin;
    for (; st + 1 < s_end; st += 2) {
      kstep(st, w0, ra0);
      kstep(st + 1, w1, ra0);
    }
    if (st < s_end) kstep(st, w0, ra0);
  }

  // ---- epilogue.  LoRA term (ksplit == 1): out += (scaling * L) R^T on the
  // matrix cores, 16 ranks per MFMA step; the fp32 factor scaling * L is
  // split into bf16 hi + lo parts so the product keeps fp32 accuracy.
  if (ksplit == 1 && lora.r > 0) {
    for (int j0 = 0; j0 < lora.r; j0 += 16) {
      // B fragments: R[o][j0 + 8*lg + e] (the rank index is the contraction)
      u32x4_t rb[2];
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
        const int64_t o = min(o0 + wn * 64 + 32 * nt + lr, O - 1);
        uint32_t h[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int j = j0 + 8 * lg + e;
          h[e] = j < lora.r ? lora.R[o * lora.rs_c + (int64_t)j * lora.rs_j] : 0u;
        }
        rb[nt] = u32x4_t{h[0] | h[1] << 16, h[2] | h[3] << 16, h[4] | h[5] << 16, h[6] | h[7] << 16};
      }
      // A fragments: s * L[m][j], split into bf16 hi + lo (exact to 2^-16)
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) {
        const int64_t m = min(m0 + wm * 64 + 32 * mt + lr, M - 1);
        float tv[8], lo[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int j = j0 + 8 * lg + e;
          tv[e] = j < lora.r ? lora.scaling * lora.L[m * lora.r + j] : 0.f;
        }
        u32x4_t ahi, alo;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          ahi[e] = pack_bf16x2(tv[2 * e], tv[2 * e + 1]);
          lo[2 * e] = tv[2 * e] - bf16_lo(ahi[e]);
          lo[2 * e + 1] = tv[2 * e + 1] - bf16_hi(ahi[e]);
          alo[e] = pack_bf16x2(lo[2 * e], lo[2 * e + 1]);
        }
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
          acc[mt][nt] = mfma32(ahi, rb[nt], acc[mt][nt]);
          acc[mt][nt] = mfma32(alo, rb[nt], acc[mt][nt]);
        }
      }
    }
  }
#pragma unroll
  for (int mt = 0; mt < 2; ++mt)
#pragma unroll
    for (int nt = 0; nt < 2; ++nt)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int64_t m = m0 + wm * 64 + 32 * mt + 8 * (i >> 2) + 4 * lg + (i & 3);
        const int64_t o = o0 + wn * 64 + 32 * nt + lr;
        if (m < M && o < O) {
          const float v = acc[mt][nt][i];
          if (ksplit > 1)
            part[((int64_t)split * M + m) * O + o] = v;
          else if (out_bf16)
            reinterpret_cast<uint16_t*>(out)[m * O + o] = to_bf16(v);
          else
            reinterpret_cast<float*>(out)[m * O + o] = v;
        }
      }
}

template <bool DX>
static constexpr size_t smem_bytes() {
  return sizeof(uint16_t) * NA * A_STAGE;   // dynamic part: the activation ring
}

template <bool DX, bool VEC>
static hipError_t launch_one(dim3 grid, hipStream_t s, const uint16_t* act, const Nf4View& w,
                             const float* codebook, int64_t M, const LoraTerm& lora, void* out,
                             bool bf16, float* part, int ksplit, int per, int64_t mtiles,
                             int64_t otiles) {
  static bool attr_set = false;   // idempotent: the same value every time
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_gemm<DX, VEC>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize,
                                       (int)smem_bytes<DX>());
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  hipLaunchKernelGGL((k_gemm<DX, VEC>), grid, dim3(512), smem_bytes<DX>(), s, act, w, codebook, M,
                     lora, out, (int)bf16, part, ksplit, per, mtiles, otiles);
  return hipGetLastError();
}

template <bool DX>
static hipError_t launch(const Nf4View& w, const float* codebook, const uint16_t* act, int64_t M,
                         const LoraTerm& lora, void* out, bool bf16, float* part, int ksplit,
                         hipStream_t s) {
  const int64_t C = DX ? w.n : w.k, O = DX ? w.k : w.n;
  const int nsteps = (int)((C + GBK - 1) / GBK);
  const int per = (nsteps + ksplit - 1) / ksplit;
  const int64_t mtiles = (M + GBM - 1) / GBM, otiles = (O + GBN - 1) / GBN;
  const dim3 grid((unsigned)(mtiles * otiles * ksplit));
  if (!DX || C % 8 == 0)
    return launch_one<DX, true>(grid, s, act, w, codebook, M, lora, out, bf16, part, ksplit, per,
                                mtiles, otiles);
  return launch_one<DX, false>(grid, s, act, w, codebook, M, lora, out, bf16, part, ksplit, per,
                               mtiles, otiles);
}

hipError_t launch_gemm_fwd(const Nf4View& w, const float* codebook, const uint16_t* X, int64_t M,
                           const LoraTerm& lora, void* Y, bool y_bf16, float* part, int ksplit,
                           hipStream_t s) {
  return launch<false>(w, codebook, X, M, lora, Y, y_bf16, part, ksplit, s);
}

hipError_t launch_gemm_dx(const Nf4View& w, const float* codebook, const uint16_t* dY, int64_t M,
                          const LoraTerm& lora, void* dX, bool dx_bf16, float* part, int nsplit,
                          hipStream_t s) {
  return launch<true>(w, codebook, dY, M, lora, dX, dx_bf16, part, nsplit, s);
}

}  // namespace ql
