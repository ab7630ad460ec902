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
// gfx950 design (producer / consumer):
//  * 256 x 128 output tile per workgroup of 8 waves; wave w and wave w + 4 run
//    on the same SIMD.  Waves 0-3 (consumers) own rows 64w .. +63 x all 128
//    columns and issue every MFMA (32x32x16, 16-bit operands, fp32
//    accumulators): 32 per 64-deep K-step, back to back.  Waves 4-7
//    (producers) decode the weight tile of the next K-step into LDS.  The
//    vector ALU work of the decode co-issues with the other wave's MFMAs on
//    the same SIMD (measured: the MFMA rate is unchanged while a second wave
//    runs table lookups at one per 6 cycles), so the decode is hidden as long
//    as it takes less time than the 32 MFMAs of a step.
//  * The activation rows of a consumer are used by no other wave: each
//    consumer moves its own 64 rows into an LDS ring with the gfx950
//    global_load_lds b128 DMA, two K-steps ahead, issued between its MFMAs,
//    and needs no barrier for them.
//  * One workgroup barrier per K-step.  Between barriers t and t+1 the
//    consumers read weight stage t % 2 (and activation stage t % 3) and the
//    producers write the weight of step t+1; the packed weight is loaded
//    three steps ahead.
//  * Each producer lane decodes half a 64-weight unit (32 weights): the two
//    lanes of a unit build its 16-entry table together (each half of the
//    entries, exchanged with DPP); Q8_0 bytes are scaled directly.
//  * Forward reads weight fragments with ds_read_b128 from the [n][k] stage;
//    the backward contracts over n and reads them with the transposing
//    ds_read_b64_tr_b16 from a [n][k] stage.
//  * The weight fragment is the MFMA's first operand, so each accumulator
//    lane holds 4 consecutive output columns; the finished tile goes through
//    LDS so that every store instruction writes whole 256-byte row pieces.
//  * Tiles are renumbered so that each XCD (workgroup ids are dealt to the 8
//    XCDs round robin) runs a contiguous run of a grouped order: two
//    activation row tiles, then the column tiles, so the 32 tiles an XCD
//    runs at once share 2 activation row tiles and 16 weight column tiles
//    through its L2.
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
  // LDS stage of one K-step of the weight, 16-bit, [rows][ld].  Forward:
  // 144-byte rows put the 16 rows of a ds_read_b128 quarter-wave on 16
  // different bank groups.  Backward: unpadded 256-byte rows whose dword
  // index is XORed with (row % 4) in bits 4-5 and in bits 2-3 (element
  // column XOR 40 (row % 4)).  A 32-lane pass of the transposing reads covers
  // four consecutive rows of one aligned 16-dword block, which the bits 4-5
  // term puts on four different 16-bank groups; a 16-lane pass of a producer
  // wave's 16-byte writes covers four consecutive rows x the four 16-dword
  // blocks at one 4-dword offset, which the bits 2-3 term moves to four
  // different offsets.  Both then hit every one of the 64 banks once per
  // pass.  (A row pitch alone cannot do both: the reads need a pitch of
  // 16 mod 64 dwords, the writes 4 or 12 mod 16; the former 76-dword pitch
  // kept the writes conflict-free and made every read take two passes.)
  static constexpr int rows = DX ? GBK : GBN;    // n (dx: contraction) or n (fwd: output)
  static constexpr int cols = DX ? GBN : GBK;    // k
  static constexpr int ld = DX ? cols : cols + 8;
  static constexpr int stage = rows * ld;
  // element offset of (row r, column c) in a stage; c even
  static QL_DEV int at(int r, int c) { return DX ? r * ld + (c ^ ((r & 3) * 40)) : r * ld + c; }
};

// Logical tile of this workgroup: consecutive logical tiles (row-tile major)
// go to the same XCD.
QL_DEV int64_t logical_tile(int64_t id, int64_t total) {
  const int64_t xcd = id & 7, slot = id >> 3;
  const int64_t base = total >> 3, rem = total & 7;
  return xcd * base + (xcd < rem ? xcd : rem) + slot;
}

// Row tiles per group of the logical tile order.  With two, the 32 tiles an
// XCD runs at once are 2 row tiles x 16 column tiles, which fetches about a
// fifth fewer bytes into the XCD's L2 than 1 x 32 (each weight column tile
// then serves two row tiles) or 4 x 8 (measured at M = 2048).
constexpr int kGroupRows = 2;

constexpr int NA = 3;                 // activation stages in the ring
constexpr int A_STAGE = GBM * GBK;     // 16-bit elements per activation stage (32 KiB)

// Physical 16-byte chunk of logical chunk c in activation row r of a stage.
QL_DEV int a_chunk(int r, int c) { return c ^ ((r >> 1) & 7); }

// Workgroup barrier of the K loop after this wave's LDS traffic.  (A plain
// __syncthreads() would add a release fence that waits for every outstanding
// vector load, draining the prefetch pipeline at each step.)  The empty asm
// statements keep the compiler from moving memory accesses across it.
QL_DEV void k_barrier() {
  QL_LGKMCNT0();
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// The same barrier with this wave's last 4 LDS operations still allowed in
// flight (LDS operations complete in order, and the producer loop issues no
// other operation counted by lgkmcnt).
QL_DEV void k_barrier_lgkm4() {
  __builtin_amdgcn_s_waitcnt(0xC47F);   // lgkmcnt(4), vmcnt and expcnt not waited
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}


// Adapter-gradient partials of launch_wgrad into their outputs: elements
// t0, t0 + stride, ... of the concatenated outputs (job a's r x ca, then job
// b's r x cb; element j * C + c), each the scaled sum of its msplit partials
// in split order, eight loads in flight.
QL_DEV void fold_wgrad(const WgradFold& f, int64_t t0, int64_t stride) {
  const int64_t na = (int64_t)f.r * f.ca, total = na + (int64_t)f.r * f.cb;
  for (int64_t idx = t0; idx < total; idx += stride) {
    const bool second = idx >= na;
    const int64_t i = second ? idx - na : idx;
    const int64_t C = second ? f.cb : f.ca;
    const int64_t pstride = (int64_t)f.r * C;
    const float* p = f.part + (second ? (int64_t)f.msplit * na : 0) + i;
    float v = 0.f;
    int s = 0;
    for (; s + 8 <= f.msplit; s += 8) {
      float t[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) t[u] = p[(int64_t)(s + u) * pstride];
#pragma unroll
      for (int u = 0; u < 8; ++u) v += t[u];
    }
    for (; s < f.msplit; ++s) v += p[(int64_t)s * pstride];
    const int64_t j = i / C, c = i - j * C;
    if (second ? f.tb : f.ta)
      (second ? f.out_b : f.out_a)[c * f.r + j] = f.scaling * v;
    else
      (second ? f.out_b : f.out_a)[i] = f.scaling * v;
  }
}

template <bool DX, bool VEC, int FMT>
__global__ __launch_bounds__(512, 1) void k_gemm(const uint16_t* __restrict__ act, Nf4View w,
                                                 const float* __restrict__ codebook, int64_t M,
                                                 LoraTerm lora, void* __restrict__ out, int out16,
                                                 float* __restrict__ part, int ksplit,
                                                 int steps_per_split, int64_t mtiles, int64_t otiles,
                                                 WgradFold fold) {
  using G = Geo<DX>;
  using FI = FmtInfo<FMT>;
  extern __shared__ __attribute__((aligned(16))) uint16_t sA[];   // [NA][GBM rows][GBK], swizzled
  __shared__ __attribute__((aligned(16))) uint16_t sW[3 * G::stage];   // decoded weight stages

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lr = lane & 31, lg = lane >> 5;
  const int64_t N = w.n, K = w.k, nkb = K / kBlock;
  const int64_t C = DX ? N : K;       // contraction length
  const int64_t O = DX ? K : N;       // output columns

  const int64_t total = mtiles * otiles * ksplit;
  const int64_t L = logical_tile(blockIdx.x, total);
  // logical order: groups of kGroupRows row tiles; inside a group, column
  // tile, then row tile, then split
  const int64_t g0 = L / (kGroupRows * otiles * ksplit) * kGroupRows;
  const int64_t gsz = min((int64_t)kGroupRows, mtiles - g0);
  const int64_t gi = L - g0 * otiles * ksplit;
  const int64_t ot_ = gi / (gsz * ksplit);
  const int64_t gr = gi - ot_ * gsz * ksplit;
  const int64_t mt_ = g0 + gr / ksplit;
  const int split = (int)(gr - gr / ksplit * ksplit);
  const int64_t m0 = mt_ * GBM, o0 = ot_ * GBN;

  const int nsteps = (int)((C + GBK - 1) / GBK);
  const int s_begin = split * steps_per_split;
  const int s_end = min(nsteps, s_begin + steps_per_split);
  const int ns = max(0, s_end - s_begin);   // K-steps of this workgroup
  const int last = s_end - 1;
  // steps whose 64 columns all lie inside the contraction (the forward's
  // contraction is a whole number of 64-blocks)
  const int full_steps = (int)(C / GBK);

  if (wave >= 4) {
    // ============================== producers ==============================
    const int ptid = tid - 256;
    // Weight role: the step's tile holds 128 units (64 weights: one row, 64
    // consecutive k); lane pair pb = ptid / 2 shares unit pb, lane ph = ptid %
    // 2 decodes its elements [32 ph, 32 ph + 32).  Forward: unit pb is weight
    // row o0 + pb at k-block st, stage row pb.  Backward: weight row 64 st +
    // pb / 2 at k-block o0 / 64 + pb % 2, stage row pb / 2, columns
    // 64 (pb % 2) + 32 ph.
    const int pb = ptid >> 1, ph = ptid & 1;
    const int wr = DX ? (pb >> 1) : pb;                              // stage row
    const int wc = DX ? 64 * (pb & 1) + 32 * ph : 32 * ph;          // stage column
    struct WRaw {
      u32x4_t c[FMT == kFmtQ8 ? 2 : 1];   // the lane's 32 weights: 16 code bytes, or 32 int8
      uint32_t qbyte;   // NF4 with double quantization: the 8-bit scale; Q8_0: the fp16 scale
      float step;       // NF4: the group's fp32 constant, or the block absmax; uint4: the scale
      float zp;         // uint4: the zero-point
    };
    // This lane's half unit at step st.  Storage position (rows in groups of
    // 16, k-block-major inside a group): forward fp0 + st * fR (fixed row; fR
    // = 16 except in a partial last group), backward st * 64 * nkb plus a
    // fixed part whenever all 64 rows of the step are present.  Positions are
    // taken relative to a per-step base in scalar registers; units outside the
    // weight get an offset past the buffer end, so the hardware returns zeros
    // (scale 0, hence decoded zeros).  Per-unit data at the storage position:
    // CB code bytes and PB parameter bytes (the 8-bit scale with double
    // quantization, whose fp32 constant of flat block b sits at step[b / 256];
    // the fp32 absmax; the uint4 scale and zero-point; the two Q8_0 scales).
    constexpr uint32_t CB = FI::code_bytes, PB = FI::param_bytes;
    constexpr uint32_t kOut = 0x80000000u;
    // NF4 scale entries: block 64 one per unit (its position), block 32 two
    // per unit (2p + half), block 128 one per unit pair, in the row-group order
    // over the k/128 block columns (nkb2); the second-level constant of flat
    // block b is step[b / 256].
    constexpr int BS = FI::block;
    const int64_t nkb2 = nkb / 2;
    const uint32_t hq = (uint32_t)ph;   // block 32: the lane's half is its own block
    const int64_t kb_dx = o0 / kBlock + (pb & 1);
    const int64_t frow = o0 + pb;
    const int64_t fg0 = frow & ~int64_t(15);
    const bool f_ok = frow < N;
    const uint32_t fR = f_ok ? (uint32_t)min(int64_t(16), N - fg0) : 16u;
    const uint32_t f_prel = (uint32_t)((fg0 - o0) * nkb + (frow - fg0));   // fp0 - o0 * nkb
    const uint32_t f_prel2 = (uint32_t)((fg0 - o0) * nkb2 + (frow - fg0));
    const bool d_kok = kb_dx < nkb;
    const uint32_t d_prel = (uint32_t)((wr & ~15) * nkb + kb_dx * 16 + (wr & 15));
    const uint32_t d_prel2 = (uint32_t)((wr & ~15) * nkb2 + (kb_dx >> 1) * 16 + (wr & 15));
    auto sent = [&](uint32_t prel, uint32_t prel2) -> uint32_t {   // scale entry of the lane's unit
      return BS == 64 ? prel : (BS == 32 ? 2 * prel + hq : prel2);
    };
    const uint32_t c_vo0 =
        DX ? (d_kok ? d_prel * CB + ph * (CB / 2) : kOut) : (f_ok ? f_prel * CB + ph * (CB / 2) : kOut);
    const uint32_t p_vo0 =
        DX ? (d_kok ? sent(d_prel, d_prel2) * PB : kOut) : (f_ok ? sent(f_prel, f_prel2) * PB : kOut);
    const uint32_t b_lane = (uint32_t)(BS == 64    ? (DX ? wr * nkb + kb_dx : frow * nkb)
                                       : BS == 32 ? 2 * (DX ? wr * nkb + kb_dx : frow * nkb) + hq
                                                  : (DX ? wr * nkb2 + (kb_dx >> 1) : frow * nkb2));
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
          cvo = ok ? prel * CB + ph * (CB / 2) : kOut;
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
      r.c[0] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(crs, cvo, 0, 0));
      if constexpr (FMT == kFmtQ8) {
        r.c[1] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(crs, cvo + 16, 0, 0));
        // the fp16 scale of the lane's 32-element half
        r.qbyte = __builtin_amdgcn_raw_buffer_load_b16(buf_rsrc(w.qscale + pbase * 4), pvo + 2 * ph, 0, 0);
      } else if constexpr (FI::nf4 && FI::dq) {
        r.qbyte = __builtin_amdgcn_raw_buffer_load_b8(buf_rsrc(w.qscale + sbase), pvo, 0, 0);
        r.step = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(step_rsrc, (bidx >> 8) * 4, 0, 0));
      } else if constexpr (FI::nf4) {
        r.qbyte = 1u;   // scale = 1 * absmax, exact
        r.step = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(buf_rsrc(w.step + sbase), pvo, 0, 0));
      } else {
        // two dword loads (the backend may merge them): a 64-bit buffer load
        // whose halves are bit-cast to float is shrunk to one dword by this
        // compiler, both halves then holding the scale
        const auto prs = buf_rsrc(w.step + 2 * pbase);
        r.step = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(prs, pvo, 0, 0));
        r.zp = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(prs, pvo + 4, 0, 0));
      }
    };
    // vector-memory loads issued per load_w (codes, then the parameters: the
    // Q8_0 scale, the NF4 8-bit scale and group constant, the NF4 absmax, the
    // uint4 pair, counted as one load since the backend may merge its two);
    // the wait below counts them (a count below the real one only waits
    // longer)
    constexpr int kWLoads = FMT == kFmtQ8 ? 3 : ((FI::nf4 && FI::dq) ? 3 : 2);
    // NF4 levels of this lane's table entries: level[8 ph + i] (block 32: all
    // 16, each lane its own table)
    float lv[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) lv[i] = 0.f;
    if constexpr (FI::nf4) {
      if constexpr (BS == 32) {
#pragma unroll
        for (int i = 0; i < 16; ++i) lv[i] = gptr(codebook)[i];
      } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) lv[i] = gptr(codebook)[8 * ph + i];
      }
    }
    // Decode the lane's 32 weights into weight stage `stage`: the 4-bit
    // formats through the unit's table (entries level[c] * s for NF4,
    // (c - zp) * scale for uint4), Q8_0 bytes times the fp16 scale.
    auto decode_to = [&](const WRaw& r, int stage) {
      uint16_t* const sw = sW + stage * G::stage;
      // the lane's four 8-column groups (16 bytes each)
      auto dst = [&](int j) -> u32x4_t& {
        return *reinterpret_cast<u32x4_t*>(sw + G::at(wr, wc + 8 * j));
      };
      if constexpr (FMT == kFmtQ8) {
        const float d = half_bits_to_float(r.qbyte & 0xFFFFu);
        dst(0) = decode_q8x8(r.c[0][0], r.c[0][1], d);
        dst(1) = decode_q8x8(r.c[0][2], r.c[0][3], d);
        dst(2) = decode_q8x8(r.c[1][0], r.c[1][1], d);
        dst(3) = decode_q8x8(r.c[1][2], r.c[1][3], d);
      } else {
        Lut t;
        if constexpr (FMT == kFmtU4) {
          const int zp = (int)r.zp;   // c - zp formed as an integer: +0 at c == zp
          float lvr[8];
#pragma unroll
          for (int i = 0; i < 8; ++i) lvr[i] = (float)(8 * ph + i - zp);
          t = make_lut_pair(lvr, r.step);
        } else if constexpr (BS == 32) {
          t = make_lut(lv, (float)r.qbyte * r.step);
        } else {
          t = make_lut_pair<FI::f16>(lv, (float)r.qbyte * r.step);
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) dst(j) = decode8(t, r.c[0][j]);
      }
    };

    if (ns > 0) {
      // Weight stages: step s in stage s % 3, decoded two steps ahead, so
      // that a step's LDS writes have a whole iteration to complete (they
      // queue behind the consumers' fragment reads) before the barrier that
      // hands the step over.  Codes ring of kRing steps: the codes of step s
      // in rw[(s - s_begin) % kRing], loaded kRing - 2 iterations before
      // their decode (under full load the loads take more than two steps to
      // return).
      constexpr int kRing = 6;
      WRaw rw[kRing];
#pragma unroll
      for (int j = 0; j < kRing; ++j) load_w(min(s_begin + j, last), rw[j]);
      QL_VMCNT((kRing - 1) * kWLoads);
      decode_to(rw[0], 0);
      QL_VMCNT((kRing - 2) * kWLoads);
      if (ns > 1) decode_to(rw[1], 1);
      k_barrier();
      // Iteration t (between barriers t and t+1): codes of step t+kRing into
      // the ring slot of step t (decoded two iterations ago), then, once the
      // codes of step t+2 have landed, decode it into stage (t+2) % 3 (the
      // stage of step t-1, whose reads finished before barrier t); at the
      // barrier only this iteration's 4 writes may still be in flight (step
      // t+2 is read after barrier t+2).  Steps past the end re-load the last
      // one (never decoded).  (Fenced: left free, the scheduler pulls the
      // next iterations' scale arithmetic into this decode, which then waits
      // for their loads.)
      auto iter = [&](int t, auto PHc) {
        constexpr int PH = decltype(PHc)::value;   // t % kRing
        __builtin_amdgcn_sched_barrier(0);
        load_w(min(s_begin + t + kRing, last), rw[PH]);
        __builtin_amdgcn_sched_barrier(0);
        QL_VMCNT((kRing - 2) * kWLoads);
        if (t + 2 < ns) decode_to(rw[(PH + 2) % kRing], (t + 2) % 3);
        __builtin_amdgcn_sched_barrier(0);
        k_barrier_lgkm4();
      };
      using P0 = std::integral_constant<int, 0>;
      using P1 = std::integral_constant<int, 1>;
      using P2 = std::integral_constant<int, 2>;
      using P3 = std::integral_constant<int, 3>;
      using P4 = std::integral_constant<int, 4>;
      using P5 = std::integral_constant<int, 5>;
      int t = 0;
      for (; t + kRing - 1 < ns; t += kRing) {
        iter(t, P0{});
        iter(t + 1, P1{});
        iter(t + 2, P2{});
        iter(t + 3, P3{});
        iter(t + 4, P4{});
        iter(t + 5, P5{});
      }
      if (t < ns) iter(t, P0{});
      if (t + 1 < ns) iter(t + 1, P1{});
      if (t + 2 < ns) iter(t + 2, P2{});
      if (t + 3 < ns) iter(t + 3, P3{});
      if (t + 4 < ns) iter(t + 4, P4{});
      k_barrier();   // the consumers' epilogue
    }
    // backward: the adapter-gradient reduction handed to this launch, in
    // global memory only (the consumers are storing the output meanwhile)
    if constexpr (DX) {
      if (fold.msplit > 1) fold_wgrad(fold, (int64_t)blockIdx.x * 256 + ptid, (int64_t)gridDim.x * 256);
    }
    return;
  }

  // ================================ consumers ================================
  const int cw = wave;
  // Wave tile: in the forward each consumer takes 64 rows x the 128 columns
  // of the tile; in the backward 128 rows x 64 columns (two waves per row
  // block), which costs 8 LDS reads per 16-deep slice (2 x 2 transposing
  // reads + 4) instead of 10, so two slices in flight stay close to the 15
  // LDS operations a wave can have outstanding (past that, issue stalls).
  constexpr int WM = DX ? 128 : 64, WN = DX ? 64 : 128;
  constexpr int MT = WM / 32, NT = WN / 32;         // 32 x 32 MFMA tiles
  const int wr0 = DX ? 128 * (cw >> 1) : 64 * cw;   // first tile row of the wave
  const int wc0 = DX ? 64 * (cw & 1) : 0;           // first tile column
  // Activation tile of step st into ring stage `stage`: each consumer moves
  // rows [64 cw, 64 cw + 64) (read after the step barrier, also by the other
  // wave of its row block in the backward) with 8 DMA
  // loads of 8 rows, issued between its MFMAs; lane l lands at byte 16 l of
  // its load's 1 KiB, i.e. row l / 8, physical chunk l % 8.  With 16-byte
  // rows (VEC) the loads are buffer loads whose resource ends at the end of
  // the activation matrix, so rows past M read as zeros; the address is a
  // per-step base in scalar registers, a scalar row offset and one of two
  // per-lane offsets (the chunk swizzle repeats every two loads).  In a
  // ragged last step (backward, n % 64 != 0) a lane whose piece lies past
  // the contraction takes an offset past any resource (zeros), selected
  // without a branch.  Without 16-byte rows the loads go through
  // registers with zero fill, rows past M clamped to row M-1 (their products
  // are discarded).  (Loading the MFMA fragments straight into
  // registers instead was measured slower: each such load touches 32 rows.)
  uint32_t a_vo[2], a_vo_last[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int rl = cw * 64 + i * 8 + (lane >> 3);
    const int lc = a_chunk(rl, lane & 7);
    a_vo[i] = (uint32_t)((rl * C + lc * 8) * 2);
    a_vo_last[i] = (int64_t)full_steps * GBK + lc * 8 < C ? a_vo[i] : 0x80000000u;
  }
  const uint16_t* a_tile = act + m0 * C;
  const int64_t a_bytes = (M - m0) * C * 2;   // from the tile's first row to the matrix end
  auto fill_a_one = [&](int st, int stage, int i) {
    const int64_t c0 = (int64_t)st * GBK;
    uint16_t* dst = sA + stage * A_STAGE + (cw * 64 + i * 8) * GBK;
    const int rl = cw * 64 + i * 8 + (lane >> 3);
    const int lc = a_chunk(rl, lane & 7);
    const int a_so = (i >> 1) * 16 * (int)C * 2;   // rows 16 (i / 2) further
    if (VEC) {
      if (!DX) {
        __builtin_amdgcn_raw_ptr_buffer_load_lds(buf_rsrc(a_tile + c0, rsrc_bytes(a_bytes - c0 * 2)),
                                                 (QL_LDS void*)dst, 16, a_vo[i & 1], a_so, 0, 0);
      } else {
        // The backward reads its weight fragments with ds_read_b64_tr_b16,
        // which the compiler cannot tell apart from the DMA's LDS target: it
        // would wait for every DMA in flight before each of those reads.  The
        // DMA is therefore issued as inline assembly, which the compiler does
        // not track (it sets M0, which nothing else in this loop uses); the
        // explicit vmcnt waits of the K loop count these loads.
        const uint32_t lds_addr = (uint32_t)(uintptr_t)(QL_LDS void*)dst;
        const auto rs = buf_rsrc(a_tile + c0, rsrc_bytes(a_bytes - c0 * 2));
        const uint32_t vo = st < full_steps ? a_vo[i & 1] : a_vo_last[i & 1];
        asm volatile("s_mov_b32 m0, %1\n\tbuffer_load_dwordx4 %0, %2, %3 offen lds"
                     :: "v"(vo), "s"(lds_addr), "s"(rs), "s"(a_so) : "memory", "m0");
      }
    } else {
      const int64_t row = min(m0 + rl, M - 1);
      const int64_t c = c0 + lc * 8;
      const u32x4_t v = c < C ? load_act8(act + row * C, c, C, false) : u32x4_t{0u, 0u, 0u, 0u};
      *reinterpret_cast<u32x4_t*>(dst + lane * 8) = v;
    }
  };

  f32x16_t acc[NT][MT];    // [column tile nt][row tile mt]: D[n][m]
#pragma unroll
  for (int nt = 0; nt < NT; ++nt)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[nt][mt][i] = 0.f;

  if (ns > 0) {
    // fragments of one 16-deep contraction slice, three buffers: slice kk of
    // step t lives in slot (t + kk) % 3 (4 slices per step), read two slices
    // before its MFMAs.  The backward without 16-byte activation rows, whose
    // register-path loads need more registers, keeps two.
    constexpr bool kTwoSlots = DX && !VEC;
    constexpr int NS = kTwoSlots ? 2 : 3;
    u32x4_t wf[NS][NT], xf[NS][MT];
    // fragment f of slice kk of step t into slot b: f < MT the activation
    // rows of row tile f, else the weight fragment of column tile f - MT
    auto read_one = [&](int t, int kk, auto SLc, int f) {
      constexpr int b = decltype(SLc)::value;
      if (f < MT) {
        const uint16_t* sa = sA + (t % NA) * A_STAGE;
        const int r = wr0 + 32 * f + lr;
        xf[b][f] = *reinterpret_cast<const u32x4_t*>(sa + r * GBK + a_chunk(r, 2 * kk + lg) * 8);
      } else {
        const int nt = f - MT;
        const uint16_t* sw = sW + (t % 3) * G::stage;
        if (DX) {
          const int G16 = lane >> 4, i16 = lane & 15;
          const int row = 16 * kk + 8 * (G16 >> 1) + (i16 >> 2);
          const int col = wc0 + 32 * nt + 16 * (G16 & 1) + 4 * (i16 & 3);
          const u32x2_t lo = ds_tr16(sw + G::at(row, col));
          const u32x2_t hi = ds_tr16(sw + G::at(row + 4, col));
          wf[b][nt] = u32x4_t{lo[0], lo[1], hi[0], hi[1]};
        } else {
          wf[b][nt] = *reinterpret_cast<const u32x4_t*>(sw + (wc0 + 32 * nt + lr) * G::ld + 16 * kk + 8 * lg);
        }
      }
    };
    auto read = [&](int t, int kk, auto SLc) {
#pragma unroll
      for (int f = 0; f < MT + NT; ++f) read_one(t, kk, SLc, f);
    };
    // 8 MFMAs of slice kk from slot b; after the 4th and the 8th, DMA loads
    // 2 kk and 2 kk + 1 of the activation tile of step sa into ring stage
    // `stage`
    auto mma = [&](auto SLc, int kk, int sa, int stage) {
      constexpr int b = decltype(SLc)::value;
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          acc[nt][mt] = mfma32<FI::f16>(wf[b][nt], xf[b][mt], acc[nt][mt]);
          const int q = nt * MT + mt;
          if ((q & 3) == 3) {
            __builtin_amdgcn_sched_barrier(0);
            fill_a_one(sa, stage, 2 * kk + (q >> 2));
            __builtin_amdgcn_sched_barrier(0);
          }
        }
      }
    };
    // The same 8 MFMAs in a fixed order with one fragment read of slice rkk
    // of step rt (into slot rs) after each of the first MT + NT: the reads
    // then leave one by one between the MFMAs instead of as a burst that can
    // fill the LDS queue and hold up the MFMAs behind it (a wave issues in
    // order).
    auto slice = [&](auto SLc, int kk, int sa, int stage, int rt, int rkk, auto RSc) {
      constexpr int b = decltype(SLc)::value;
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const int nt = q / MT, mt = q % MT;
        acc[nt][mt] = mfma32<FI::f16>(wf[b][nt], xf[b][mt], acc[nt][mt]);
        __builtin_amdgcn_sched_barrier(0);
        if (q < MT + NT) read_one(rt, rkk, RSc, q);
        __builtin_amdgcn_sched_barrier(0);
        if ((q & 3) == 3) {
          fill_a_one(sa, stage, 2 * kk + (q >> 2));
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    };
    using S0 = std::integral_constant<int, 0>;
    using S1 = std::integral_constant<int, 1>;
    using S2 = std::integral_constant<int, 2>;
    // prologue: activations of the first two steps (this wave's rows)
    for (int i = 0; i < 8; ++i) fill_a_one(s_begin, 0, i);
    for (int i = 0; i < 8; ++i) fill_a_one(min(s_begin + 1, last), 1, i);
    QL_VMCNT(VEC ? 8 : 0);   // step 0's rows have landed
    k_barrier();             // weight stage 0 ready
    read(0, 0, S0{});
    if constexpr (!kTwoSlots) read(0, 1, S1{});
    // Iteration t (P = t % 3): slices 0-3 of step t from slots P, P+1, P+2,
    // P, with the DMA of step t+2's activation rows (ring stage (t+2) % 3,
    // last read before the previous barrier) spread over the MFMAs.  Slices
    // 0 and 1 read slices 2 and 3 of step t; the barrier follows (every read
    // of weight stage t and of step t's rows has been issued, and this
    // wave's rows of step t+1, issued in iteration t-1, have landed: only
    // the 4 DMAs of this iteration may still be in flight); slices 2 and 3
    // then read slices 0 and 1 of step t+1.  Past the last step the reads
    // take stale stages and the DMAs re-load the last step (never used).
    auto iter = [&](int t, auto PHc) {
      constexpr int P = decltype(PHc)::value;
      using A = std::integral_constant<int, P>;
      using B = std::integral_constant<int, (P + 1) % 3>;
      using C2 = std::integral_constant<int, (P + 2) % 3>;
      const int sa = min(s_begin + t + 2, last), stage = (t + 2) % NA;
      __builtin_amdgcn_sched_barrier(0);
      slice(A{}, 0, sa, stage, t, 2, C2{});
      slice(B{}, 1, sa, stage, t, 3, A{});
      QL_VMCNT(VEC ? 4 : 0);
      k_barrier();
      __builtin_amdgcn_sched_barrier(0);
      slice(C2{}, 2, sa, stage, t + 1, 0, B{});
      slice(A{}, 3, sa, stage, t + 1, 1, C2{});
      __builtin_amdgcn_sched_barrier(0);
    };
    // Two slots: slice kk in slot kk % 2, read one slice ahead.
    auto iter2 = [&](int t) {
      const int sa = min(s_begin + t + 2, last), stage = (t + 2) % NA;
      __builtin_amdgcn_sched_barrier(0);
      read(t, 1, S1{});
      __builtin_amdgcn_sched_barrier(0);
      mma(S0{}, 0, sa, stage);
      __builtin_amdgcn_sched_barrier(0);
      read(t, 2, S0{});
      __builtin_amdgcn_sched_barrier(0);
      mma(S1{}, 1, sa, stage);
      __builtin_amdgcn_sched_barrier(0);
      read(t, 3, S1{});
      __builtin_amdgcn_sched_barrier(0);
      mma(S0{}, 2, sa, stage);
      __builtin_amdgcn_sched_barrier(0);
      QL_VMCNT(VEC ? 6 : 0);
      k_barrier();
      __builtin_amdgcn_sched_barrier(0);
      if (t + 1 < ns) read(t + 1, 0, S0{});
      __builtin_amdgcn_sched_barrier(0);
      mma(S1{}, 3, sa, stage);
    };
    if constexpr (kTwoSlots) {
      for (int t = 0; t < ns; ++t) iter2(t);
    } else {
      int t = 0;
      for (; t + 2 < ns; t += 3) {
        iter(t, S0{});
        iter(t + 1, S1{});
        iter(t + 2, S2{});
      }
      if (t < ns) iter(t, S0{});
      if (t + 1 < ns) iter(t + 1, S1{});
    }
    // no DMA of this wave may still be writing LDS when the epilogue reuses it
    QL_VMCNT(0);
  }

  // ---- epilogue.  LoRA term (ksplit == 1): out += (scaling * L) R^T on the
  // matrix cores, 16 ranks per MFMA step; the fp32 factor scaling * L is
  // split into 16-bit hi + lo parts so the product keeps fp32 accuracy.  The
  // operands of each 16-rank chunk are fetched without branches (indices
  // clamped into the matrices, values past the rank masked to zero), as
  // 16-byte loads where the layout allows, and the next chunk's fetch is
  // issued before the current chunk's MFMAs.
  if (ksplit == 1 && lora.r > 0) {
    const int r = lora.r;
    int64_t orow[NT], mrow[MT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) orow[nt] = min(o0 + wc0 + 32 * nt + lr, O - 1);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) mrow[mt] = min(m0 + wr0 + 32 * mt + lr, M - 1);
    const bool rvec = lora.rs_j == 1 && r % 8 == 0 && (lora.rs_c % 8) == 0 &&
                      (reinterpret_cast<uintptr_t>(lora.R) & 15) == 0;
    const bool lvec = r % 8 == 0 && (reinterpret_cast<uintptr_t>(lora.L) & 15) == 0;
    struct Ops {
      u32x4_t rb[NT];      // R[o][jb .. jb+7], 16-bit pairs
      f32x4_t lv[MT][2];   // L[m][jb .. jb+7]
    };
    // this lane's ranks of the chunk at j0: jb .. jb+7, jb = j0 + 8 lg
    auto fetch = [&](int j0, Ops& op) {
      const int jb = j0 + 8 * lg;
      const int jc = min(jb, r - 8 > 0 ? r - 8 : 0);   // vector start kept inside the row
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        if (rvec) {
          op.rb[nt] = *reinterpret_cast<const u32x4_t*>(lora.R + orow[nt] * lora.rs_c + jc);
        } else {
          uint32_t h[8];
#pragma unroll
          for (int e = 0; e < 8; ++e)
            h[e] = lora.R[orow[nt] * lora.rs_c + (int64_t)min(jb + e, r - 1) * lora.rs_j];
          op.rb[nt] = u32x4_t{h[0] | h[1] << 16, h[2] | h[3] << 16, h[4] | h[5] << 16, h[6] | h[7] << 16};
        }
      }
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
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
      u32x4_t rb[NT];
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        rb[nt] = op.rb[nt];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const bool k0 = jb + 2 * e < r, k1 = jb + 2 * e + 1 < r;
          rb[nt][e] = (k0 ? rb[nt][e] & 0xFFFFu : 0u) | (k1 ? rb[nt][e] & 0xFFFF0000u : 0u);
        }
      }
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
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
        for (int nt = 0; nt < NT; ++nt) {
          acc[nt][mt] = mfma32<FI::f16>(rb[nt], ahi, acc[nt][mt]);
          acc[nt][mt] = mfma32<FI::f16>(rb[nt], alo, acc[nt][mt]);
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

  // ---- stores.  Lane element i of acc[nt][mt] is output row m = m0 + wr0 +
  // 32 mt + l % 32, column o = o0 + wc0 + 32 nt + 8 (i / 4) + 4 (l / 32) + i % 4.
  // The wave tile goes through LDS (the activation ring, free once the
  // producers have drained their last loads) so that each store instruction
  // writes whole row pieces of the wave tile (WN / 8 lanes x 16 bytes per
  // row), 16-bit output in one pass, fp32 in two passes of 64 x 64.
  // Written once: non-temporal stores leave the L2 to the operand tiles the
  // other workgroups reuse.
  if (ns > 0) k_barrier();   // every wave is done with the stages (DMA drained)
  const bool o8 = (O & 7) == 0;   // 8-column pieces are 16-byte aligned in 16-bit rows
  const bool o4 = (O & 3) == 0;   // 4-column pieces are 16-byte aligned in fp32 rows
  if (ksplit == 1 && out16) {
    // [WM rows][WN + 8] 16-bit per consumer (the row pitch, 4 banks past a
    // multiple of 64, spreads the 8-byte writes of a wave's 32 rows over the
    // banks)
    constexpr int LDO = WN + 8;
    uint16_t* st = sA + cw * WM * LDO;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const u32x2_t pk = {pack16x2<FI::f16>(acc[nt][mt][4 * q], acc[nt][mt][4 * q + 1]),
                              pack16x2<FI::f16>(acc[nt][mt][4 * q + 2], acc[nt][mt][4 * q + 3])};
          *reinterpret_cast<u32x2_t*>(st + (32 * mt + lr) * LDO + 32 * nt + 8 * q + 4 * lg) = pk;
        }
    QL_LGKMCNT0();
    // lane l: row RPI j + l / LPR, columns 8 (l % LPR) .. + 7
    constexpr int LPR = WN / 8, RPI = 64 / LPR;
    uint16_t* outp = reinterpret_cast<uint16_t*>(out);
#pragma unroll
    for (int j = 0; j < WM / RPI; ++j) {
      const int rl = RPI * j + lane / LPR, cl = 8 * (lane % LPR);
      const int64_t m = m0 + wr0 + rl, o = o0 + wc0 + cl;
      const u32x4_t v = *reinterpret_cast<const u32x4_t*>(st + rl * LDO + cl);
      if (m < M) {
        uint16_t* dst = outp + m * O + o;
        if (o8 && o + 7 < O) {
          __builtin_nontemporal_store(v, reinterpret_cast<u32x4_t*>(dst));
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e)
            if (o + e < O) dst[e] = (uint16_t)(e & 1 ? v[e >> 1] >> 16 : v[e >> 1] & 0xFFFFu);
        }
      }
    }
  } else {
    // fp32 (output or split partials): [64 rows][68] floats per consumer and
    // pass; pass p holds column tiles 2 pg, 2 pg + 1 and row tiles 2 pm,
    // 2 pm + 1 of the wave tile (forward: pg = p, pm = 0; backward: pg = 0,
    // pm = p)
    constexpr int LDO = 68;
    float* st = reinterpret_cast<float*>(sA) + cw * 64 * LDO;
    float* base = ksplit > 1 ? part + (int64_t)split * M * O : reinterpret_cast<float*>(out);
#pragma unroll
    for (int pass = 0; pass < 2; ++pass) {
      const int pg = NT == 4 ? pass : 0, pm = MT == 4 ? pass : 0;
      if (pass) QL_LGKMCNT0();   // (the reads of pass 0 are done before the writes of pass 1)
#pragma unroll
      for (int m2 = 0; m2 < 2; ++m2)
#pragma unroll
        for (int n2 = 0; n2 < 2; ++n2)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int nt = 2 * pg + n2, mt = 2 * pm + m2;
            const f32x4_t v = {acc[nt][mt][4 * q], acc[nt][mt][4 * q + 1], acc[nt][mt][4 * q + 2],
                               acc[nt][mt][4 * q + 3]};
            *reinterpret_cast<f32x4_t*>(st + (32 * m2 + lr) * LDO + 32 * n2 + 8 * q + 4 * lg) = v;
          }
      QL_LGKMCNT0();
      // lane l: row 4 j + l / 16, columns 4 (l % 16) .. + 3 of this pass's 64
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const int rl = 4 * j + (lane >> 4), cl = 4 * (lane & 15);
        const int64_t m = m0 + wr0 + 64 * pm + rl, o = o0 + wc0 + 64 * pg + cl;
        const f32x4_t v = *reinterpret_cast<const f32x4_t*>(st + rl * LDO + cl);
        if (m < M) {
          float* dst = base + m * O + o;
          if (o4 && o + 3 < O) {
            __builtin_nontemporal_store(v, reinterpret_cast<f32x4_t*>(dst));
          } else {
#pragma unroll
            for (int e = 0; e < 4; ++e)
              if (o + e < O) dst[e] = v[e];
          }
        }
      }
    }
  }
}


static constexpr size_t smem_bytes() {
  return sizeof(uint16_t) * NA * A_STAGE;   // dynamic part: the activation ring
}

template <bool DX, bool VEC, int FMT>
static hipError_t launch_one(dim3 grid, hipStream_t s, const uint16_t* act, const Nf4View& w,
                             const float* codebook, int64_t M, const LoraTerm& lora, void* out,
                             bool out16, float* part, int ksplit, int per, int64_t mtiles,
                             int64_t otiles, const WgradFold& fold) {
  // the dynamic LDS limit of this instantiation, set once per process (a
  // function-local static is initialized exactly once, thread-safely)
  static const hipError_t attr = hipFuncSetAttribute(
      reinterpret_cast<const void*>(&k_gemm<DX, VEC, FMT>), hipFuncAttributeMaxDynamicSharedMemorySize,
      (int)smem_bytes());
  if (attr != hipSuccess) return attr;
  hipLaunchKernelGGL((k_gemm<DX, VEC, FMT>), grid, dim3(512), smem_bytes(), s, act, w, codebook,
                     M, lora, out, (int)out16, part, ksplit, per, mtiles, otiles, fold);
  return hipGetLastError();
}

template <bool DX, bool VEC>
static hipError_t launch_fmt(dim3 grid, hipStream_t s, const uint16_t* act, const Nf4View& w,
                             const float* codebook, int64_t M, const LoraTerm& lora, void* out,
                             bool out16, float* part, int ksplit, int per, int64_t mtiles,
                             int64_t otiles, const WgradFold& fold) {
#define QL_ONE(F) \
  launch_one<DX, VEC, F>(grid, s, act, w, codebook, M, lora, out, out16, part, ksplit, per, mtiles, \
                         otiles, fold)
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
                         hipStream_t s, const WgradFold& fold) {
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
                                   per, mtiles, otiles, fold);
  }
  return launch_fmt<DX, true>(grid, s, act, w, codebook, M, lora, out, out16, part, ksplit, per,
                              mtiles, otiles, fold);
}

hipError_t launch_gemm_fwd(const Nf4View& w, const float* codebook, const uint16_t* X, int64_t M,
                           const LoraTerm& lora, void* Y, bool y16, float* part, int ksplit,
                           hipStream_t s) {
  return launch<false>(w, codebook, X, M, lora, Y, y16, part, ksplit, s, WgradFold{});
}

hipError_t launch_gemm_dx(const Nf4View& w, const float* codebook, const uint16_t* dY, int64_t M,
                          const LoraTerm& lora, void* dX, bool dx16, float* part, int nsplit,
                          hipStream_t s, const WgradFold* fold) {
  if (fold && fold->msplit > 1 && nsplit != 1) return hipErrorInvalidValue;
  return launch<true>(w, codebook, dY, M, lora, dX, dx16, part, nsplit, s, fold ? *fold : WgradFold{});
}

}  // namespace ql
