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
//  * 256 x 128 output tile per workgroup, 4 waves; wave w owns rows
//    [64w, 64w+64) and all 128 columns: 2 x 4 MFMA 32x32x16 bf16 tiles with
//    fp32 accumulators (128 per lane).
//  * The activation operand (X or dY) streams global -> registers directly in
//    the MFMA A layout, one K-step ahead; it never touches LDS.
//  * The weight tile of each K-step (128 x 64 weights = 128 NF4 blocks) is
//    decoded by all 256 threads, half a block each, into a double-buffered LDS
//    stage; the decode of step s+1 overlaps the MFMAs of step s, one barrier
//    per step.  Decoding is amortized over 256 output rows.
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
  // LDS stage of one K-step of the weight, bf16, [rows][cols + 8]
  static constexpr int rows = DX ? GBK : GBN;    // n (dx: contraction) or n (fwd: output)
  static constexpr int cols = DX ? GBN : GBK;    // k
  static constexpr int ld = cols + 8;
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

template <bool DX>
__global__ __launch_bounds__(256) void k_gemm(const uint16_t* __restrict__ act, Nf4View w,
                                              const float* __restrict__ codebook, int64_t M,
                                              LoraTerm lora, void* __restrict__ out, int out_bf16,
                                              float* __restrict__ part, int ksplit,
                                              int steps_per_split, int64_t mtiles, int64_t otiles) {
  using G = Geo<DX>;
  __shared__ __attribute__((aligned(16))) uint16_t sW[2][G::stage];
  __shared__ float s_lv[16];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
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

  // ---- per-thread roles
  const bool vec = DX ? (N % 8) == 0 : true;
  const int64_t arow0 = m0 + wave * 64 + lr;                // + 32*mt
  // weight decode role: half a 64-block
  const int half = tid & 1;
  const int wr = DX ? (tid >> 2) : (tid >> 1);              // stage row
  const int wcb = DX ? ((tid >> 1) & 1) : 0;                // block within the stage row (dx)

  auto load_a = [&](int st, u32x4_t (&a)[4][2]) {
    const int64_t c0 = (int64_t)st * GBK;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) {
        const int64_t row = arow0 + 32 * mt, c = c0 + 16 * kk + 8 * lg;
        a[kk][mt] = (row < M && c < C) ? load_act8(act + row * C, c, C, vec && c + 8 <= C)
                                       : u32x4_t{0u, 0u, 0u, 0u};
      }
  };
  auto load_w = [&](int st, u32x4_t& codes, float& sc) {
    int64_t n, kb;
    if (DX) {
      n = (int64_t)st * GBK + wr;
      kb = o0 / kBlock + wcb;
    } else {
      n = o0 + wr;
      kb = st;
    }
    if (n < N && kb < nkb) {
      const int64_t b = n * nkb + kb;
      codes = *reinterpret_cast<const u32x4_t*>(w.codes + b * 32 + half * 16);
      sc = block_scale(w.qscale, w.step, b);
    } else {
      codes = u32x4_t{0u, 0u, 0u, 0u};
      sc = 0.f;
    }
  };
  __syncthreads();
  float lv[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) lv[i] = s_lv[i];
  auto decode_w = [&](int stage, const u32x4_t codes, float sc) {
    const Lut t = make_lut(lv, sc);
    uint16_t* base = &sW[stage][wr * G::ld + wcb * 64 + half * 32];
    u32x4_t* dst = reinterpret_cast<u32x4_t*>(base);
#pragma unroll
    for (int j = 0; j < 4; ++j) dst[j] = decode8(t, codes[j]);
  };

  f32x16_t acc[2][4];
#pragma unroll
  for (int mt = 0; mt < 2; ++mt)
#pragma unroll
    for (int nt = 0; nt < 4; ++nt)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[mt][nt][i] = 0.f;

  if (s_begin < s_end) {
    u32x4_t acur[4][2], anext[4][2];
    u32x4_t wc, wc_next = {0u, 0u, 0u, 0u};
    float ws, ws_next = 0.f;
    load_w(s_begin, wc, ws);
    load_a(s_begin, acur);
    decode_w(0, wc, ws);
    if (s_begin + 1 < s_end) load_w(s_begin + 1, wc, ws);
    __syncthreads();

    for (int st = s_begin; st < s_end; ++st) {
      const int stage = (st - s_begin) & 1;
      const bool more = st + 1 < s_end;
      if (more) load_a(st + 1, anext);
      if (st + 2 < s_end) load_w(st + 2, wc_next, ws_next);
      const uint16_t* sw = sW[stage];
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        u32x4_t b[4];
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) {
          if (DX) {
            const int G16 = lane >> 4, i16 = lane & 15;
            const int row = 16 * kk + 8 * (G16 >> 1) + (i16 >> 2);
            const int col = 32 * nt + 16 * (G16 & 1) + 4 * (i16 & 3);
            const u32x2_t lo = ds_tr16(sw + row * G::ld + col);
            const u32x2_t hi = ds_tr16(sw + (row + 4) * G::ld + col);
            b[nt] = u32x4_t{lo[0], lo[1], hi[0], hi[1]};
          } else {
            b[nt] = *reinterpret_cast<const u32x4_t*>(sw + (32 * nt + lr) * G::ld + 16 * kk + 8 * lg);
          }
        }
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
          for (int nt = 0; nt < 4; ++nt) acc[mt][nt] = mfma32(acur[kk][mt], b[nt], acc[mt][nt]);
      }
      if (more) decode_w(stage ^ 1, wc, ws);
      __syncthreads();
      if (more) {
#pragma unroll
        for (int kk = 0; kk < 4; ++kk)
#pragma unroll
          for (int mt = 0; mt < 2; ++mt) acur[kk][mt] = anext[kk][mt];
        wc = wc_next;
        ws = ws_next;
      }
    }
  }

  // ---- epilogue
#pragma unroll
  for (int mt = 0; mt < 2; ++mt)
#pragma unroll
    for (int nt = 0; nt < 4; ++nt)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int64_t m = m0 + wave * 64 + 32 * mt + 8 * (i >> 2) + 4 * lg + (i & 3);
        const int64_t o = o0 + 32 * nt + lr;
        if (m < M && o < O) {
          float v = acc[mt][nt][i];
          if (ksplit > 1) {
            part[((int64_t)split * M + m) * O + o] = v;
          } else {
            if (lora.r > 0) v += lora.scaling * lora_dot_g(lora, m, o);
            if (out_bf16)
              reinterpret_cast<uint16_t*>(out)[m * O + o] = to_bf16(v);
            else
              reinterpret_cast<float*>(out)[m * O + o] = v;
          }
        }
      }
}

template <bool DX>
static hipError_t launch(const Nf4View& w, const float* codebook, const uint16_t* act, int64_t M,
                         const LoraTerm& lora, void* out, bool bf16, float* part, int ksplit,
                         hipStream_t s) {
  const int64_t C = DX ? w.n : w.k, O = DX ? w.k : w.n;
  const int nsteps = (int)((C + GBK - 1) / GBK);
  const int per = (nsteps + ksplit - 1) / ksplit;
  const int64_t mtiles = (M + GBM - 1) / GBM, otiles = (O + GBN - 1) / GBN;
  const int64_t total = mtiles * otiles * ksplit;
  hipLaunchKernelGGL(k_gemm<DX>, dim3((unsigned)total), dim3(256), 0, s, act, w, codebook, M, lora,
                     out, (int)bf16, part, ksplit, per, mtiles, otiles);
  return hipGetLastError();
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
