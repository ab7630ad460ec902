// Host-side launchers of the HIP kernels (one per kernel family).  Shapes are
// validated by the caller (api.cpp) before any of these runs.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ql {

// Weight formats as the kernels see them (a template parameter of each kernel):
// NF4 with double-quantized (Dq) or single-level scales at block 64, 32 or
// 128, asymmetric uint4, Q8_0; every one computes in bf16 except
// kFmtNf4DqF16, NF4 with double quantization at block 64 whose dequantized
// weight, activations and adapter factors are fp16.
enum WFmt : int {
  kFmtNf4Dq = 0, kFmtNf4 = 1, kFmtU4 = 2, kFmtQ8 = 3,
  kFmtNf4Dq32 = 4, kFmtNf4_32 = 5, kFmtNf4Dq128 = 6, kFmtNf4_128 = 7,
  kFmtNf4DqF16 = 8
};
constexpr int kNumFmt = 9;
inline bool fmt_f16(int fmt) { return fmt == kFmtNf4DqF16; }

// LoRA term added by epilogues:  out[m][c] += scaling * sum_j L[m*r + j] * R[c*rs_c + j*rs_j]
struct LoraTerm {
  const float* L;      // [M x r] fp32 (T in the forward, U in the backward), or nullptr
  const uint16_t* R;   // 16-bit (B [N x r] in the forward, A [r x K] in the backward)
  int64_t rs_c, rs_j;  // strides of R
  int r;
  float scaling;
};

// Packed weight; fmt is a WFmt (common.h) and says what the arrays hold:
//   kFmtNf4Dq  codes, qscale (8-bit), step (fp32 per 256 units)
//   kFmtNf4    codes, step (fp32 absmax per unit); qscale unused
//   kFmtU4     codes, step (fp32 scale, zero-point per unit); qscale unused
//   kFmtQ8     codes (int8), qscale (two fp16 per unit); step unused
struct Nf4View {
  const uint8_t* codes;
  const uint8_t* qscale;
  const float* step;
  int64_t n, k;
  int fmt;
};

// The 16-bit weight W is fp16 for kFmtNf4DqF16, else bf16 (likewise the
// dequantized output).
hipError_t launch_quantize(const uint16_t* W, const float* codebook, uint8_t* codes,
                           uint8_t* qscale, float* step, int64_t n, int64_t k, int fmt,
                           hipStream_t s);
hipError_t launch_dequant(const Nf4View& w, const float* codebook, uint16_t* out, hipStream_t s);
// Copy of a packed weight from the library layout to the plain flat layout
// (to_plain) or back: source arrays sc / sq / ss, destination dc / dq / ds (the
// arrays the format uses; same sizes in both layouts, disjoint buffers).
hipError_t launch_relayout(const uint8_t* sc, const uint8_t* sq, const float* ss, uint8_t* dc,
                           uint8_t* dq, float* ds, int64_t n, int64_t k, int fmt, bool to_plain,
                           hipStream_t s);
// W[n][k] <- rne(W + s * (B A)[n][k]) in place (A [r x k], B [n x r]; all 16-bit,
// fp16 when f16 else bf16; k % 8 == 0, W and A 16-byte aligned).
hipError_t launch_merge(uint16_t* W, const uint16_t* A, const uint16_t* B, int64_t n, int64_t k, int r,
                        float s, bool f16, hipStream_t st);

// Forward base product Y = X deq(W)^T (+ LoRA term), tiled MFMA GEMM.
// ksplit > 1 writes fp32 partials part[ksplit][M][N] and leaves the epilogue
// to launch_reduce.
hipError_t launch_gemm_fwd(const Nf4View& w, const float* codebook, const uint16_t* X, int64_t M,
                           const LoraTerm& lora, void* Y, bool y16, float* part, int ksplit,
                           hipStream_t s);
// One projection of the small-M forward.  rg_begin: first 64-row workgroup of
// this job in a grouped launch (ascending over the job list).
struct GemvJob {
  const uint16_t* X;
  Nf4View w;
  LoraTerm lora;
  void* Y;
  float* part;
  int64_t M;
  int y16;
  int64_t rg_begin;
};

// Forward for small M (<= 64): streaming split-K over the packed weight.
hipError_t launch_gemv_fwd(const Nf4View& w, const float* codebook, const uint16_t* X, int64_t M,
                           const LoraTerm& lora, void* Y, bool y16, float* part, int ksplit,
                           hipStream_t s);
// Grouped small-M forward: one launch over `njobs` device-resident jobs that
// share M and the weight format `fmt` (a WFmt), covering `row_groups` 64-row
// workgroups in total; no split of the contraction.  max_quads: the largest
// k/256 (rounded up) over the jobs.
hipError_t launch_gemv_grouped(const GemvJob* jobs, int njobs, int64_t row_groups, int64_t M,
                               const float* codebook, int64_t max_quads, int fmt, hipStream_t s);
// The reduction of the adapter-gradient partials of launch_wgrad (msplit >
// 1, launched with reduce = false), carried out by another kernel: out of
// job a / b = scaling * (sum of the msplit partials, in split order), the
// partials laid out as launch_wgrad writes them.
struct WgradFold {
  const float* part = nullptr;
  int msplit = 0;   // 0: nothing to add
  int r = 0;
  float scaling = 0.f;
  int64_t ca = 0, cb = 0;   // columns of job a and of job b
  float* out_a = nullptr;
  float* out_b = nullptr;
  int ta = 0, tb = 0;       // their transpose_out
};
// dX = dY deq(W) (+ LoRA term), contraction over n; nsplit > 1 -> partials.
// With a fold (nsplit == 1 only) the producer waves of the workgroups also
// carry out that reduction once their K loop is over.
hipError_t launch_gemm_dx(const Nf4View& w, const float* codebook, const uint16_t* dY, int64_t M,
                          const LoraTerm& lora, void* dX, bool dx16, float* part, int nsplit,
                          hipStream_t s, const WgradFold* fold = nullptr);
// Small-M input gradient (M <= 32): dX = dY deq(W) (+ LoRA term) with the
// weight streamed once.  Workgroups run over the k/64 blocks x nsplit splits
// of the rows; nsplit must be gemv_dx_splits(w.n, w.k), and when it is above
// 1, `part` holds nsplit * M * w.k floats for launch_reduce (which then adds
// the LoRA term).
inline int gemv_dx_splits(int64_t N, int64_t K) {
  // about 512 workgroups (one per k-block and split), each split a whole
  // number of 256-row iterations and none empty
  const int64_t nkb = K / 64, niter = (N + 255) / 256;   // 64-wide k-blocks
  int64_t ns0 = (512 + nkb - 1) / nkb;
  ns0 = ns0 < 1 ? 1 : (ns0 > niter ? niter : ns0);
  const int64_t iters = (niter + ns0 - 1) / ns0;
  return (int)((niter + iters - 1) / iters);
}
hipError_t launch_gemv_dx(const Nf4View& w, const float* codebook, const uint16_t* dY, int64_t M,
                          const LoraTerm& lora, void* dX, bool dx16, float* part, int nsplit,
                          hipStream_t s);
// A rank projection formed where it is used: row m of L = P Q^T,
// L[m][j] = sum_{c < C} P[m][c] Q[j qs_j + c qs_c] (T = X A^T: Q = A, qs_j =
// C, qs_c = 1; U = dY B: Q = B, qs_j = 1, qs_c = r).  Used when rank_row_ok.
struct RankRow {
  const uint16_t* P = nullptr;   // [M x C]
  const uint16_t* Q = nullptr;
  int64_t qs_j = 0, qs_c = 0;
  int r = 0;
  int64_t C = 0;                 // contraction length
  float* out = nullptr;          // [M x r], written when given
};
// Ranks in whole 16-byte pieces up to 64; 16-byte aligned P and Q with C % 8
// == 0; at least 256 output columns (a reduce workgroup then spans at most two
// rows).
inline bool rank_row_ok(int r, int64_t C, const void* P, const void* Q, int64_t out_cols) {
  return r > 0 && r % 8 == 0 && r <= 64 && C % 8 == 0 && out_cols >= 256 &&
         (reinterpret_cast<uintptr_t>(P) & 15) == 0 && (reinterpret_cast<uintptr_t>(Q) & 15) == 0;
}
// out[m][c] = sum_s part[s][m][c] + LoRA term, for C columns (R and a 16-bit
// out in fp16 when f16, else bf16).
hipError_t launch_reduce(const float* part, int nsplit, int64_t M, int64_t C,
                         const LoraTerm& lora, void* out, bool out16, bool f16, hipStream_t s);
// The same with the LoRA factor rows formed in the kernel from `rank`
// (lora.L unused; rank_row_ok must hold with C output columns) and written to
// rank.out when given.
hipError_t launch_reduce_rows(const float* part, int nsplit, int64_t M, int64_t C,
                              const LoraTerm& lora, void* out, bool out16, bool f16, hipStream_t s,
                              const RankRow& rank);
// rank->out = P Q^T for all M rows, each row formed exactly as launch_reduce
// forms it (one workgroup per row).
hipError_t launch_rank_rows(const RankRow& rank, int64_t M, bool f16, hipStream_t s);

// Rank projection plan.  For M >= 512 and 16 < r <= 64 (and 16-byte rows)
// the projection runs on 128-row tiles with the contraction split so that
// about 256 workgroups run; rowdot_splits() is the number of splits (each
// needing M * r floats of partials when > 1; the launcher and the workspace
// sizing both use it).  At r <= 16 the rank factor is small enough that the
// single-pass kernel, which needs no partials, is faster -- unless the rank
// factor is given transposed (qt: read in place on the split path instead
// of being transposed by a launch of its own).
inline bool rowdot_uses_split_path(int64_t M, int r, bool qt = false) {
  return M >= 512 && (r > 16 || qt) && r <= 64;
}
inline int rowdot_splits(int64_t M, int64_t C, int r, bool qt = false) {
  if (!rowdot_uses_split_path(M, r, qt)) return 1;
  const int64_t ch = r <= 32 ? 256 : 128;
  const int64_t tiles = (M + 127) / 128, chunks = (C + ch - 1) / ch;
  int64_t want = (256 + tiles - 1) / tiles;
  if (want > chunks) want = chunks;
  if (want < 1) want = 1;
  const int64_t per = (chunks + want - 1) / want;
  return (int)((chunks + per - 1) / per);
}
// out[m][j] = sum_c P[m][c] * Q[j][c]   (P [M x C], Q [r x C], both fp16 when
// f16 else bf16; out fp32 [M x r]);
// `part` holds rowdot_splits(M, C, r) * M * r floats when that is above 1.
hipError_t launch_rowdot(const uint16_t* P, const uint16_t* Q, int64_t M, int64_t C, int r,
                         float* out, float* part, bool f16, hipStream_t s);
// The same product with Q given transposed, Qs [C x r] row-major (Q[j][c] =
// Qs[c][j]), on the split path (rowdot_t_supported: rowdot_uses_split_path
// with qt, r % 8 == 0, C % 8 == 0, P and Qs 16-byte aligned): each staged
// chunk of Qs is transposed on its way into LDS, so no transposed copy is
// made.  `part` must be given when rowdot_splits(M, C, r, true) > 1.
inline bool rowdot_t_supported(const uint16_t* P, const uint16_t* Qs, int64_t M, int64_t C, int r) {
  return rowdot_uses_split_path(M, r, true) && r % 8 == 0 && C % 8 == 0 &&
         (reinterpret_cast<uintptr_t>(P) & 15) == 0 && (reinterpret_cast<uintptr_t>(Qs) & 15) == 0;
}
hipError_t launch_rowdot_t(const uint16_t* P, const uint16_t* Qs, int64_t M, int64_t C, int r,
                           float* out, float* part, bool f16, hipStream_t s);
// One product of the grouped rowdot: out[m][j] = sum_c P[m][c] Q[j][c].
struct RowdotJob {
  const uint16_t* P;
  const uint16_t* Q;
  float* out;
  int64_t C;
  int r;
};
// All jobs share M and the 16-bit type; max_r is the largest r among them.
hipError_t launch_rowdot_grouped(const RowdotJob* jobs, int njobs, int64_t M, int max_r,
                                 bool f16, hipStream_t s);
// Qt[j][n] = Q[n][j] for a 16-bit [N x r] matrix.
hipError_t launch_transpose_bf16(const uint16_t* Q, int64_t N, int r, uint16_t* Qt, hipStream_t s);
// One weight gradient of the adapter: out = scaling * sum_m Q[m][j] * P[m][c]
// (P [M x C] fp16 when f16 else bf16, Q fp32 [M x r]); written as out[j][c]
// (transpose_out 0, [r x C]) or out[c][j] (1, [C x r]).
struct WgradJob {
  const uint16_t* P;
  const float* Q;
  int64_t C;
  float* out;
  int transpose_out;
};
// Both gradients of a backward (a: dA, b: dB) in one launch, plus one
// reduction launch when msplit > 1 (`part`: msplit * r * (a.C + b.C) floats)
// unless reduce is false (a WgradFold then adds the partials).
hipError_t launch_wgrad(const WgradJob& a, const WgradJob& b, int64_t M, int r, float scaling,
                        float* part, int msplit, bool f16, hipStream_t s, bool reduce = true);

// Scratch of the allocation-free forward: a file-scope device array of
// kScratchBytes per GPU.  device_scratch() returns its device address on the
// current device (looked up once per device, thread-safe).
constexpr size_t kScratchBytes = size_t(64) << 20;
hipError_t device_scratch(void** ptr);

}  // namespace ql
