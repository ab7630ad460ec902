// Host-only check of the C ABI's validation and workspace layout, built with
// AddressSanitizer and UndefinedBehaviorSanitizer (g++, no GPU, no HIP runtime).
//
// The library's host code (api.cpp) is compiled unchanged and linked against
// the stub launchers below instead of the HIP kernels.  Device pointers are
// fake addresses from a registry of "allocations"; they are never
// dereferenced.  Every stub checks that each buffer it is handed, with the
// extent the launch would touch, lies inside one registered allocation (the
// caller's tensors or its workspace of exactly qlora_workspace_bytes()), so a
// wrong workspace offset or size shows up as a failure here.  Any sanitizer
// report aborts the run (built with -fno-sanitize-recover).
#include <cstdint>
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "../../include/qlora_nf4.h"
#include "../../qlora_fine_tuning_nf4_amd/csrc/kernels.h"

namespace ql {
extern void* g_scratch_base;   // the stub scratch (re-registered after each reset)
}

namespace {

struct Alloc {
  uintptr_t base;
  size_t bytes;
};
std::vector<Alloc> g_allocs;
uintptr_t g_next = 0x100000000000ull;
int g_fail = 0;
int g_launches = 0;
int g_relayouts = 0;   // plain-layout conversions launched
int g_folds = 0;       // dX GEMMs that add the adapter-gradient partials
int g_rank_rows = 0;   // split reduces that form the LoRA factor rows themselves
int g_unreduced = 0;   // adapter-gradient launches that leave their partials to a fold

void* fake_alloc(size_t bytes) {
  const uintptr_t b = g_next;
  g_next += (bytes + 0xFFFFF) & ~uintptr_t(0xFFFF);   // 64 KiB aligned, with a gap after
  g_next += 0x10000;
  g_allocs.push_back({b, bytes});
  return reinterpret_cast<void*>(b);
}
void reset_allocs() { g_allocs.clear(); }

void fail(const char* what, const char* file, int line) {
  std::fprintf(stderr, "FAIL %s:%d: %s\n", file, line, what);
  ++g_fail;
}
#define CHECK(c) ((c) ? (void)0 : fail(#c, __FILE__, __LINE__))

// [p, p + bytes) must lie inside one allocation (bytes == 0: nothing touched)
void in_bounds(const void* p, double bytes, const char* name) {
  if (bytes <= 0) return;
  const uintptr_t a = reinterpret_cast<uintptr_t>(p);
  for (const Alloc& al : g_allocs)
    if (a >= al.base && a + (uintptr_t)bytes <= al.base + al.bytes) return;
  std::fprintf(stderr, "FAIL buffer %s [%#lx, +%.0f) outside every allocation\n", name,
               (unsigned long)a, bytes);
  ++g_fail;
}

size_t code_bytes(const ql::Nf4View& w) {
  return (size_t)(w.fmt == ql::kFmtQ8 ? w.n * w.k : w.n * w.k / 2);
}
void check_view(const ql::Nf4View& w) {
  in_bounds(w.codes, (double)code_bytes(w), "codes");
}
void check_lora(const ql::LoraTerm& l, int64_t M, int64_t C, bool l_needed = true) {
  if (l.r == 0) return;
  if (l_needed) in_bounds(l.L, 4.0 * M * l.r, "lora.L");
  // R is [C x r] (stride rs_c) or [r x C] (stride rs_j)
  in_bounds(l.R, 2.0 * ((C - 1) * l.rs_c + (l.r - 1) * l.rs_j + 1), "lora.R");
}

}  // namespace

// ---- stub launchers (same signatures as kernels.h) ----
namespace ql {
hipError_t launch_quantize(const uint16_t* W, const float*, uint8_t* codes, uint8_t*, float*, int64_t n,
                           int64_t k, int fmt, hipStream_t) {
  ++g_launches;
  in_bounds(W, 2.0 * n * k, "W");
  in_bounds(codes, fmt == kFmtQ8 ? 1.0 * n * k : 0.5 * n * k, "codes");
  return hipSuccess;
}
hipError_t launch_dequant(const Nf4View& w, const float*, uint16_t* out, hipStream_t) {
  ++g_launches;
  check_view(w);
  in_bounds(out, 2.0 * w.n * w.k, "dequant out");
  return hipSuccess;
}
hipError_t launch_relayout(const uint8_t* sc, const uint8_t* sq, const float* ss, uint8_t* dc,
                           uint8_t* dq, float* ds, int64_t n, int64_t k, int fmt, bool, hipStream_t) {
  ++g_launches;
  ++g_relayouts;
  const double units = (double)n * (k / 64);
  const double cb = fmt == kFmtQ8 ? 64.0 : 32.0;
  in_bounds(sc, cb * units, "relayout src codes");
  in_bounds(dc, cb * units, "relayout dst codes");
  // the per-unit constants each format keeps, in bytes (qscale / step)
  double qb = 0, sb = 0, groups = 0;
  switch (fmt) {
    case kFmtNf4Dq: case kFmtNf4DqF16: qb = units; groups = n * k / 64; break;
    case kFmtNf4Dq32: qb = 2 * units; groups = n * k / 32; break;
    case kFmtNf4Dq128: qb = units / 2; groups = n * k / 128; break;
    case kFmtNf4: sb = 4 * units; break;
    case kFmtNf4_32: case kFmtU4: sb = 8 * units; break;
    case kFmtNf4_128: sb = 2 * units; break;
    case kFmtQ8: qb = 4 * units; break;
    default: CHECK(false);
  }
  if (groups > 0) sb = 4.0 * std::ceil(groups / 256.0);
  CHECK((qb > 0) == (sq != nullptr) && (qb > 0) == (dq != nullptr));
  CHECK((sb > 0) == (ss != nullptr) && (sb > 0) == (ds != nullptr));
  if (qb > 0) { in_bounds(sq, qb, "relayout src qscale"); in_bounds(dq, qb, "relayout dst qscale"); }
  if (sb > 0) { in_bounds(ss, sb, "relayout src step"); in_bounds(ds, sb, "relayout dst step"); }
  return hipSuccess;
}
hipError_t launch_merge(uint16_t* W, const uint16_t* A, const uint16_t* B, int64_t n, int64_t k, int r,
                        float, bool, hipStream_t) {
  ++g_launches;
  in_bounds(W, 2.0 * n * k, "merge W");
  in_bounds(A, 2.0 * r * k, "merge A");
  in_bounds(B, 2.0 * n * r, "merge B");
  return hipSuccess;
}
hipError_t launch_gemm_fwd(const Nf4View& w, const float*, const uint16_t* X, int64_t M,
                           const LoraTerm& lora, void* Y, bool y16, float* part, int ksplit,
                           hipStream_t) {
  ++g_launches;
  check_view(w);
  in_bounds(X, 2.0 * M * w.k, "X");
  if (ksplit > 1) in_bounds(part, 4.0 * ksplit * M * w.n, "gemm fwd partials");
  else in_bounds(Y, (y16 ? 2.0 : 4.0) * M * w.n, "Y");
  check_lora(lora, M, w.n);
  return hipSuccess;
}
hipError_t launch_gemv_fwd(const Nf4View& w, const float*, const uint16_t* X, int64_t M,
                           const LoraTerm& lora, void* Y, bool y16, float* part, int ksplit,
                           hipStream_t) {
  ++g_launches;
  CHECK(M <= QLORA_GEMV_MAX_M);
  check_view(w);
  in_bounds(X, 2.0 * M * w.k, "X");
  if (ksplit > 1) in_bounds(part, 4.0 * ksplit * M * w.n, "gemv partials");
  else in_bounds(Y, (y16 ? 2.0 : 4.0) * M * w.n, "Y");
  // a split launch leaves the LoRA term (and its factor) to the reduce
  check_lora(lora, M, w.n, ksplit == 1);
  return hipSuccess;
}
hipError_t launch_gemv_grouped(const GemvJob*, int, int64_t, int64_t M, const float*, int64_t, int,
                               hipStream_t) {
  ++g_launches;
  CHECK(M <= QLORA_GEMV_MAX_M);
  return hipSuccess;
}
hipError_t launch_gemm_dx(const Nf4View& w, const float*, const uint16_t* dY, int64_t M,
                          const LoraTerm& lora, void* dX, bool dx16, float* part, int nsplit,
                          hipStream_t, const WgradFold* fold) {
  ++g_launches;
  check_view(w);
  in_bounds(dY, 2.0 * M * w.n, "dY");
  if (nsplit > 1) in_bounds(part, 4.0 * nsplit * M * w.k, "dx partials");
  else in_bounds(dX, (dx16 ? 2.0 : 4.0) * M * w.k, "dX");
  check_lora(lora, M, w.k);
  if (fold && fold->msplit > 1) {
    ++g_folds;
    CHECK(nsplit == 1);
    CHECK(fold->r == lora.r && fold->ca == w.k && fold->cb == w.n);
    in_bounds(fold->part, 4.0 * fold->msplit * fold->r * (fold->ca + fold->cb), "folded wgrad partials");
    in_bounds(fold->out_a, 4.0 * fold->r * fold->ca, "folded dA");
    in_bounds(fold->out_b, 4.0 * fold->r * fold->cb, "folded dB");
  }
  return hipSuccess;
}
hipError_t launch_gemv_dx(const Nf4View& w, const float*, const uint16_t* dY, int64_t M,
                          const LoraTerm& lora, void* dX, bool dx16, float* part, int nsplit,
                          hipStream_t) {
  ++g_launches;
  check_view(w);
  CHECK(M >= 1 && M <= 32);
  CHECK(nsplit == gemv_dx_splits(w.n, w.k));
  in_bounds(dY, 2.0 * M * w.n, "dY");
  if (nsplit > 1) in_bounds(part, 4.0 * nsplit * M * w.k, "gemv dx partials");
  else in_bounds(dX, (dx16 ? 2.0 : 4.0) * M * w.k, "dX");
  check_lora(lora, M, w.k);
  return hipSuccess;
}
// A rank projection formed in a kernel: P [M x C], Q rank-major [r x C]
// (qs_c == 1) or contraction-major [C x r]; out [M x r] when given.
void check_rank_row(const ql::RankRow& f, int64_t M) {
  CHECK(f.qs_c == 1 ? f.qs_j == f.C : (f.qs_j == 1 && f.qs_c == f.r));
  in_bounds(f.P, 2.0 * M * f.C, "rank row P");
  in_bounds(f.Q, 2.0 * f.r * f.C, "rank row Q");
  if (f.out) in_bounds(f.out, 4.0 * M * f.r, "rank row out");
}
hipError_t launch_reduce(const float* part, int nsplit, int64_t M, int64_t C, const LoraTerm& lora,
                         void* out, bool out16, bool, hipStream_t) {
  ++g_launches;
  in_bounds(part, 4.0 * nsplit * M * C, "reduce partials");
  in_bounds(out, (out16 ? 2.0 : 4.0) * M * C, "reduce out");
  check_lora(lora, M, C);
  return hipSuccess;
}
hipError_t launch_reduce_rows(const float* part, int nsplit, int64_t M, int64_t C, const LoraTerm& lora,
                              void* out, bool out16, bool, hipStream_t, const RankRow& rank) {
  ++g_launches;
  ++g_rank_rows;
  in_bounds(part, 4.0 * nsplit * M * C, "reduce partials");
  in_bounds(out, (out16 ? 2.0 : 4.0) * M * C, "reduce out");
  check_lora(lora, M, C, false);
  CHECK(lora.r == rank.r && ql::rank_row_ok(rank.r, rank.C, rank.P, rank.Q, C));
  check_rank_row(rank, M);
  return hipSuccess;
}
hipError_t launch_rank_rows(const RankRow& rank, int64_t M, bool, hipStream_t) {
  ++g_launches;
  CHECK(rank.out != nullptr && rank.qs_c == 1);
  check_rank_row(rank, M);
  return hipSuccess;
}
hipError_t launch_rowdot(const uint16_t* P, const uint16_t* Q, int64_t M, int64_t C, int r, float* out,
                         float* part, bool, hipStream_t) {
  ++g_launches;
  in_bounds(P, 2.0 * M * C, "rowdot P");
  in_bounds(Q, 2.0 * r * C, "rowdot Q");
  in_bounds(out, 4.0 * M * r, "rowdot out");
  const int ns = rowdot_splits(M, C, r);
  if (ns > 1) in_bounds(part, 4.0 * ns * M * r, "rowdot partials");
  return hipSuccess;
}
hipError_t launch_rowdot_t(const uint16_t* P, const uint16_t* Qs, int64_t M, int64_t C, int r,
                           float* out, float* part, bool, hipStream_t) {
  ++g_launches;
  CHECK(rowdot_t_supported(P, Qs, M, C, r));
  in_bounds(P, 2.0 * M * C, "rowdot_t P");
  in_bounds(Qs, 2.0 * C * r, "rowdot_t Qs");
  in_bounds(out, 4.0 * M * r, "rowdot_t out");
  const int ns = rowdot_splits(M, C, r, true);
  if (ns > 1) in_bounds(part, 4.0 * ns * M * r, "rowdot_t partials");
  return hipSuccess;
}
hipError_t launch_rowdot_grouped(const RowdotJob*, int, int64_t, int, bool, hipStream_t) {
  ++g_launches;
  return hipSuccess;
}
hipError_t launch_transpose_bf16(const uint16_t* Q, int64_t N, int r, uint16_t* Qt, hipStream_t) {
  ++g_launches;
  in_bounds(Q, 2.0 * N * r, "transpose in");
  in_bounds(Qt, 2.0 * N * r, "transpose out");
  return hipSuccess;
}
hipError_t launch_wgrad(const WgradJob& a, const WgradJob& b, int64_t M, int r, float, float* part,
                        int msplit, bool, hipStream_t, bool reduce) {
  ++g_launches;
  if (!reduce) ++g_unreduced;
  in_bounds(a.P, 2.0 * M * a.C, "wgrad a.P");
  in_bounds(a.Q, 4.0 * M * r, "wgrad a.Q");
  in_bounds(a.out, 4.0 * r * a.C, "wgrad a.out");
  in_bounds(b.P, 2.0 * M * b.C, "wgrad b.P");
  in_bounds(b.Q, 4.0 * M * r, "wgrad b.Q");
  in_bounds(b.out, 4.0 * r * b.C, "wgrad b.out");
  if (msplit > 1) in_bounds(part, 4.0 * msplit * r * (a.C + b.C), "wgrad partials");
  return hipSuccess;
}
void* g_scratch_base = nullptr;
hipError_t device_scratch(void** ptr) {
  if (!g_scratch_base) g_scratch_base = fake_alloc(kScratchBytes);
  *ptr = g_scratch_base;
  return hipSuccess;
}
}  // namespace ql

// hipMemcpy is the one HIP runtime call of the host code (group setup): it
// reports failure here, as it would without a device.
extern "C" hipError_t hipMemcpy(void*, const void*, size_t, hipMemcpyKind) { return hipErrorNoDevice; }

namespace {

qlora_nf4 make_weight(int64_t n, int64_t k, int fmt, int block, bool dq) {
  qlora_nf4 w{};
  w.n = n;
  w.k = k;
  w.format = fmt;
  w.block = block;
  size_t c = 0, q = 0, s = 0;
  if (fmt == QLORA_FMT_NF4) CHECK(qlora_nf4_block_bytes(n, k, block ? block : 64, dq, &c, &q, &s) == 0);
  else CHECK(qlora_weight_bytes(fmt, n, k, &c, &q, &s) == 0);
  w.codes = (uint8_t*)fake_alloc(c);
  w.qscale = q ? (uint8_t*)fake_alloc(q) : nullptr;
  w.step = s ? (float*)fake_alloc(s) : nullptr;
  return w;
}

void run_fwd_bwd(int64_t m, int64_t n, int64_t k, int r, int path, bool save_t, int fmt, int block) {
  reset_allocs();
  const qlora_nf4 w = make_weight(n, k, fmt, block, true);
  const float* cb = (const float*)fake_alloc(4 * QLORA_CODEBOOK_LEN);
  const uint16_t* X = (const uint16_t*)fake_alloc(2 * m * k);
  const uint16_t* dY = (const uint16_t*)fake_alloc(2 * m * n);
  const uint16_t* A = r ? (const uint16_t*)fake_alloc(2 * r * k) : nullptr;
  const uint16_t* B = r ? (const uint16_t*)fake_alloc(2 * n * r) : nullptr;
  void* Y = fake_alloc(4 * m * n);
  float* T = r && save_t ? (float*)fake_alloc(4 * m * r) : nullptr;
  void* dX = fake_alloc(4 * m * k);
  float* dA = r ? (float*)fake_alloc(4 * r * k) : nullptr;
  float* dB = r ? (float*)fake_alloc(4 * n * r) : nullptr;
  const size_t wf = qlora_workspace_bytes(0, m, n, k, r), wb = qlora_workspace_bytes(1, m, n, k, r);
  void* wsf = wf ? fake_alloc(wf) : nullptr;
  void* wsb = wb ? fake_alloc(wb) : nullptr;
  for (int dt : {QLORA_F32, QLORA_BF16}) {
    const int e = qlora_linear_fwd(&w, cb, X, m, A, B, r, 2.0f, Y, dt, T, wsf, wf, path, nullptr);
    if (path == QLORA_PATH_GEMV && m > QLORA_GEMV_MAX_M) {
      CHECK(e == QLORA_ERR_ARG);
      continue;
    }
    if (e != QLORA_OK) std::fprintf(stderr, "fwd m=%ld n=%ld k=%ld r=%d path=%d -> %d\n", (long)m, (long)n, (long)k, r, path, e);
    CHECK(e == QLORA_OK);
    // the allocation-free forward: the same launches with the device scratch
    {
      ql::g_scratch_base = nullptr;
      const int before = g_launches;
      const int en = qlora_linear_fwd_noalloc(&w, cb, X, m, A, B, r, 2.0f, Y, dt, T, path, nullptr);
      CHECK(wf <= ql::kScratchBytes ? en == QLORA_OK : en == QLORA_ERR_WORKSPACE);
      CHECK(en == QLORA_OK ? g_launches > before : g_launches == before);
    }
    const int f0 = g_folds, u0 = g_unreduced;
    const int e2 = qlora_linear_bwd(&w, cb, X, dY, m, A, B, r, 2.0f, T, dX, dt, dA, dB, wsb, wb, path,
                                    nullptr);
    // a wgrad launch without its reduction is always paired with a fold
    CHECK(g_folds - f0 == g_unreduced - u0 && g_folds - f0 <= 1);
    const bool bwd_refused = path == QLORA_PATH_GEMV && m > QLORA_GEMV_MAX_M;
    if (e2 != (bwd_refused ? QLORA_ERR_ARG : QLORA_OK))
      std::fprintf(stderr, "bwd m=%ld n=%ld k=%ld r=%d path=%d -> %d\n", (long)m, (long)n, (long)k, r, path, e2);
    CHECK(e2 == (bwd_refused ? QLORA_ERR_ARG : QLORA_OK));
    // a workspace one byte short is refused before any launch
    if (wb > 0 && !bwd_refused) {
      const int before = g_launches;
      CHECK(qlora_linear_bwd(&w, cb, X, dY, m, A, B, r, 2.0f, T, dX, dt, dA, dB, wsb, wb - 1, path,
                             nullptr) == QLORA_ERR_WORKSPACE);
      CHECK(g_launches == before);
    }
  }
}

// Both conversions for every format, block size and scale level, on shapes
// with a partial last row group; overlapping buffers are refused first.
void plain_layout() {
  struct F { int fmt, block; bool dq; };
  const F fs[] = {{QLORA_FMT_NF4, 0, true},   {QLORA_FMT_NF4, 32, true}, {QLORA_FMT_NF4, 128, true},
                  {QLORA_FMT_NF4, 0, false},  {QLORA_FMT_NF4, 32, false}, {QLORA_FMT_NF4, 128, false},
                  {QLORA_FMT_U4_ASYM, 0, false}, {QLORA_FMT_Q8_0, 0, false}};
  const int64_t nks[][2] = {{1, 128}, {17, 256}, {300, 384}, {4096, 11008}};
  for (const F& f : fs)
    for (const auto& nk : nks) {
      if (f.block == 128 && nk[1] % 128) continue;
      reset_allocs();
      qlora_nf4 a = make_weight(nk[0], nk[1], f.fmt, f.block, f.dq);
      qlora_nf4 b = make_weight(nk[0], nk[1], f.fmt, f.block, f.dq);
      if (f.fmt == QLORA_FMT_NF4 && !f.dq) a.qscale = b.qscale = nullptr;
      const int before = g_relayouts;
      CHECK(qlora_to_plain(&a, &b, nullptr) == QLORA_OK);
      CHECK(qlora_from_plain(&b, &a, nullptr) == QLORA_OK);
      CHECK(g_relayouts == before + 2);
      qlora_nf4 c = b;
      c.codes = a.codes;   // the destination's codes on the source's
      CHECK(qlora_to_plain(&a, &c, nullptr) == QLORA_ERR_ARG);
      CHECK(qlora_to_plain(&a, &a, nullptr) == QLORA_ERR_ARG);
      CHECK(g_relayouts == before + 2);
    }
}

void error_paths() {
  reset_allocs();
  const qlora_nf4 w = make_weight(64, 128, QLORA_FMT_NF4, 0, true);
  const float* cb = (const float*)fake_alloc(4 * QLORA_CODEBOOK_LEN);
  const uint16_t* X = (const uint16_t*)fake_alloc(2 * 16 * 128);
  void* Y = fake_alloc(4 * 16 * 64);
  const int before = g_launches;
  CHECK(qlora_linear_fwd(nullptr, cb, X, 16, nullptr, nullptr, 0, 0, Y, 0, nullptr, nullptr, 0, 0, nullptr) == QLORA_ERR_NULL);
  CHECK(qlora_linear_fwd(&w, nullptr, X, 16, nullptr, nullptr, 0, 0, Y, 0, nullptr, nullptr, 0, 0, nullptr) == QLORA_ERR_NULL);
  CHECK(qlora_linear_fwd(&w, cb, X, 0, nullptr, nullptr, 0, 0, Y, 0, nullptr, nullptr, 0, 0, nullptr) == QLORA_ERR_SHAPE);
  CHECK(qlora_linear_fwd(&w, cb, X, 16, nullptr, nullptr, -1, 0, Y, 0, nullptr, nullptr, 0, 0, nullptr) == QLORA_ERR_RANK);
  CHECK(qlora_linear_fwd(&w, cb, X, 16, nullptr, nullptr, 0, 0, Y, 7, nullptr, nullptr, 0, 0, nullptr) == QLORA_ERR_DTYPE);
  CHECK(qlora_linear_fwd(&w, cb, X, 16, nullptr, nullptr, 0, 0, Y, 0, nullptr, nullptr, 0, 9, nullptr) == QLORA_ERR_ARG);
  CHECK(qlora_linear_fwd(&w, cb, (const uint16_t*)((uintptr_t)X + 2), 16, nullptr, nullptr, 0, 0, Y, 0, nullptr, nullptr, 0, 0, nullptr) == QLORA_ERR_ALIGN);
  qlora_nf4 bad = w;
  bad.k = 100;
  CHECK(qlora_linear_fwd(&bad, cb, X, 16, nullptr, nullptr, 0, 0, Y, 0, nullptr, nullptr, 0, 0, nullptr) == QLORA_ERR_SHAPE);
  bad = w;
  bad.n = int64_t(1) << 40;
  CHECK(qlora_linear_fwd(&bad, cb, X, 16, nullptr, nullptr, 0, 0, Y, 0, nullptr, nullptr, 0, 0, nullptr) == QLORA_ERR_SHAPE);
  bad = w;
  bad.format = 9;
  CHECK(qlora_quantize(X, cb, &bad, nullptr) == QLORA_ERR_ARG);
  CHECK(qlora_dequantize(&w, cb, nullptr, nullptr) == QLORA_ERR_NULL);
  CHECK(g_launches == before);
  // size helpers at the limits: no overflow, no launch
  size_t c, q, s;
  CHECK(qlora_nf4_bytes((int64_t(1) << 22) - 1, (int64_t(1) << 16), &c, &q, &s) == QLORA_OK);
  CHECK(qlora_nf4_bytes(int64_t(1) << 22, 64, &c, &q, &s) == QLORA_ERR_SHAPE);
  CHECK(qlora_nf4_bytes(INT64_MAX, INT64_MAX - 63, &c, &q, &s) == QLORA_ERR_SHAPE);
  CHECK(qlora_nf4_bytes(-5, 64, &c, &q, &s) == QLORA_ERR_SHAPE);
  CHECK(qlora_weight_bytes(QLORA_FMT_Q8_0, 3, INT64_MAX, &c, &q, &s) == QLORA_ERR_SHAPE);
  CHECK(qlora_workspace_bytes(1, INT64_MAX, 64, 64, 8) == 0);
  CHECK(qlora_workspace_bytes(0, QLORA_MAX_M + 1, 64, 64, 8) == 0);
  CHECK(qlora_workspace_bytes(1, QLORA_MAX_M, 4096, (int64_t(1) << 22) - 64, 128) > 0);
  CHECK(qlora_workspace_bytes(0, 1, INT64_MAX, 64, 8) == 0);
  float book[QLORA_CODEBOOK_LEN];
  CHECK(qlora_nf4_codebook(book) == QLORA_OK);
  for (int i = 0; i + 1 < 16; ++i) CHECK(book[i] < book[i + 1]);
  for (int s2 = -1; s2 < 12; ++s2) CHECK(qlora_strerror(s2) != nullptr);
  // grouped forward: validation, then the (failing) table copy
  qlora_fwd_job job{};
  job.w = w;
  job.X = X;
  job.Y = Y;
  qlora_group g{};
  void* table = fake_alloc(qlora_group_table_bytes(1));
  CHECK(qlora_group_init(&g, &job, 1, 64, QLORA_F32, table, qlora_group_table_bytes(1)) == QLORA_ERR_ARG);
  CHECK(qlora_group_init(&g, &job, 1, 4, QLORA_F32, table, 1) == QLORA_ERR_WORKSPACE);
  CHECK(qlora_group_init(&g, &job, 1, 4, QLORA_F32, table, qlora_group_table_bytes(1)) == QLORA_ERR_HIP);
}

}  // namespace

int main() {
  error_paths();
  plain_layout();
  const int64_t ms[] = {1, 5, 16, 32, 33, 100, 256, 513, 2048};
  const int64_t nks[][2] = {{64, 64}, {200, 384}, {4096, 4096}, {11008, 4096}, {4096, 11008}, {3072, 8192}};
  const int rs[] = {0, 1, 8, 16, 24, 64, 128};
  for (int64_t m : ms)
    for (const auto& nk : nks)
      for (int r : rs)
        for (int path : {QLORA_PATH_AUTO, QLORA_PATH_GEMV, QLORA_PATH_GEMM})
          run_fwd_bwd(m, nk[0], nk[1], r, path, (m + r) % 2 == 0, QLORA_FMT_NF4, 0);
  for (int fmt : {QLORA_FMT_U4_ASYM, QLORA_FMT_Q8_0})
    run_fwd_bwd(100, 200, 384, 8, QLORA_PATH_AUTO, true, fmt, 0);
  run_fwd_bwd(16, 256, 512, 8, QLORA_PATH_AUTO, false, QLORA_FMT_NF4, 32);
  run_fwd_bwd(600, 256, 512, 32, QLORA_PATH_AUTO, false, QLORA_FMT_NF4, 128);
  CHECK(g_folds > 0);   // the folded reduction was exercised
  CHECK(g_rank_rows > 0);   // and the factor rows formed by split reduces
  CHECK(g_relayouts > 0);
  std::printf("abi host check: %d launches, %d folds, %d relayouts, %d failures\n", g_launches, g_folds,
              g_relayouts, g_fail);
  return g_fail == 0 ? 0 : 1;
}
