// C ABI: argument validation, path and split choice, launches.  Everything is
// checked before the first HIP call; on error nothing is enqueued.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <vector>
#include <cmath>
#include <cstdint>
#include <cstring>

#include "../../include/qlora_nf4.h"
#include "kernels.h"

namespace {

constexpr int64_t kB = QLORA_BLOCK;
constexpr int64_t kG = QLORA_GROUP;

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }
size_t up16(size_t b) { return (b + 15) & ~size_t(15); }
int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// ---- inverse standard-normal CDF: rational first guess refined by Halley's
// method on Phi(x) = erfc(-x / sqrt 2) / 2, which converges to full double
// precision in two steps.
double norm_cdf(double x) { return 0.5 * std::erfc(-x / std::sqrt(2.0)); }

double norm_ppf(double p) {
  // first guess: tail/central rational approximation (Acklam's coefficients)
  static const double a[] = {-3.969683028665376e+01, 2.209460984245205e+02, -2.759285104469687e+02,
                             1.383577518672690e+02,  -3.066479806614716e+01, 2.506628277459239e+00};
  static const double b[] = {-5.447609879822406e+01, 1.615858368580409e+02, -1.556989798598866e+02,
                             6.680131188771972e+01,  -1.328068155288572e+01};
  static const double c[] = {-7.784894002430293e-03, -3.223964580411365e-01, -2.400758277161838e+00,
                             -2.549732539343734e+00, 4.374664141464968e+00,  2.938163982698783e+00};
  static const double d[] = {7.784695709041462e-03, 3.224671290700398e-01, 2.445134137142996e+00,
                             3.754408661907416e+00};
  double x;
  if (p < 0.02425) {
    const double q = std::sqrt(-2 * std::log(p));
    x = (((((c[0] * q + c[1]) * q + c[2]) * q + c[3]) * q + c[4]) * q + c[5]) /
        ((((d[0] * q + d[1]) * q + d[2]) * q + d[3]) * q + 1);
  } else if (p > 1 - 0.02425) {
    const double q = std::sqrt(-2 * std::log(1 - p));
    x = -(((((c[0] * q + c[1]) * q + c[2]) * q + c[3]) * q + c[4]) * q + c[5]) /
        ((((d[0] * q + d[1]) * q + d[2]) * q + d[3]) * q + 1);
  } else {
    const double q = p - 0.5, t = q * q;
    x = (((((a[0] * t + a[1]) * t + a[2]) * t + a[3]) * t + a[4]) * t + a[5]) * q /
        (((((b[0] * t + b[1]) * t + b[2]) * t + b[3]) * t + b[4]) * t + 1);
  }
  for (int it = 0; it < 3; ++it) {
    const double e = norm_cdf(x) - p;
    const double u = e * std::sqrt(2 * M_PI) * std::exp(x * x / 2);
    x = x - u / (1 + x * u / 2);
  }
  return x;
}

// j-th of `num` points equally spaced over [start, stop], stop hit exactly.
double spaced(double start, double stop, int num, int j) {
  if (j == num - 1) return stop;
  const double step = (stop - start) / (num - 1);
  return j * step + start;
}

struct FwdPlan {
  bool gemv;
  int ksplit;
};

FwdPlan plan_fwd(int64_t m, int64_t n, int64_t k, int path) {
  FwdPlan p;
  p.gemv = path == QLORA_PATH_GEMV || (path == QLORA_PATH_AUTO && m <= 32);
  if (p.gemv) {
    // 64-row workgroups; split the contraction until there are ~512 of them,
    // keeping at least 4 quads (1024 k) per split
    const int64_t ntiles = cdiv(n, 64), nquads = cdiv(k / kB, 4);
    const int64_t cap = std::max<int64_t>(1, nquads / 4);
    p.ksplit = (int)std::min<int64_t>(cap, std::max<int64_t>(1, cdiv(512, ntiles)));
  } else {
    // 256 x 128 output tiles, 64-deep steps; split the contraction only when
    // the tiles cannot fill the 256 CUs
    const int64_t tiles = cdiv(m, 256) * cdiv(n, 128), nsteps = cdiv(k, 64);
    const int64_t cap = std::max<int64_t>(1, nsteps / 4);
    p.ksplit = tiles >= 192 ? 1 : (int)std::min<int64_t>(cap, cdiv(256, tiles));
  }
  return p;
}

// The split streaming forward forms T = X A^T inside its reduce.
bool t_in_reduce_ok(const FwdPlan& p, int64_t m, int64_t n, int64_t k, int r, const void* X,
                    const void* A) {
  (void)m;
  return p.gemv && p.ksplit > 1 && ql::rank_row_ok(r, k, X, A, n);
}

int plan_dx_split(int64_t m, int64_t n, int64_t k) {
  const int64_t tiles = cdiv(m, 256) * cdiv(k, 128), nsteps = cdiv(n, 64);
  const int64_t cap = std::max<int64_t>(1, nsteps / 4);
  return tiles >= 192 ? 1 : (int)std::min<int64_t>(cap, cdiv(256, tiles));
}

// input-gradient path: the streaming kernel for small m (or when forced),
// else the MFMA GEMM; the number of contraction splits of either
struct DxPlan {
  bool gemv;
  int nsplit;
};
DxPlan plan_dx(int64_t m, int64_t n, int64_t k, int path) {
  DxPlan p;
  p.gemv = path == QLORA_PATH_GEMV || (path == QLORA_PATH_AUTO && m <= QLORA_GEMV_MAX_M);
  p.nsplit = p.gemv ? ql::gemv_dx_splits(n, k) : plan_dx_split(m, n, k);
  return p;
}

// adapter-gradient splits over the rows (dA over k columns and dB over n in
// one launch): enough workgroups (tiles of 128 columns x 32 or 64 ranks, times
// the splits) to fill the chip twice over, each split at least one 64-row
// chunk
int plan_wgrad_split(int64_t m, int64_t k, int64_t n, int r) {
  const int64_t jw = r <= 32 ? 32 : 64;
  const int64_t tiles = (cdiv(k, 128) + cdiv(n, 128)) * cdiv(std::max(r, 1), jw);
  return (int)std::min<int64_t>(std::max<int64_t>(1, cdiv(512, tiles)), cdiv(m, 64));
}

struct FwdWs {
  size_t t_off, part_off, total;
};
FwdWs fwd_ws(int64_t m, int64_t n, int64_t k, int r, int path) {
  const FwdPlan p = plan_fwd(m, n, k, path);
  FwdWs w;
  w.t_off = 0;
  w.part_off = up16(sizeof(float) * (size_t)(m * r));
  // the region after T holds the GEMM's split partials, and before the GEMM
  // runs the rank projection's split partials
  const int rs = r > 0 ? ql::rowdot_splits(m, k, r) : 1;
  const size_t gemm_part = p.ksplit > 1 ? sizeof(float) * (size_t)p.ksplit * m * n : 0;
  const size_t rd_part = rs > 1 ? sizeof(float) * (size_t)rs * m * r : 0;
  w.total = w.part_off + std::max(gemm_part, rd_part);
  return w;
}

struct BwdWs {
  size_t u_off, t_off, bt_off, dx_off, wg_off, total;
};
BwdWs bwd_ws(int64_t m, int64_t n, int64_t k, int r) {
  BwdWs w;
  w.u_off = 0;
  w.t_off = w.u_off + up16(sizeof(float) * (size_t)(m * r));
  w.bt_off = w.t_off + up16(sizeof(float) * (size_t)(m * r));
  w.dx_off = w.bt_off + up16(sizeof(uint16_t) * (size_t)(r * n));
  // the input gradient's split partials, for whichever path runs
  size_t dxp = 0;
  for (int path : {QLORA_PATH_GEMV, QLORA_PATH_GEMM}) {
    if (path == QLORA_PATH_GEMV && m > QLORA_GEMV_MAX_M) continue;
    const DxPlan p = plan_dx(m, n, k, path);
    if (p.nsplit > 1) dxp = std::max(dxp, sizeof(float) * (size_t)p.nsplit * m * k);
  }
  w.wg_off = w.dx_off + up16(dxp);
  // the last region holds the adapter-gradient split partials, and before
  // those run the rank projections' split partials (U over n, T over k)
  size_t wg = 0;
  if (r > 0) {
    const int sw = plan_wgrad_split(m, k, n, r);
    wg = sw > 1 ? sizeof(float) * (size_t)sw * r * (k + n) : 0;
    // U reads B in place when it can (its own split count), else a transposed copy
    const int ru = std::max(ql::rowdot_splits(m, n, r), ql::rowdot_splits(m, n, r, true));
    const int rt = ql::rowdot_splits(m, k, r);
    wg = std::max(wg, sizeof(float) * (size_t)std::max(ru * (ru > 1), rt * (rt > 1)) * m * r);
  }
  w.total = w.wg_off + up16(wg);
  return w;
}

// block counts are kept below 2^32 (n * k < 2^38 weights per matrix)
// n and k stay below 2^22 so that the kernels' per-tile byte offsets fit in
// 32 bits; the element count below 2^38 keeps block indices in 32 bits.
bool shape_ok(int64_t n, int64_t k) {
  return n >= 1 && k >= kB && k % kB == 0 && n < (int64_t(1) << 22) && k < (int64_t(1) << 22) &&
         n <= ((int64_t(1) << 38) - 1) / k;
}

// NF4 block size of a descriptor (0 means 64); 0 for an invalid one.
int nf4_block(const qlora_nf4* W) {
  const int b = W->block == 0 ? 64 : W->block;
  if (W->format != QLORA_FMT_NF4) return b == 64 ? 64 : 0;
  return (b == 32 || b == 64 || b == 128) ? b : 0;
}

// Shape limits of a block size: block 128 needs whole 128-blocks per row,
// block 32 keeps its block count below 2^32.
bool block_shape_ok(int64_t n, int64_t k, int block) {
  if (block == 128 && k % 128 != 0) return false;
  if (block == 32 && n > ((int64_t(1) << 37) - 1) / k) return false;
  return true;
}

// Token count: at least one row, fewer than 2^31 (with n, k < 2^22 every
// activation, output and workspace size stays far inside 64 bits).
bool m_ok(int64_t m) { return m >= 1 && m <= QLORA_MAX_M; }

// Compute type of a descriptor: fp16 (QLORA_F16) or the bf16 default.
bool is_f16(const qlora_nf4* W) { return W->dtype == QLORA_F16; }

// The arrays each format uses (NF4: qscale NULL selects the single-level
// scales), their alignment, the shape, the compute type (fp16 only for NF4
// at block 64 with double quantization).
int check_desc(const qlora_nf4* W) {
  if (!W) return QLORA_ERR_NULL;
  if (!nf4_block(W)) return QLORA_ERR_ARG;
  if (W->dtype != 0 && W->dtype != QLORA_BF16 && W->dtype != QLORA_F16) return QLORA_ERR_DTYPE;
  if (is_f16(W) && (W->format != QLORA_FMT_NF4 || nf4_block(W) != 64 || !W->qscale))
    return QLORA_ERR_DTYPE;
  switch (W->format) {
    case QLORA_FMT_NF4:
      if (!W->codes || !W->step) return QLORA_ERR_NULL;
      break;
    case QLORA_FMT_U4_ASYM:
      if (!W->codes || !W->step) return QLORA_ERR_NULL;
      if (W->qscale) return QLORA_ERR_ARG;
      break;
    case QLORA_FMT_Q8_0:
      if (!W->codes || !W->qscale) return QLORA_ERR_NULL;
      break;
    default:
      return QLORA_ERR_ARG;
  }
  if (!shape_ok(W->n, W->k) || !block_shape_ok(W->n, W->k, nf4_block(W))) return QLORA_ERR_SHAPE;
  if (!aligned(W->codes, 16)) return QLORA_ERR_ALIGN;
  if (W->format == QLORA_FMT_NF4 && !aligned(W->step, 4)) return QLORA_ERR_ALIGN;
  if (W->format == QLORA_FMT_U4_ASYM && !aligned(W->step, 8)) return QLORA_ERR_ALIGN;
  if (W->format == QLORA_FMT_Q8_0 && !aligned(W->qscale, 4)) return QLORA_ERR_ALIGN;
  return QLORA_OK;
}

// The codebook: required (and 4-byte aligned) for NF4 only.
int check_codebook(const qlora_nf4* W, const float* codebook) {
  if (W->format != QLORA_FMT_NF4) return QLORA_OK;
  if (!codebook) return QLORA_ERR_NULL;
  return aligned(codebook, 4) ? QLORA_OK : QLORA_ERR_ALIGN;
}

// 16-bit output dtype allowed for this weight: fp32 or its compute type.
bool out_dtype_ok(const qlora_nf4* W, int dtype) {
  return dtype == QLORA_F32 || dtype == (is_f16(W) ? QLORA_F16 : QLORA_BF16);
}

int kernel_fmt(const qlora_nf4* W) {
  if (is_f16(W)) return ql::kFmtNf4DqF16;
  switch (W->format) {
    case QLORA_FMT_U4_ASYM: return ql::kFmtU4;
    case QLORA_FMT_Q8_0: return ql::kFmtQ8;
    default: {
      const bool dq = W->qscale != nullptr;
      switch (nf4_block(W)) {
        case 32: return dq ? ql::kFmtNf4Dq32 : ql::kFmtNf4_32;
        case 128: return dq ? ql::kFmtNf4Dq128 : ql::kFmtNf4_128;
        default: return dq ? ql::kFmtNf4Dq : ql::kFmtNf4;
      }
    }
  }
}

ql::Nf4View view(const qlora_nf4* W) {
  return ql::Nf4View{W->codes, W->qscale, W->step, W->n, W->k, kernel_fmt(W)};
}

// Byte sizes of the three arrays of a valid descriptor (0 for an unused one).
void desc_bytes(const qlora_nf4* W, size_t sz[3]) {
  if (W->format == QLORA_FMT_NF4)
    qlora_nf4_block_bytes(W->n, W->k, nf4_block(W), W->qscale != nullptr, &sz[0], &sz[1], &sz[2]);
  else
    qlora_weight_bytes(W->format, W->n, W->k, &sz[0], &sz[1], &sz[2]);
}

// Two descriptors of the same weight in the two layouts: both valid, the
// same shape, format, block size, compute type and scale level, and no array
// of one overlapping an array of the other.
int check_relayout(const qlora_nf4* src, const qlora_nf4* dst) {
  if (!src || !dst) return QLORA_ERR_NULL;
  if (int e = check_desc(src)) return e;
  if (int e = check_desc(dst)) return e;
  if (src->n != dst->n || src->k != dst->k) return QLORA_ERR_SHAPE;
  if (src->format != dst->format || nf4_block(src) != nf4_block(dst) ||
      (src->qscale == nullptr) != (dst->qscale == nullptr))
    return QLORA_ERR_ARG;
  if (is_f16(src) != is_f16(dst)) return QLORA_ERR_DTYPE;
  size_t a[3], b[3];
  desc_bytes(src, a);
  desc_bytes(dst, b);
  const uintptr_t pa[3] = {(uintptr_t)src->codes, (uintptr_t)src->qscale, (uintptr_t)src->step};
  const uintptr_t pb[3] = {(uintptr_t)dst->codes, (uintptr_t)dst->qscale, (uintptr_t)dst->step};
  for (int i = 0; i < 3; ++i)
    for (int j = 0; j < 3; ++j)
      if (a[i] && b[j] && pa[i] < pb[j] + b[j] && pb[j] < pa[i] + a[i]) return QLORA_ERR_ARG;
  return QLORA_OK;
}

}  // namespace

extern "C" {

const char* qlora_strerror(int s) {
  switch (s) {
    case QLORA_OK: return "ok";
    case QLORA_ERR_NULL: return "a required pointer is NULL";
    case QLORA_ERR_SHAPE: return "bad shape (m, n, k must be >= 1 and k a multiple of 64)";
    case QLORA_ERR_ALIGN: return "pointer not aligned as required";
    case QLORA_ERR_DTYPE: return "unknown dtype, or a dtype the weight or its compute type does not allow";
    case QLORA_ERR_RANK: return "LoRA rank out of range [0, 128]";
    case QLORA_ERR_WORKSPACE: return "workspace missing or too small";
    case QLORA_ERR_HIP: return "HIP launch failed";
    case QLORA_ERR_ARG: return "argument out of range";
    default: return "unknown status";
  }
}

int qlora_nf4_codebook(float* out) {
  if (!out) return QLORA_ERR_NULL;
  const double cp = norm_ppf(1.0 - 1.0 / 32.0), cn = norm_ppf(1.0 - 1.0 / 30.0);
  double lv[16];
  for (int j = 1; j <= 8; ++j) lv[7 + j] = norm_ppf(spaced(0.5, 1.0 - 1.0 / 32.0, 9, j)) / cp;
  for (int j = 1; j <= 7; ++j) lv[7 - j] = -norm_ppf(spaced(0.5, 1.0 - 1.0 / 30.0, 8, j)) / cn;
  lv[7] = 0.0;
  for (int i = 0; i < 16; ++i) out[i] = (float)lv[i];
  for (int i = 0; i < 15; ++i) {
    const double exact = ((double)out[i] + (double)out[i + 1]) / 2.0;
    float mid = (float)exact;
    if ((double)mid > exact) mid = std::nextafter(mid, -INFINITY);
    out[16 + i] = mid;
  }
  return QLORA_OK;
}

int qlora_nf4_bytes(int64_t n, int64_t k, size_t* codes, size_t* qscale, size_t* step) {
  if (!shape_ok(n, k)) return QLORA_ERR_SHAPE;
  const int64_t nb = n * (k / kB);
  if (codes) *codes = (size_t)(n * k / 2);
  if (qscale) *qscale = (size_t)nb;
  if (step) *step = sizeof(float) * (size_t)cdiv(nb, kG);
  return QLORA_OK;
}

int qlora_nf4_single_bytes(int64_t n, int64_t k, size_t* codes, size_t* absmax) {
  if (!shape_ok(n, k)) return QLORA_ERR_SHAPE;
  if (codes) *codes = (size_t)(n * k / 2);
  if (absmax) *absmax = sizeof(float) * (size_t)(n * (k / kB));
  return QLORA_OK;
}

int qlora_nf4_block_bytes(int64_t n, int64_t k, int block, int double_quant, size_t* codes,
                          size_t* qscale, size_t* step) {
  if (block != 32 && block != 64 && block != 128) return QLORA_ERR_ARG;
  if (!shape_ok(n, k) || !block_shape_ok(n, k, block)) return QLORA_ERR_SHAPE;
  const size_t nb = (size_t)(n * k / block);
  if (codes) *codes = (size_t)(n * k / 2);
  if (qscale) *qscale = double_quant ? nb : 0;
  if (step) *step = double_quant ? sizeof(float) * ((nb + kG - 1) / kG) : sizeof(float) * nb;
  return QLORA_OK;
}

int qlora_weight_bytes(int format, int64_t n, int64_t k, size_t* codes, size_t* qscale,
                       size_t* step) {
  if (format < QLORA_FMT_NF4 || format > QLORA_FMT_Q8_0) return QLORA_ERR_ARG;
  if (!shape_ok(n, k)) return QLORA_ERR_SHAPE;
  if (format == QLORA_FMT_NF4) return qlora_nf4_bytes(n, k, codes, qscale, step);
  const size_t units = (size_t)(n * (k / kB));
  const bool u4 = format == QLORA_FMT_U4_ASYM;
  if (codes) *codes = u4 ? (size_t)(n * k / 2) : (size_t)(n * k);
  if (qscale) *qscale = u4 ? 0 : 4 * units;
  if (step) *step = u4 ? 8 * units : 0;
  return QLORA_OK;
}

size_t qlora_workspace_bytes(int op, int64_t m, int64_t n, int64_t k, int r) {
  if (!m_ok(m) || !shape_ok(n, k) || r < 0 || r > QLORA_MAX_RANK) return 0;
  if (op == 0) {
    size_t b = 0;
    for (int path : {QLORA_PATH_AUTO, QLORA_PATH_GEMV, QLORA_PATH_GEMM}) {
      if (path == QLORA_PATH_GEMV && m > QLORA_GEMV_MAX_M) continue;
      b = std::max(b, fwd_ws(m, n, k, r, path).total);
    }
    return b;
  }
  if (op == 1) return bwd_ws(m, n, k, r).total;
  return 0;
}

int qlora_quantize(const uint16_t* W, const float* codebook, const qlora_nf4* out, void* stream) {
  if (!W) return QLORA_ERR_NULL;
  if (int e = check_desc(out)) return e;
  if (int e = check_codebook(out, codebook)) return e;
  if (!aligned(W, 16)) return QLORA_ERR_ALIGN;
  if (ql::launch_quantize(W, codebook, out->codes, out->qscale, out->step, out->n, out->k,
                          kernel_fmt(out), (hipStream_t)stream) != hipSuccess)
    return QLORA_ERR_HIP;
  return QLORA_OK;
}

int qlora_dequantize(const qlora_nf4* W, const float* codebook, uint16_t* out, void* stream) {
  if (!out) return QLORA_ERR_NULL;
  if (int e = check_desc(W)) return e;
  if (int e = check_codebook(W, codebook)) return e;
  if (!aligned(out, 16)) return QLORA_ERR_ALIGN;
  if (ql::launch_dequant(view(W), codebook, out, (hipStream_t)stream) != hipSuccess)
    return QLORA_ERR_HIP;
  return QLORA_OK;
}

int qlora_to_plain(const qlora_nf4* src, const qlora_nf4* dst, void* stream) {
  if (int e = check_relayout(src, dst)) return e;
  if (ql::launch_relayout(src->codes, src->qscale, src->step, dst->codes, dst->qscale, dst->step, src->n,
                          src->k, kernel_fmt(src), true, (hipStream_t)stream) != hipSuccess)
    return QLORA_ERR_HIP;
  return QLORA_OK;
}

int qlora_from_plain(const qlora_nf4* src, const qlora_nf4* dst, void* stream) {
  if (int e = check_relayout(src, dst)) return e;
  if (ql::launch_relayout(src->codes, src->qscale, src->step, dst->codes, dst->qscale, dst->step, src->n,
                          src->k, kernel_fmt(src), false, (hipStream_t)stream) != hipSuccess)
    return QLORA_ERR_HIP;
  return QLORA_OK;
}

int qlora_merge(const qlora_nf4* W, const float* codebook, const uint16_t* A, const uint16_t* B,
                int r, float scaling, uint16_t* merged, const qlora_nf4* out, void* stream) {
  if (!merged) return QLORA_ERR_NULL;
  if (int e = check_desc(W)) return e;
  if (int e = check_codebook(W, codebook)) return e;
  if (out) {
    if (int e = check_desc(out)) return e;
    if (int e = check_codebook(out, codebook)) return e;
    if (out->n != W->n || out->k != W->k) return QLORA_ERR_SHAPE;
    if (is_f16(out) != is_f16(W)) return QLORA_ERR_DTYPE;
  }
  if (r < 0 || r > QLORA_MAX_RANK) return QLORA_ERR_RANK;
  if (r > 0 && (!A || !B)) return QLORA_ERR_NULL;
  if (!aligned(merged, 16) || (r > 0 && (!aligned(A, 16) || !aligned(B, 2)))) return QLORA_ERR_ALIGN;
  hipStream_t s = (hipStream_t)stream;
  if (ql::launch_dequant(view(W), codebook, merged, s) != hipSuccess) return QLORA_ERR_HIP;
  if (r > 0 && ql::launch_merge(merged, A, B, W->n, W->k, r, scaling, is_f16(W), s) != hipSuccess)
    return QLORA_ERR_HIP;
  if (out && ql::launch_quantize(merged, codebook, out->codes, out->qscale, out->step, out->n,
                                 out->k, kernel_fmt(out), s) != hipSuccess)
    return QLORA_ERR_HIP;
  return QLORA_OK;
}

}  // extern "C"

namespace {

// Argument checks of the forward (everything but the workspace).
int check_fwd(const qlora_nf4* W, const float* codebook, const uint16_t* X, int64_t m,
              const uint16_t* A, const uint16_t* B, int r, void* Y, int y_dtype, float* T_save,
              int path) {
  if (!X || !Y) return QLORA_ERR_NULL;
  if (int e = check_desc(W)) return e;
  if (int e = check_codebook(W, codebook)) return e;
  if (!m_ok(m)) return QLORA_ERR_SHAPE;
  if (r < 0 || r > QLORA_MAX_RANK) return QLORA_ERR_RANK;
  if (r > 0 && (!A || !B)) return QLORA_ERR_NULL;
  if (!out_dtype_ok(W, y_dtype)) return QLORA_ERR_DTYPE;
  if (path < QLORA_PATH_AUTO || path > QLORA_PATH_GEMM) return QLORA_ERR_ARG;
  if (path == QLORA_PATH_GEMV && m > QLORA_GEMV_MAX_M) return QLORA_ERR_ARG;
  if (!aligned(X, 16) || !aligned(Y, 16)) return QLORA_ERR_ALIGN;
  if (r > 0 && (!aligned(A, 16) || !aligned(B, 2) || (T_save && !aligned(T_save, 4))))
    return QLORA_ERR_ALIGN;
  return QLORA_OK;
}

// Bytes of workspace this forward uses (0 when it needs none).
size_t fwd_ws_needed(int64_t m, int64_t n, int64_t k, int r, bool t_saved, int path) {
  const FwdWs L = fwd_ws(m, n, k, r, path);
  const bool need_ws = L.total > L.part_off || (r > 0 && !t_saved);
  return need_ws ? L.total : 0;
}

// The forward's launches, arguments already checked and the workspace
// (ws, at least fwd_ws_needed bytes when that is not 0) in hand.
int run_fwd(const qlora_nf4* W, const float* codebook, const uint16_t* X, int64_t m,
            const uint16_t* A, const uint16_t* B, int r, float scaling, void* Y, int y_dtype,
            float* T_save, void* ws, int path, hipStream_t s) {
  const int64_t n = W->n, k = W->k;
  const FwdWs L = fwd_ws(m, n, k, r, path);
  const FwdPlan p = plan_fwd(m, n, k, path);
  char* wsb = (char*)ws;
  // split streaming forward: T is formed by the split reduce, which needs it
  // (no rank-projection launch)
  const bool t_in_reduce = t_in_reduce_ok(p, m, n, k, r, X, A);
  float* T = nullptr;
  if (r > 0 && !t_in_reduce) {
    T = T_save ? T_save : (float*)(wsb + L.t_off);
    float* rpart = ws ? (float*)(wsb + L.part_off) : nullptr;   // needed only with splits
    if (ql::launch_rowdot(X, A, m, k, r, T, rpart, is_f16(W), s) != hipSuccess)
      return QLORA_ERR_HIP;
  }
  ql::LoraTerm lora{T, B, (int64_t)r, 1, r, scaling};
  float* part = p.ksplit > 1 ? (float*)(wsb + L.part_off) : nullptr;
  const ql::Nf4View v = view(W);
  const bool bf = y_dtype != QLORA_F32;   // a 16-bit output of the compute type
  hipError_t e = p.gemv ? ql::launch_gemv_fwd(v, codebook, X, m, lora, Y, bf, part, p.ksplit, s)
                        : ql::launch_gemm_fwd(v, codebook, X, m, lora, Y, bf, part, p.ksplit, s);
  if (e != hipSuccess) return QLORA_ERR_HIP;
  if (p.ksplit > 1) {
    const hipError_t er =
        t_in_reduce ? ql::launch_reduce_rows(part, p.ksplit, m, n, lora, Y, bf, is_f16(W), s,
                                             ql::RankRow{X, A, k, 1, r, k, T_save})
                    : ql::launch_reduce(part, p.ksplit, m, n, lora, Y, bf, is_f16(W), s);
    if (er != hipSuccess) return QLORA_ERR_HIP;
  }
  return QLORA_OK;
}

}  // namespace

extern "C" {

int qlora_linear_fwd_noalloc(const qlora_nf4* W, const float* codebook, const uint16_t* X,
                             int64_t m, const uint16_t* A, const uint16_t* B, int r,
                             float scaling, void* Y, int y_dtype, float* T_save, int path,
                             void* stream) {
  if (int e = check_fwd(W, codebook, X, m, A, B, r, Y, y_dtype, T_save, path)) return e;
  const size_t need = fwd_ws_needed(m, W->n, W->k, r, T_save != nullptr, path);
  if (need > ql::kScratchBytes) return QLORA_ERR_WORKSPACE;
  void* ws = nullptr;
  if (need > 0 && ql::device_scratch(&ws) != hipSuccess) return QLORA_ERR_HIP;
  return run_fwd(W, codebook, X, m, A, B, r, scaling, Y, y_dtype, T_save, ws, path,
                 (hipStream_t)stream);
}

int qlora_linear_fwd(const qlora_nf4* W, const float* codebook, const uint16_t* X, int64_t m,
                     const uint16_t* A, const uint16_t* B, int r, float scaling, void* Y,
                     int y_dtype, float* T_save, void* ws, size_t ws_bytes, int path,
                     void* stream) {
  if (int e = check_fwd(W, codebook, X, m, A, B, r, Y, y_dtype, T_save, path)) return e;
  const size_t need = fwd_ws_needed(m, W->n, W->k, r, T_save != nullptr, path);
  if (need > 0 && (!ws || ws_bytes < need)) return QLORA_ERR_WORKSPACE;
  if (ws && !aligned(ws, 16)) return QLORA_ERR_ALIGN;
  return run_fwd(W, codebook, X, m, A, B, r, scaling, Y, y_dtype, T_save, ws, path,
                 (hipStream_t)stream);
}

size_t qlora_group_table_bytes(int count) {
  if (count < 1) return 0;
  return up16(sizeof(ql::GemvJob) * (size_t)count) + up16(sizeof(ql::RowdotJob) * (size_t)count);
}

int qlora_group_init(qlora_group* g, const qlora_fwd_job* jobs, int count, int64_t m, int y_dtype,
                     void* table, size_t table_bytes) {
  if (!g || !jobs || !table) return QLORA_ERR_NULL;
  if (count < 1 || m > QLORA_GEMV_MAX_M) return QLORA_ERR_ARG;
  if (!m_ok(m)) return QLORA_ERR_SHAPE;
  if (y_dtype != QLORA_F32 && y_dtype != QLORA_BF16 && y_dtype != QLORA_F16) return QLORA_ERR_DTYPE;
  if (!aligned(table, 16)) return QLORA_ERR_ALIGN;
  if (table_bytes < qlora_group_table_bytes(count)) return QLORA_ERR_WORKSPACE;
  const size_t rd_off = up16(sizeof(ql::GemvJob) * (size_t)count);
  ql::GemvJob* gj = new ql::GemvJob[count];
  ql::RowdotJob* rj = new ql::RowdotJob[count];
  int nl = 0, max_r = 0;
  int64_t rgs = 0, maxq = 0;
  int st = QLORA_OK;
  int fmt = -1;
  for (int i = 0; i < count && st == QLORA_OK; ++i) {
    const qlora_fwd_job& J = jobs[i];
    if ((st = check_desc(&J.w))) break;
    if (i == 0) fmt = kernel_fmt(&J.w);
    if (kernel_fmt(&J.w) != fmt) { st = QLORA_ERR_ARG; break; }   // one format per group
    if (!out_dtype_ok(&J.w, y_dtype)) { st = QLORA_ERR_DTYPE; break; }
    if (!J.X || !J.Y) { st = QLORA_ERR_NULL; break; }
    if (J.r < 0 || J.r > QLORA_MAX_RANK) { st = QLORA_ERR_RANK; break; }
    if (J.r > 0 && (!J.A || !J.B || !J.T)) { st = QLORA_ERR_NULL; break; }
    if (!aligned(J.X, 16) || !aligned(J.Y, 16) ||
        (J.r > 0 && (!aligned(J.A, 16) || !aligned(J.B, 2) || !aligned(J.T, 4)))) {
      st = QLORA_ERR_ALIGN;
      break;
    }
    const int64_t k = J.w.k;
    maxq = std::max(maxq, cdiv(k / kB, 4));
    if (J.r > 0) {
      rj[nl++] = ql::RowdotJob{J.X, J.A, J.T, k, J.r};
      max_r = std::max(max_r, J.r);
    }
  }
  if (st == QLORA_OK) {
    // The launch's workgroup ranges go to the jobs longest contraction first
    // (stable): workgroups are dispatched in range order, so the launch ends
    // on the shortest ones instead of on a few long ones running alone.  The
    // table is in range order, as the kernel's search needs.
    std::vector<int> order(count);
    for (int i = 0; i < count; ++i) order[i] = i;
    std::stable_sort(order.begin(), order.end(),
                     [&](int a, int b) { return jobs[a].w.k > jobs[b].w.k; });
    for (int p = 0; p < count; ++p) {
      const qlora_fwd_job& J = jobs[order[p]];
      ql::LoraTerm lora{J.r > 0 ? J.T : nullptr, J.B, (int64_t)J.r, 1, J.r, J.scaling};
      gj[p] = ql::GemvJob{J.X, view(&J.w), lora, J.Y, nullptr, m, y_dtype != QLORA_F32, rgs};
      rgs += cdiv(J.w.n, 64);
    }
  }
  if (st == QLORA_OK) {
    if (hipMemcpy(table, gj, sizeof(ql::GemvJob) * (size_t)count, hipMemcpyHostToDevice) != hipSuccess ||
        (nl > 0 && hipMemcpy((char*)table + rd_off, rj, sizeof(ql::RowdotJob) * (size_t)nl,
                             hipMemcpyHostToDevice) != hipSuccess))
      st = QLORA_ERR_HIP;
  }
  delete[] gj;
  delete[] rj;
  if (st != QLORA_OK) return st;
  *g = qlora_group{table, count, nl, max_r, y_dtype, fmt, m, rgs, maxq};
  return QLORA_OK;
}

int qlora_linear_fwd_grouped(const qlora_group* g, const float* codebook, void* stream) {
  if (!g || !g->table) return QLORA_ERR_NULL;
  if (g->count < 1 || g->m < 1 || g->m > QLORA_GEMV_MAX_M || g->lora_count < 0 ||
      g->lora_count > g->count || g->row_groups < 1 || g->variant < 0 || g->variant >= ql::kNumFmt)
    return QLORA_ERR_ARG;
  const bool nf4 = g->variant != ql::kFmtU4 && g->variant != ql::kFmtQ8;
  if (nf4 && !codebook) return QLORA_ERR_NULL;
  if (nf4 && !aligned(codebook, 4)) return QLORA_ERR_ALIGN;
  hipStream_t s = (hipStream_t)stream;
  const char* tb = (const char*)g->table;
  const size_t rd_off = up16(sizeof(ql::GemvJob) * (size_t)g->count);
  if (g->lora_count > 0 &&
      ql::launch_rowdot_grouped((const ql::RowdotJob*)(tb + rd_off), g->lora_count, g->m, g->max_r,
                                ql::fmt_f16(g->variant), s) != hipSuccess)
    return QLORA_ERR_HIP;
  if (ql::launch_gemv_grouped((const ql::GemvJob*)tb, g->count, g->row_groups, g->m, codebook,
                              g->max_quads, g->variant, s) != hipSuccess)
    return QLORA_ERR_HIP;
  return QLORA_OK;
}

int qlora_linear_bwd(const qlora_nf4* W, const float* codebook, const uint16_t* X,
                     const uint16_t* dY, int64_t m, const uint16_t* A, const uint16_t* B, int r,
                     float scaling, const float* T_saved, void* dX, int dx_dtype, float* dA,
                     float* dB, void* ws, size_t ws_bytes, int path, void* stream) {
  if (!dY) return QLORA_ERR_NULL;
  if (int e = check_desc(W)) return e;
  if (int e = check_codebook(W, codebook)) return e;
  if (!m_ok(m)) return QLORA_ERR_SHAPE;
  if (r < 0 || r > QLORA_MAX_RANK) return QLORA_ERR_RANK;
  if (r > 0 && (!A || !B || !dA || !dB || !X)) return QLORA_ERR_NULL;
  if (!out_dtype_ok(W, dx_dtype)) return QLORA_ERR_DTYPE;
  if (path < QLORA_PATH_AUTO || path > QLORA_PATH_GEMM) return QLORA_ERR_ARG;
  if (path == QLORA_PATH_GEMV && m > QLORA_GEMV_MAX_M) return QLORA_ERR_ARG;
  if (!aligned(dY, 16) || (dX && !aligned(dX, 16)) || (X && !aligned(X, 16)))
    return QLORA_ERR_ALIGN;
  if (r > 0 && (!aligned(A, 16) || !aligned(B, 2) || !aligned(dA, 4) || !aligned(dB, 4) ||
                (T_saved && !aligned(T_saved, 4))))
    return QLORA_ERR_ALIGN;
  const int64_t n = W->n, k = W->k;
  const BwdWs L = bwd_ws(m, n, k, r);
  if (L.total > 0 && (!ws || ws_bytes < L.total)) return QLORA_ERR_WORKSPACE;
  if (ws && !aligned(ws, 16)) return QLORA_ERR_ALIGN;

  hipStream_t s = (hipStream_t)stream;
  char* wsb = (char*)ws;
  const DxPlan p = plan_dx(m, n, k, path);
  // split streaming input gradient: U = dY B is formed by its split reduce,
  // which writes it for the adapter gradients that follow (no rank-projection
  // or transpose launch)
  const bool u_in_reduce = dX && p.gemv && p.nsplit > 1 && ql::rank_row_ok(r, n, dY, B, k);
  float* U = nullptr;
  const float* T = T_saved;
  if (r > 0) {
    U = (float*)(wsb + L.u_off);
    float* rpart = (float*)(wsb + L.wg_off);
    if (u_in_reduce) {
      // formed by the input gradient's reduce below
    } else if (ql::rowdot_t_supported(dY, B, m, n, r)) {   // U = dY B reading B as stored
      if (ql::launch_rowdot_t(dY, B, m, n, r, U, rpart, is_f16(W), s) != hipSuccess)
        return QLORA_ERR_HIP;
    } else {
      uint16_t* Bt = (uint16_t*)(wsb + L.bt_off);
      if (ql::launch_transpose_bf16(B, n, r, Bt, s) != hipSuccess) return QLORA_ERR_HIP;
      if (ql::launch_rowdot(dY, Bt, m, n, r, U, rpart, is_f16(W), s) != hipSuccess)
        return QLORA_ERR_HIP;
    }
    if (!T) {
      // recomputed bit for bit as the forward's AUTO path forms it
      float* Tw = (float*)(wsb + L.t_off);
      if (t_in_reduce_ok(plan_fwd(m, n, k, QLORA_PATH_AUTO), m, n, k, r, X, A)) {
        if (ql::launch_rank_rows(ql::RankRow{X, A, k, 1, r, k, Tw}, m, is_f16(W), s) != hipSuccess)
          return QLORA_ERR_HIP;
      } else if (ql::launch_rowdot(X, A, m, k, r, Tw, rpart, is_f16(W), s) != hipSuccess) {
        return QLORA_ERR_HIP;
      }
      T = Tw;
    }
  }
  // Adapter gradients.  When the input gradient runs as one tiled GEMM, the
  // gradients' split partials go first and that GEMM adds them up (its
  // producer waves are idle once their last decode is done), which saves the
  // reduction launch; otherwise they come last with their own reduction.
  const int msplit = r > 0 ? plan_wgrad_split(m, k, n, r) : 1;
  const bool fold = r > 0 && dX && !p.gemv && p.nsplit == 1 && msplit > 1;
  const ql::WgradJob ja{X, U, k, dA, 0}, jb{dY, T, n, dB, 1};
  float* wpart = (float*)(wsb + L.wg_off);
  if (fold && ql::launch_wgrad(ja, jb, m, r, scaling, wpart, msplit, is_f16(W), s, false) != hipSuccess)
    return QLORA_ERR_HIP;
  if (dX) {
    const int ns = p.nsplit;
    ql::LoraTerm lora{U, A, 1, k, r, scaling};
    float* part = ns > 1 ? (float*)(wsb + L.dx_off) : nullptr;
    const bool bf = dx_dtype != QLORA_F32;   // a 16-bit output of the compute type
    ql::WgradFold wf;
    if (fold) wf = ql::WgradFold{wpart, msplit, r, scaling, k, n, dA, dB, 0, 1};
    const hipError_t e = p.gemv ? ql::launch_gemv_dx(view(W), codebook, dY, m, lora, dX, bf, part, ns, s)
                                : ql::launch_gemm_dx(view(W), codebook, dY, m, lora, dX, bf, part, ns, s,
                                                     fold ? &wf : nullptr);
    if (e != hipSuccess) return QLORA_ERR_HIP;
    if (ns > 1) {
      const hipError_t er =
          u_in_reduce ? ql::launch_reduce_rows(part, ns, m, k, lora, dX, bf, is_f16(W), s,
                                               ql::RankRow{dY, B, 1, r, r, n, U})
                      : ql::launch_reduce(part, ns, m, k, lora, dX, bf, is_f16(W), s);
      if (er != hipSuccess) return QLORA_ERR_HIP;
    }
  }
  if (r > 0 && !fold &&
      ql::launch_wgrad(ja, jb, m, r, scaling, wpart, msplit, is_f16(W), s) != hipSuccess)
    return QLORA_ERR_HIP;
  return QLORA_OK;
}

}  // extern "C"
