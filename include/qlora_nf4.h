/*
 * qlora_nf4.h -- C ABI of the QLoRA NF4 quantized-linear library (gfx950 / MI355X).
 *
 * The frozen base weight W [n x k] (out_features x in_features) is stored as
 * block-wise 4-bit NF4 with double quantization of the block scales (or in
 * one of the alternate block formats below); the forward and backward of the
 * LoRA-augmented linear layer dequantize it to bf16 (or fp16, see "Compute
 * type") inside the kernels.
 *
 * Pages cited (address and section):
 *   news.rkmt.cn/news/4821   (QLoRA double / block-wise quantization)
 *   zky001.github.io/llm-training-guide/docs/post-training/qlora (section 5.8)
 *   kwkr.cn/news/627310      (quantized vs. non-quantized)
 *   www.lqnn.cn/news/228537  (course notes: quantization + LoRA)
 *   www.cf-1.com/news/5705389 (LoRA training on a quantized base)
 *
 * Conventions for every entry point
 *   - Device pointers are owned by the caller; the library never allocates,
 *     frees or synchronizes.  Work is enqueued on `stream` (a hipStream_t, or
 *     NULL for the null stream) and is ordered with other work on it.
 *   - Matrices are row-major and contiguous.  bf16 and fp16 tensors are passed
 *     as raw 16-bit patterns (uint16_t).
 *   - codes, X, Y, dY and dX must be 16-byte aligned; every other device
 *     pointer 4-byte aligned.
 *   - k % 64 == 0; m >= 1 and n >= 1 are arbitrary (ragged tails are masked);
 *     m <= QLORA_MAX_M (2^31 - 1), n < 2^22, k < 2^22 and a packed weight
 *     holds fewer than 2^38 elements (n * k / 64 < 2^32 blocks).
 *   - r == 0 switches the LoRA branch off: A, B, T_save, T_saved, dA and dB
 *     are then ignored and may be NULL.
 *   - All arguments are validated before any HIP call; on error nothing is
 *     enqueued and a positive status is returned.  A failed launch returns
 *     QLORA_ERR_HIP.  Asynchronous faults surface at the caller's next
 *     synchronization.  Non-finite weights are outside the contract (no check).
 *   - The library keeps no state between calls (apart from once-per-process
 *     kernel attributes and the per-GPU scratch of qlora_linear_fwd_noalloc):
 *     calls are re-entrant and thread-safe; two calls that write the same
 *     buffers race, and so do overlapping qlora_linear_fwd_noalloc calls on
 *     one GPU.
 *   - Results are deterministic: the same inputs give the same bits.
 */
#ifndef QLORA_NF4_H
#define QLORA_NF4_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* status codes */
enum {
  QLORA_OK = 0,
  QLORA_ERR_NULL = 1,      /* a required pointer is NULL */
  QLORA_ERR_SHAPE = 2,     /* m, n or k <= 0, k % 64 != 0, or descriptor sizes mismatch */
  QLORA_ERR_ALIGN = 3,     /* a pointer is not aligned as required */
  QLORA_ERR_DTYPE = 4,     /* unknown dtype enum, or one the weight does not allow */
  QLORA_ERR_RANK = 5,      /* LoRA rank r < 0 or r > QLORA_MAX_RANK */
  QLORA_ERR_WORKSPACE = 6, /* workspace NULL or smaller than qlora_workspace_bytes() */
  QLORA_ERR_HIP = 7,       /* a HIP launch failed */
  QLORA_ERR_ARG = 8        /* another argument is out of range (path, op) */
};

/* dtypes: of outputs (y_dtype, dx_dtype) and the compute type (qlora_nf4.dtype) */
enum { QLORA_F32 = 0, QLORA_BF16 = 1, QLORA_F16 = 2 };

/* path selection for qlora_linear_fwd / qlora_linear_bwd */
enum {
  QLORA_PATH_AUTO = 0, /* by m: split-K streaming path for small m, MFMA GEMM otherwise */
  QLORA_PATH_GEMV = 1, /* force the small-m streaming path (m <= QLORA_GEMV_MAX_M, else
                          QLORA_ERR_ARG); in the backward it computes dX */
  QLORA_PATH_GEMM = 2  /* force the tiled MFMA GEMM path */
};

/* weight formats (qlora_nf4.format; 0, the NF4 format, when zero-initialized) */
enum {
  QLORA_FMT_NF4 = 0,     /* NF4 codes, double-quantized or single-level scales */
  QLORA_FMT_U4_ASYM = 1, /* asymmetric 4-bit min/max blocks of 64, fp32 scale + zero-point */
  QLORA_FMT_Q8_0 = 2     /* int8 blocks of 32 with an fp16 scale */
};

#define QLORA_BLOCK 64        /* weights per first-level block   (news.rkmt.cn/news/4821 §1.2) */
#define QLORA_GROUP 256       /* block scales per second-level group (news.rkmt.cn/news/4821 §2.2) */
#define QLORA_MAX_RANK 128    /* largest supported LoRA rank */
#define QLORA_GEMV_MAX_M 32   /* largest m the streaming path accepts */
#define QLORA_CODEBOOK_LEN 31 /* 16 NF4 levels then 15 decision midpoints */
#define QLORA_MAX_M 2147483647LL /* largest token count m (2^31 - 1) */

/*
 * Packed NF4 + double-quantized weight (device buffers owned by the caller).
 * Flat block b = row * (k/64) + kb covers elements [64b, 64b+64) of the
 * row-major weight; group g covers flat blocks [256g, 256g+256).  Sizes come
 * from qlora_nf4_bytes().
 *   codes : n*k/2 bytes, 32 per block.  Inside a block, the 4-byte word w
 *           holds elements 8w..8w+7: byte j (j = 0..3) is
 *           code(8w+j) | code(8w+j+4) << 4.
 *   qscale: n*k/64 bytes, the block absmax quantized to 8 bits.
 *   step  : ceil(n*k/16384) floats, the fp32 second-level constant per group,
 *           indexed by flat group.
 * Storage order of the blocks in codes and qscale: rows are taken in groups
 * of 16 (the last group holds R = n mod 16 rows if that is not 0, else 16);
 * inside a group the blocks are ordered by kb, then by row, so block
 * (row, kb) sits at position g0*(k/64) + kb*R + (row - g0), g0 = 16*(row/16).
 * The 16 rows of a group are contiguous at every kb, which lets the kernels
 * read a group's codes as one coalesced run.
 * Dequantized weight: w = bf16_rne(level[code] * fp32(qscale_b * step_g)).
 * (news.rkmt.cn/news/4821 §1.3, §2.2, §2.3; zky001 section 5.8 "double quantization")
 *
 * Single-level format (no double quantization; news.rkmt.cn/news/4821 §1.2,
 * §2.3: one fp32 scale per 64-block, 0.5 bit per weight): qscale = NULL and
 * step holds n*k/64 floats, the fp32 absmax of each block at the block's
 * storage position (the order above); w = bf16_rne(level[code] * absmax_b).
 *
 * Alternate formats.  The weight is cut into 64-weight units (one row, 64
 * consecutive k: the NF4 block) stored in the order above, unit (row, kb) at
 * position p.
 *   QLORA_FMT_U4_ASYM (news.rkmt.cn/news/4821 §1.3, §2.1; kwkr.cn/news/627310
 *     §2.1): per 64-block lo = min(min, 0), hi = max(max, 0),
 *     scale = fp32(fp32(hi - lo) / 15), zp = clamp(rint_even(-lo * 15 / (hi - lo)),
 *     0, 15) evaluated in binary64 from the range (the reading that reproduces
 *     kwkr.cn/news/627310 §2.1's printed zero-point), q = clamp(rint_even(fp32(x /
 *     scale)) + zp, 0, 15) (all 0 when
 *     scale is 0); w = bf16_rne(fp32(scale * (q - zp))).  codes: n*k/2 bytes,
 *     q packed as the NF4 codes; step: 2*n*k/64 floats, step[2p] = scale,
 *     step[2p+1] = zp (an integer value); qscale must be NULL.  8-byte aligned
 *     step.
 *   QLORA_FMT_Q8_0 (www.cf-1.com/news/5705389 §1.1, §2.2; symmetric scale of
 *     kwkr.cn/news/627310 §2.1): per 32-block d16 = fp16_rne(fp32(absmax / 127)),
 *     q = clamp(rint_even(fp32(x / d16)), -127, 127) (0 when d16 is 0);
 *     w = bf16_rne(d16 * q).  codes: n*k bytes, 64 per unit, byte e of unit p
 *     the int8 q of its element e; qscale: 4*n*k/64 bytes, the fp16 scales
 *     (little-endian binary16) of the unit's elements 0-31 at bytes [4p, 4p+2)
 *     and 32-63 at [4p+2, 4p+4); step is unused (may be NULL).  Blocks with
 *     absmax above 127 * 65504 are outside the contract.
 * NF4 at other block sizes (block = 32 or 128; news.rkmt.cn/news/4821 §1.2:
 * smaller blocks quantize more finely and cost more constants): every step
 * above runs on blocks of that many consecutive weights of a row; codes keep
 * the 64-weight unit layout and order; second-level groups still hold 256
 * block scales (flat block index b = row * (k/block) + kb).  Scale entries
 * (qscale bytes, or single-level fp32 absmax in step): block 32 stores the
 * unit's two scales at 2p and 2p + 1; block 128 stores one scale per pair of
 * units, block (row, kb) at g0*(k/128) + kb*R + (row - g0).  Block 128 needs
 * k % 128 == 0 and block 32 n*k < 2^37.  Sizes from qlora_nf4_block_bytes.
 * The codebook argument of every entry point is used by (and required for)
 * the NF4 format only.  Every entry point accepts every format; a grouped
 * forward needs one format (and for NF4 one scale level) for all its jobs.
 *
 * Compute type (news.rkmt.cn/news/4821 §3.3: the compute dtype is float16 or
 * bfloat16; kwkr.cn/news/627310 §4.3: fp16 where bf16 is not supported).
 * dtype = QLORA_BF16 (or 0) is the default: every 16-bit tensor is bf16.
 * dtype = QLORA_F16, allowed for NF4 at block 64 with double quantization
 * only (else QLORA_ERR_DTYPE): the weight handed to qlora_quantize, X, A, B,
 * dY, the dequantized and merged weights and every 16-bit output are IEEE
 * fp16; the dequantized weight is w = fp16_rne(level[code] * s'), subnormals
 * kept, and the products run on fp16 operands with fp32 accumulation.  The
 * codes and scales are computed the same way from the exact fp32 values, so
 * a weight exact in both types packs to the same bytes.  Values beyond the
 * fp16 range (65504), in inputs or results, are outside the contract.
 * A 16-bit y_dtype / dx_dtype must name the compute type (QLORA_BF16 for
 * bf16, QLORA_F16 for fp16); QLORA_F32 is always allowed.
 */
typedef struct {
  int64_t n;       /* out_features */
  int64_t k;       /* in_features, k % 64 == 0 */
  uint8_t *codes;
  uint8_t *qscale;
  float *step;
  int32_t format;  /* QLORA_FMT_* */
  int32_t block;   /* NF4 block size: 0 or 64 (default), 32 or 128; 0 or 64 for other formats */
  int32_t dtype;   /* compute type: 0 or QLORA_BF16 (default), or QLORA_F16 (see above) */
} qlora_nf4;

/*
 * Host.  Writes the NF4 table to out[0..30]: 16 ascending levels in [-1, 1]
 * (level 0 at index 7, exactly 0), then the 15 decision midpoints, midpoint i
 * being the largest fp32 not above (level[i] + level[i+1]) / 2.  Levels are
 * standard-normal quantiles normalised to [-1, 1], 8 positive and 7 negative
 * plus an exact zero (zky001 section 5.8 "NF4"; kwkr.cn/news/627310 §2.1 on
 * the exact zero).  Copy it to the device and pass it as `codebook` below.
 * Returns QLORA_ERR_NULL if out is NULL.
 */
int qlora_nf4_codebook(float *out);

/*
 * Host.  Byte sizes of the three arrays of an n x k packed weight
 * (news.rkmt.cn/news/4821 §2.3: 4-bit codes + 8-bit scale per 64 + fp32 per
 * 256 scales).  Any output pointer may be NULL.  QLORA_ERR_SHAPE unless
 * n >= 1, k >= 64, k % 64 == 0, n < 2^22, k < 2^22 and n * k < 2^38.
 */
int qlora_nf4_bytes(int64_t n, int64_t k, size_t *codes, size_t *qscale, size_t *step);

/*
 * Host.  Byte sizes of the two arrays of an n x k weight in the single-level
 * format: codes n*k/2, absmax (passed as `step`) 4*n*k/64.  Errors as
 * qlora_nf4_bytes.
 */
int qlora_nf4_single_bytes(int64_t n, int64_t k, size_t *codes, size_t *absmax);

/*
 * Host.  Byte sizes of the arrays of an n x k NF4 weight with blocks of
 * `block` weights (32, 64 or 128), with (double_quant != 0) or without double
 * quantization: codes n*k/2; double-quantized: qscale n*k/block, step
 * 4*ceil(n*k/block/256); single level: qscale 0, step 4*n*k/block.
 * QLORA_ERR_ARG for another block, QLORA_ERR_SHAPE as qlora_nf4_bytes or when
 * the block's limits above are not met.
 */
int qlora_nf4_block_bytes(int64_t n, int64_t k, int block, int double_quant, size_t *codes,
                          size_t *qscale, size_t *step);

/*
 * Host.  Byte sizes of the three arrays of an n x k weight in `format`
 * (QLORA_FMT_NF4: the double-quantized sizes of qlora_nf4_bytes); arrays the
 * format does not use get 0.  Errors as qlora_nf4_bytes, QLORA_ERR_ARG for an
 * unknown format.
 */
int qlora_weight_bytes(int format, int64_t n, int64_t k, size_t *codes, size_t *qscale,
                       size_t *step);

/*
 * Host.  Workspace bytes needed by qlora_linear_fwd (op = 0) or
 * qlora_linear_bwd (op = 1) for these sizes, for any path.  0 on bad input
 * (an unknown op, m outside [1, QLORA_MAX_M], a shape qlora_nf4_bytes refuses,
 * r outside [0, QLORA_MAX_RANK]).
 */
size_t qlora_workspace_bytes(int op, int64_t m, int64_t n, int64_t k, int r);

/*
 * Quantize a 16-bit weight W [n x k] (device; bf16, or fp16 when out->dtype is
 * QLORA_F16) into `out` (device arrays sized by
 * qlora_nf4_bytes, out->n and out->k set).  Block-wise absmax scaling over 64
 * elements, nearest NF4 level of the binary32 quotient w / absmax (ties to the
 * lower level; an all-zero block gives level 0), then double quantization:
 * step_g = fp32(c2 / 255) with c2 the largest absmax of the group and
 * qscale_b = min(255, rint_even(fp32(absmax_b / step_g))), 0 when step_g is 0
 * (news.rkmt.cn/news/4821 §1.2, §2.1, §2.2; zky001 section 5.8).
 * With out->qscale == NULL the second level is skipped: the single-level
 * format, the fp32 absmax of each block written to out->step (sized by
 * qlora_nf4_single_bytes).  With out->format an alternate format, the
 * weight is encoded in that format (codebook unused, may be NULL).
 * `codebook` is the device copy of qlora_nf4_codebook().
 */
int qlora_quantize(const uint16_t *W, const float *codebook, const qlora_nf4 *out, void *stream);

/*
 * Dequantize `W` into a dense [n x k] device array `out` of its compute type
 * (bf16, or fp16 for QLORA_F16), with the same
 * arithmetic the linear kernels use internally.  For checking and for merging
 * an adapter into the base (www.lqnn.cn/news/228537 §3.3), not for the linear
 * layer itself, which never materializes the 16-bit weight.
 */
int qlora_dequantize(const qlora_nf4 *W, const float *codebook, uint16_t *out, void *stream);

/*
 * Plain layout of a packed weight, for exchange with code that knows only the
 * pages' description (news.rkmt.cn/news/4821 §4.2: the 4-bit codes live two
 * per uint8 byte; §1.2, §2.2: one constant per block of the flat row-major
 * weight and one per group of 256 block constants).  The same arrays with
 * the same sizes as the layout above, every byte in flat row-major order:
 *   codes, 4-bit formats: byte j = code(2j) | code(2j+1) << 4 over the
 *     row-major elements (the even element in the low nibble);
 *   codes, Q8_0: byte e = the int8 value of element e;
 *   block constants indexed by the flat block b = row * (k/block) + kb:
 *     NF4 double-quantized: qscale[b], and step[g] per group of 256 flat
 *     blocks (already flat above); NF4 single level: step[b] the fp32 absmax;
 *     uint4: step[2b], step[2b+1] = scale, zero-point of 64-block b; Q8_0:
 *     qscale bytes [2b, 2b+2) the little-endian fp16 scale of 32-block b.
 * qlora_to_plain copies `src` (library layout) into `dst` (plain layout);
 * qlora_from_plain copies `src` (plain layout) into `dst` (library layout),
 * which the other entry points then accept.  A descriptor whose arrays hold
 * the plain layout must not be passed anywhere else.  Both descriptors
 * describe the same weight: equal n, k, format, block and compute type, and
 * qscale NULL in both or in neither (QLORA_ERR_SHAPE, QLORA_ERR_ARG,
 * QLORA_ERR_DTYPE otherwise); each must pass the checks of a weight
 * descriptor (sizes, alignment); no array of dst may overlap an array of src
 * (QLORA_ERR_ARG).  Device buffers owned by the caller; one launch on
 * `stream`, no allocation, nothing enqueued on error.
 */
int qlora_to_plain(const qlora_nf4 *src, const qlora_nf4 *dst, void *stream);
int qlora_from_plain(const qlora_nf4 *src, const qlora_nf4 *dst, void *stream);

/*
 * Fold a trained adapter into the base weight (www.lqnn.cn/news/228537 §3.3:
 * dequantize W, add the low-rank branch at high precision, quantize again;
 * www.cf-1.com/news/5705389 §4.3 and kwkr.cn/news/627310 §4.4 on the two
 * precision losses, the 16-bit rounding of the sum and the requantization):
 *     merged[n][k] = rne16(fp32(deq(W)[n][k] + fp32(scaling * acc))),
 *     acc = sum_j B[n][j] A[j][k], accumulated in binary32 in rank order
 *           (j = 0 .. r-1; each product of two 16-bit values is exact).
 * A [r x W.k], B [W.n x r] in W's compute type (device; A 16-byte aligned),
 * r == 0 gives deq(W).  `merged` [W.n x W.k] (device, 16-byte aligned)
 * receives the merged weight in that type (rne16: bf16 or fp16 rounding).  If
 * `out` is not NULL (sizes and compute type equal to W's), the merged weight
 * is then quantized into it, in out->format, exactly as qlora_quantize would.
 * The codebook is required when W or out is NF4.
 */
int qlora_merge(const qlora_nf4 *W, const float *codebook, const uint16_t *A, const uint16_t *B,
                int r, float scaling, uint16_t *merged, const qlora_nf4 *out, void *stream);

/*
 * Forward of the LoRA-augmented quantized linear (www.cf-1.com/news/5705389
 * §2.1, §3.2; www.lqnn.cn/news/228537 §3.2-§3.3):
 *     T = X A^T            [m x r], fp32 (written to T_save if not NULL)
 *     Y = X deq(W)^T + scaling * T B^T      [m x n]
 * X [m x k], A [r x k], B [n x r] in W's compute type (bf16, or fp16),
 * scaling = alpha / r.  The product runs on 16-bit operands with fp32
 * accumulation; T stays fp32.  Y is fp32 (y_dtype QLORA_F32) or the compute
 * type rounded to nearest even (QLORA_BF16, or QLORA_F16 for fp16 compute).
 * ws: device workspace of at least qlora_workspace_bytes(0, m, n, k, r) bytes
 * (may be NULL only if that size is 0).  path: QLORA_PATH_*.  The T written
 * here is the T that qlora_linear_bwd recomputes, bit for bit, when given
 * none (path AUTO).
 */
int qlora_linear_fwd(const qlora_nf4 *W, const float *codebook, const uint16_t *X, int64_t m,
                     const uint16_t *A, const uint16_t *B, int r, float scaling,
                     void *Y, int y_dtype, float *T_save,
                     void *ws, size_t ws_bytes, int path, void *stream);

/*
 * Allocation-free variant of qlora_linear_fwd, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc): the same arguments without `ws` and
 * `ws_bytes`, the same kernels and results bit for bit.  Its workspace is a
 * file-scope device array of QLORA_NOALLOC_SCRATCH_BYTES (64 MiB) per GPU,
 * which every GPU the library is loaded on holds until the process ends; it
 * calls no allocation routine.  Calls whose workspace would exceed that size
 * (qlora_workspace_bytes(0, ...) counts it; with T_save given and a shape
 * that needs no split, none is used) return QLORA_ERR_WORKSPACE before any
 * launch.  Every call on a GPU shares that GPU's array and leaves its contents
 * behind (nothing in it needs to start at zero): calls that overlap in time on
 * one GPU (different streams or threads) race on it and must be serialized by
 * the caller.
 */
#define QLORA_NOALLOC_SCRATCH_BYTES (64u << 20)
int qlora_linear_fwd_noalloc(const qlora_nf4 *W, const float *codebook, const uint16_t *X,
                             int64_t m, const uint16_t *A, const uint16_t *B, int r,
                             float scaling, void *Y, int y_dtype, float *T_save, int path,
                             void *stream);

/*
 * Backward of the same layer (www.cf-1.com/news/5705389 §2.1: dL/dx = dL/dy W0^T
 * through the quantized matrix; www.lqnn.cn/news/228537 §3.3 and zky001
 * section 5.8: the frozen base gets no gradient, only A and B):
 *     U  = dY B                          [m x r] fp32
 *     dX = dY deq(W) + scaling * U A     [m x k]  (fp32, or the 16-bit compute type, per dx_dtype)
 *     dA = scaling * U^T X               [r x k]  fp32, overwritten
 *     dB = scaling * dY^T T              [n x r]  fp32, overwritten
 * X, dY, A and B are in W's compute type.  T = X A^T is taken from T_saved
 * ([m x r] fp32, as written by the forward) or recomputed when T_saved is NULL.  dX may be NULL to skip the input gradient;
 * dA/dB are required when r > 0.  path selects how dX is formed: the
 * streaming kernel (QLORA_PATH_GEMV, or QLORA_PATH_AUTO for m <=
 * QLORA_GEMV_MAX_M: the packed weight is read once, rows split across
 * workgroups and their partial sums added in a second pass) or the tiled
 * MFMA GEMM (QLORA_PATH_GEMM, or AUTO above that m); QLORA_ERR_ARG for
 * QLORA_PATH_GEMV with m > QLORA_GEMV_MAX_M.  ws: at least
 * qlora_workspace_bytes(1, m, n, k, r) bytes, which covers every path.
 */
int qlora_linear_bwd(const qlora_nf4 *W, const float *codebook, const uint16_t *X,
                     const uint16_t *dY, int64_t m, const uint16_t *A, const uint16_t *B,
                     int r, float scaling, const float *T_saved,
                     void *dX, int dx_dtype, float *dA, float *dB,
                     void *ws, size_t ws_bytes, int path, void *stream);

/*
 * Grouped forward for small m (decode): one launch streams the packed weights
 * of many independent projections, so that each projection does not pay a
 * kernel launch of its own.  Same arithmetic as qlora_linear_fwd on the
 * streaming path, except that the contraction is never split (the per-row
 * sums run in one pass) and T comes from one rank-projection launch for all
 * jobs (a split single-projection forward forms T in its split reduce; the
 * two T agree to fp32 rounding, not bit for bit).
 *
 * One job per projection (host struct; the buffers it points to are device
 * memory owned by the caller, with the sizes and alignments of
 * qlora_linear_fwd).  T is required (written) when r > 0.
 */
typedef struct {
  qlora_nf4 w;
  const uint16_t *X; /* [m x w.k], w's compute type */
  const uint16_t *A; /* [r x w.k], NULL when r == 0 */
  const uint16_t *B; /* [w.n x r], NULL when r == 0 */
  int r;
  float scaling;
  void *Y;           /* [m x w.n], the group's y_dtype */
  float *T;          /* [m x r] fp32 */
} qlora_fwd_job;

/* Plain-data handle filled by qlora_group_init; `table` is the caller's device buffer. */
typedef struct {
  void *table;
  int count, lora_count, max_r, y_dtype, variant;   /* variant: the jobs' weight format (internal) */
  int64_t m, row_groups, max_quads;
} qlora_group;

/* Host.  Device bytes of the job table for `count` jobs (0 if count < 1). */
size_t qlora_group_table_bytes(int count);

/*
 * Host, setup time.  Validates every job (QLORA_ERR_* as qlora_linear_fwd,
 * QLORA_ERR_ARG if m > QLORA_GEMV_MAX_M, count < 1 or the jobs' weights mix
 * formats, NF4 scale levels or compute types) and writes the device
 * job table into `table` (16-byte aligned, >= qlora_group_table_bytes(count)
 * bytes) with a blocking host-to-device copy: unlike every other call this
 * one synchronizes.  The buffers named by the jobs must stay valid while the
 * group is used.
 */
int qlora_group_init(qlora_group *g, const qlora_fwd_job *jobs, int count, int64_t m,
                     int y_dtype, void *table, size_t table_bytes);

/*
 * Enqueue the forward of every job of `g` on `stream`: T = X A^T for the jobs
 * with r > 0 (one launch), then Y = X deq(W)^T + scaling T B^T for all jobs
 * (one launch).  No workspace.  Jobs must not write overlapping outputs.
 */
int qlora_linear_fwd_grouped(const qlora_group *g, const float *codebook, void *stream);

/* Host.  Static message for a status code (never NULL). */
const char *qlora_strerror(int status);

#ifdef __cplusplus
}
#endif
#endif /* QLORA_NF4_H */
