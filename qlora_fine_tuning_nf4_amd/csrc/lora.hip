// LoRA branch pieces (www.lqnn.cn/news/228537 §3.2; www.cf-1.com/news/5705389
// §2.1, §3.2): the rank-r projections T = X A^T and U = dY B, and the adapter
// weight gradients dA = s U^T X and dB = s dY^T T.  T and U stay fp32.  The
// 16-bit operands are bf16, or fp16 in the F16 instantiations (compute type,
// news.rkmt.cn/news/4821 §3.3).
#include "common.h"
#include "kernels.h"

namespace ql {

QL_DEV u32x4_t load8_guard(const uint16_t* row, int64_t c, int64_t C, bool vec) {
  if (vec && c + 8 <= C) return *reinterpret_cast<const u32x4_t*>(row + c);
  if (c >= C) return u32x4_t{0u, 0u, 0u, 0u};
  uint32_t h[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) h[e] = (c + e < C) ? row[c + e] : 0u;
  return u32x4_t{h[0] | h[1] << 16, h[2] | h[3] << 16, h[4] | h[5] << 16, h[6] | h[7] << 16};
}

// out[m][j] = sum_c P[m][c] Q[j][c]: a workgroup of 8 waves owns `rows`
// rows (16, or 8 so that a few thousand rows still spread over every compute
// unit) and all r ranks, in RT tiles of 16.  Wave w takes the 32-wide
// contraction slices w, w+8, ..., U at a time; per slice it loads the rows'
// fragment once and one fragment per rank tile and feeds RT MFMAs 16x16x32,
// so P is read once whatever the rank.  With 16-byte rows (VEC) the loads
// are buffer loads whose masked lanes (rows past M, ranks past r, slices
// past the contraction) point past the buffer and read zeros, so there are
// no branches, and two register sets alternate: the next U slices load while
// the current ones are multiplied.  The 8 partial tiles are summed in a
// fixed order through LDS.  16-bit products are exact, sums fp32.  PAIR (rows == 8,
// r <= 8, one rank tile): the idle upper halves of the 16 x 16 MFMA tile carry
// a second contraction slice -- lanes 8-15 of each operand load rows / ranks
// 0-7 of the next slice, the two diagonal 8 x 8 blocks of D are both valid
// (the off-diagonal ones are cross terms and ignored) and are added at the
// end -- so every load and MFMA does useful work on all 16 lanes.
constexpr int RD_WAVES = 8;
template <int RT, bool GROUPED, bool VEC, bool F16, bool PAIR = false>
__global__ __launch_bounds__(512) void k_rowdot(const uint16_t* __restrict__ P,
                                                const uint16_t* __restrict__ Q, int64_t M,
                                                int64_t C, int r, float* __restrict__ out,
                                                const RowdotJob* __restrict__ jobs, int rows) {
  if constexpr (GROUPED) {
    const RowdotJob& J = jobs[blockIdx.z];
    P = J.P;
    Q = J.Q;
    out = J.out;
    C = J.C;
    r = J.r;
  }
  __shared__ f32x4_t s_red[RD_WAVES - 1][RT][64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int li = lane & 15, g = lane >> 4;
  const int64_t m0 = (int64_t)blockIdx.x * rows;
  f32x4_t acc[RT];
#pragma unroll
  for (int t = 0; t < RT; ++t) acc[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  constexpr int U = RT <= 2 ? 6 : (RT == 4 ? 4 : 2);   // slices per round (register budget)
  constexpr int64_t stride = 32 * RD_WAVES;            // elements between a wave's slices
  if constexpr (VEC) {
    constexpr uint32_t kOut = 0x80000000u;
    const int nr = (int)min((int64_t)rows, M - m0);
    const auto prs = buf_rsrc(P + m0 * C, rsrc_bytes((int64_t)nr * C * 2));
    const auto qrs = buf_rsrc(Q, rsrc_bytes((int64_t)r * C * 2));
    const int lrow = PAIR ? (li & 7) : li;                // row / rank of this lane's operands
    const uint32_t pbase = lrow < nr ? (uint32_t)(lrow * C * 2) : kOut;
    uint32_t qbase[RT];
#pragma unroll
    for (int t = 0; t < RT; ++t) {
      const int j = 16 * t + lrow;
      qbase[t] = j < r ? (uint32_t)(j * C * 2) : kOut;
    }
    // PAIR: slices u and u + 1 of a round share an MFMA (lanes 8-15 the second)
    constexpr int SU = PAIR ? 2 : 1;
    const int64_t half = PAIR ? (li >> 3) * stride : 0;
    auto ld_round = [&](int64_t c0, u32x4_t (&a)[U], u32x4_t (&b)[U][RT]) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int64_t c = c0 + u * SU * stride + half + 8 * g;
        const bool cok = c < C;
        const uint32_t co = (uint32_t)(c * 2);
        a[u] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(prs, cok ? pbase + co : kOut, 0, 0));
#pragma unroll
        for (int t = 0; t < RT; ++t)
          b[u][t] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(qrs, cok ? qbase[t] + co : kOut, 0, 0));
      }
    };
    auto mma_round = [&](const u32x4_t (&a)[U], const u32x4_t (&b)[U][RT]) {
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int t = 0; t < RT; ++t) acc[t] = mfma16x16x32<F16>(a[u], b[u][t], acc[t]);
    };
    u32x4_t a0[U], b0[U][RT], a1[U], b1[U][RT];
    int64_t c0 = wave * 32;
    constexpr int64_t RS = U * SU * stride;               // elements per round
    ld_round(c0, a0, b0);
    for (; c0 < C; c0 += 2 * RS) {
      ld_round(c0 + RS, a1, b1);
      mma_round(a0, b0);
      ld_round(c0 + 2 * RS, a0, b0);
      mma_round(a1, b1);
    }
  } else {
    const int64_t m = m0 + li;
    const bool mok = li < rows && m < M;
    const uint16_t* prow = P + (mok ? m : 0) * C;
    for (int64_t c0 = wave * 32; c0 < C; c0 += U * stride) {
      u32x4_t a[U], b[U][RT];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int64_t c = c0 + u * stride + g * 8;
        a[u] = mok ? load8_guard(prow, c, C, false) : u32x4_t{0u, 0u, 0u, 0u};
#pragma unroll
        for (int t = 0; t < RT; ++t) {
          const int j = 16 * t + li;
          b[u][t] = j < r ? load8_guard(Q + (int64_t)j * C, c, C, false) : u32x4_t{0u, 0u, 0u, 0u};
        }
      }
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int t = 0; t < RT; ++t) acc[t] = mfma16x16x32<F16>(a[u], b[u][t], acc[t]);
    }
  }
  if (wave > 0) {
#pragma unroll
    for (int t = 0; t < RT; ++t) s_red[wave - 1][t][lane] = acc[t];
  }
  __syncthreads();
  if (wave != 0) return;
  for (int w = 0; w < RD_WAVES - 1; ++w)
#pragma unroll
    for (int t = 0; t < RT; ++t) acc[t] += s_red[w][t][lane];
  if constexpr (PAIR) {
    // D[m][j] for m, j < 8 (lanes g < 2, li < 8) plus the second slice's
    // block D[m + 8][j + 8] (lane + 40)
#pragma unroll
    for (int e = 0; e < 4; ++e) acc[0][e] += __shfl(acc[0][e], (lane + 40) & 63);
  }
#pragma unroll
  for (int t = 0; t < RT; ++t) {
    const int j = 16 * t + li;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int64_t mm = m0 + g * 4 + e;
      if (g * 4 + e < rows && mm < M && j < r && (!PAIR || li < 8)) out[mm * r + j] = acc[t][e];
    }
  }
}

// Large-M rank projection, out[m][j] = sum_c P[m][c] Q[j][c], for 16-byte
// rows (C % 8 == 0, aligned bases) and 16 < r <= 64, or r <= 64 with Q read
// in place from its transpose.  Every row tile reads all of
// Q, so Q is shared through LDS: a workgroup of 8 waves owns 128 rows (wave
// w: rows 16w .. 16w+15) and the contraction range of its split, walked in
// chunks of CH columns.  Each chunk of Q (16 RT ranks x CH bf16, rows padded
// by 16 bytes so that the 16 rows of a fragment read fall on distinct bank
// groups) is staged once and read by the 8 waves, which load their own rows
// of P as buffer loads (masked lanes read zeros past the buffer).  The next
// chunk's loads are issued before the current chunk's MFMAs 16x16x32, with
// one barrier per chunk (two LDS buffers).  With several splits each one
// writes its sums to part[split][m][j] and k_rowdot_reduce adds them in
// split order; with one split the sums go to out.
constexpr int RS_ROWS = 128;
template <int RT>
struct RsGeo {
  static constexpr int CH = RT <= 2 ? 256 : 128;      // columns per chunk
  static constexpr int PITCH = CH + 8;                // LDS row pitch (bf16)
  static constexpr int QL = RT * CH / 256;            // 16-byte Q pieces per thread and chunk
  static constexpr int XS = CH / 32;                  // slices per wave and chunk
};

template <int RT, bool F16, bool QT = false>
__global__ __launch_bounds__(512) void k_rowdot_sk(const uint16_t* __restrict__ P,
                                                   const uint16_t* __restrict__ Q, int64_t M,
                                                   int64_t C, int r, float* __restrict__ out,
                                                   float* __restrict__ part, int nsplit,
                                                   int chunks_per_split) {
  using G = RsGeo<RT>;
  constexpr int CH = G::CH, PITCH = G::PITCH, QL = G::QL, XS = G::XS;
  constexpr uint32_t kOut = 0x80000000u;
  __shared__ __attribute__((aligned(16))) uint16_t sQ0[16 * RT * PITCH];
  __shared__ __attribute__((aligned(16))) uint16_t sQ1[16 * RT * PITCH];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int li = lane & 15, g = lane >> 4;
  const int64_t m0 = (int64_t)blockIdx.x * RS_ROWS;
  const int split = blockIdx.y;
  const int64_t c_begin = (int64_t)split * chunks_per_split * CH;
  const int64_t c_end = min(C, c_begin + (int64_t)chunks_per_split * CH);
  const int nch = c_begin < c_end ? (int)((c_end - c_begin + CH - 1) / CH) : 0;

  const int nr = (int)min((int64_t)RS_ROWS, M - m0);
  const auto prs = buf_rsrc(P + m0 * C, rsrc_bytes((int64_t)nr * C * 2));
  const auto qrs = buf_rsrc(Q, rsrc_bytes((int64_t)r * C * 2));
  const int prow = 16 * wave + li;
  const uint32_t pbase = prow < nr ? (uint32_t)(prow * C * 2) : kOut;

  // Q pieces of this thread: piece i covers chunk row q / (CH/8), 8 columns
  // from 8 (q % (CH/8)), q = tid + 512 i.  QT (Q given as Qs [C x r], r % 8
  // == 0): piece i is ranks 8 (q % (2 RT)) .. +7 of chunk column q / (2 RT),
  // one 16-byte load of a Qs row, stored transposed into the stage.
  auto load_q = [&](int64_t cb, u32x4_t (&v)[QL]) {
#pragma unroll
    for (int i = 0; i < QL; ++i) {
      const int q = tid + 512 * i;
      if constexpr (QT) {
        const int j8 = 8 * (q % (2 * RT));
        const int64_t c = cb + q / (2 * RT);
        const bool ok = j8 < r && c < c_end;
        v[i] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(
                                              qrs, ok ? (uint32_t)((c * r + j8) * 2) : kOut, 0, 0));
      } else {
        const int j = q / (CH / 8);
        const int64_t c = cb + 8 * (q % (CH / 8));
        const bool ok = j < r && c < c_end;
        v[i] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(
                                              qrs, ok ? (uint32_t)((j * C + c) * 2) : kOut, 0, 0));
      }
    }
  };
  auto store_q = [&](const u32x4_t (&v)[QL], uint16_t* sq) {
#pragma unroll
    for (int i = 0; i < QL; ++i) {
      const int q = tid + 512 * i;
      if constexpr (QT) {
        const int j8 = 8 * (q % (2 * RT)), cl = q / (2 * RT);
#pragma unroll
        for (int e = 0; e < 8; ++e)
          sq[(j8 + e) * PITCH + cl] = (uint16_t)(e & 1 ? v[i][e >> 1] >> 16 : v[i][e >> 1] & 0xFFFFu);
      } else {
        *reinterpret_cast<u32x4_t*>(sq + (q / (CH / 8)) * PITCH + 8 * (q % (CH / 8))) = v[i];
      }
    }
  };
  auto load_x = [&](int64_t cb, u32x4_t (&x)[XS]) {
#pragma unroll
    for (int k = 0; k < XS; ++k) {
      const int64_t c = cb + 32 * k + 8 * g;
      x[k] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(
                                            prs, c < c_end ? pbase + (uint32_t)(c * 2) : kOut, 0, 0));
    }
  };
  f32x4_t acc[RT];
#pragma unroll
  for (int t = 0; t < RT; ++t) acc[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  auto compute = [&](const uint16_t* sq, const u32x4_t (&x)[XS]) {
#pragma unroll
    for (int k = 0; k < XS; ++k)
#pragma unroll
      for (int t = 0; t < RT; ++t) {
        const u32x4_t b = *reinterpret_cast<const u32x4_t*>(sq + (16 * t + li) * PITCH + 32 * k + 8 * g);
        acc[t] = mfma16x16x32<F16>(x[k], b, acc[t]);
      }
  };

  u32x4_t qa[QL], qb[QL], xa[XS], xb[XS];
  int64_t cb = c_begin;
  if (nch > 0) {
    load_q(cb, qa);
    load_x(cb, xa);
  }
  for (int ch = 0; ch < nch; ch += 2) {
    store_q(qa, sQ0);
    __syncthreads();
    if (ch + 1 < nch) {
      load_q(cb + CH, qb);
      load_x(cb + CH, xb);
    }
    compute(sQ0, xa);
    if (ch + 1 < nch) {
      store_q(qb, sQ1);
      __syncthreads();
      if (ch + 2 < nch) {
        load_q(cb + 2 * CH, qa);
        load_x(cb + 2 * CH, xa);
      }
      compute(sQ1, xb);
    }
    cb += 2 * CH;
  }

  // D[4g + e][li]: rows m0 + 16 wave + 4g + e, rank 16t + li
#pragma unroll
  for (int t = 0; t < RT; ++t) {
    const int j = 16 * t + li;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int64_t m = m0 + 16 * wave + 4 * g + e;
      if (m < M && j < r) {
        if (nsplit > 1)
          part[((int64_t)split * M + m) * r + j] = acc[t][e];
        else
          out[m * r + j] = acc[t][e];
      }
    }
  }
}

// out[i] = sum_s part[s][i] over n values, in split order; four values per
// thread (16-byte accesses when n % 4 == 0 and out is 16-byte aligned), eight
// splits' loads in flight.
__global__ __launch_bounds__(256) void k_rowdot_reduce(const float* __restrict__ part, int nsplit,
                                                       int64_t n, float* __restrict__ out) {
  const int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
  if (i >= n) return;
  f32x4_t v = f32x4_t{0.f, 0.f, 0.f, 0.f};
  if (n % 4 == 0 && (reinterpret_cast<uintptr_t>(out) & 15) == 0) {
    int s = 0;
    for (; s + 8 <= nsplit; s += 8) {
      f32x4_t t[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) t[u] = *reinterpret_cast<const f32x4_t*>(part + (int64_t)(s + u) * n + i);
#pragma unroll
      for (int u = 0; u < 8; ++u) v += t[u];
    }
    for (; s < nsplit; ++s) v += *reinterpret_cast<const f32x4_t*>(part + (int64_t)s * n + i);
    *reinterpret_cast<f32x4_t*>(out + i) = v;
  } else {
    for (int s = 0; s < nsplit; ++s)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (i + e < n) v[e] += part[(int64_t)s * n + i + e];
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (i + e < n) out[i + e] = v[e];
  }
}

// Qt[j][n] = Q[n][j]; thread (j, n) with n fastest, so the writes coalesce
// (N * r < 2^31).
__global__ void k_transpose_bf16(const uint16_t* __restrict__ Q, int N, int r,
                                 uint16_t* __restrict__ Qt) {
  const int n = (int)blockIdx.x * 256 + (int)threadIdx.x, j = (int)blockIdx.y;
  if (n < N) Qt[(int64_t)j * N + n] = Q[(int64_t)n * r + j];
}

typedef float f32x16_t __attribute__((ext_vector_type(16)));

template <bool F16>
QL_DEV f32x16_t mfma32x32x16(const u32x4_t a, const u32x4_t b, f32x16_t c) {
  if constexpr (F16)
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8_t, a),
                                                  __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

// Weight gradient of the adapter on the matrix cores:
//   out = scaling * sum_m Q[m][j] P[m][c]   (P 16-bit [M x C], Q fp32 [M x r])
// written as out[j][c] ([r x C]) or, transposed, out[c][j] ([C x r]); with
// msplit > 1 split s writes its unscaled sum over rows
// [s * rows_per_split, +rows_per_split) to part[s][j][c] for k_wgrad_reduce.
// One launch serves both products of a backward (dA: P = X, Q = U; dB: P = dY,
// Q = T): column tiles [0, tiles_a) belong to job a, the rest to job b, whose
// partials follow job a's (msplit * r * C_a floats).
// A workgroup of 4 waves owns 32*JT ranks x 128 columns and walks its rows
// in chunks of 64.  Each chunk of P (64 x 128) and of Q (64 x 32*JT fp32,
// split into 16-bit parts of P's type, hi = rne(q) and lo = rne(q - hi),
// which carry q to about 2^-16 for bf16, 2^-22 for fp16 above its subnormal
// range) is staged in LDS; the contraction m runs down the stage rows, so
// wave w reads its 32 columns of P and every rank tile of Q with the
// transposing ds_read_b64_tr_b16 and accumulates the hi and lo products with
// MFMA 32x32x16 (16-bit products exact, sums fp32).  The next
// chunk's global loads are issued before the current chunk's MFMAs.  320- and
// 192-byte stage rows keep the 4-row footprints of a transposing read on
// disjoint banks.
constexpr int WG_CHUNK = 64;
template <int JT, bool F16>
__global__ __launch_bounds__(256) void k_wgrad(WgradJob ja, WgradJob jb, int tiles_a, int64_t M,
                                               int r, float scaling, float* __restrict__ part,
                                               int msplit, int rows_per_split) {
  const bool second = (int)blockIdx.x >= tiles_a;
  const WgradJob& J = second ? jb : ja;
  const uint16_t* __restrict__ P = J.P;
  const float* __restrict__ Q = J.Q;
  const int64_t C = J.C;
  float* __restrict__ out = J.out;
  const int transpose_out = J.transpose_out;
  if (second) part += (int64_t)msplit * r * ja.C;
  constexpr int JW = 32 * JT;              // ranks per workgroup tile
  constexpr int LDP = 128 + 32;            // stage pitches (bf16 elements)
  constexpr int LDQ = JW + 32;
  constexpr int QV = JW / 4;               // float4 pieces per Q chunk row
  constexpr int QPASS = WG_CHUNK * QV / 256;
  __shared__ __attribute__((aligned(16))) uint16_t sP[WG_CHUNK * LDP];
  __shared__ __attribute__((aligned(16))) uint16_t sQh[WG_CHUNK * LDQ];
  __shared__ __attribute__((aligned(16))) uint16_t sQl[WG_CHUNK * LDQ];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t c0 = (int64_t)(second ? (int)blockIdx.x - tiles_a : (int)blockIdx.x) * 128;
  const int split = blockIdx.y;
  const int j0 = blockIdx.z * JW;
  const int64_t m_begin = (int64_t)split * rows_per_split;
  const int64_t m_end = min(M, m_begin + rows_per_split);
  const bool pvec = (C % 8) == 0;
  const bool qvec = (r % 4) == 0 && (reinterpret_cast<uintptr_t>(Q) & 15) == 0;

  // this thread's pieces of a chunk: P rows (tid >> 4) + 16 i, columns
  // 8 (tid & 15); Q rows (tid / QV) + (256 / QV) i, ranks 4 (tid % QV)
  const int p_row = tid >> 4, p_col = 8 * (tid & 15);
  const int q_row = tid / QV, q_j = 4 * (tid % QV);
  u32x4_t pr[4];
  f32x4_t qr[QPASS];
  auto load = [&](int64_t mb) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int64_t m = mb + p_row + 16 * i;
      pr[i] = m < m_end ? load8_guard(P + m * C, c0 + p_col, C, pvec) : u32x4_t{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int i = 0; i < QPASS; ++i) {
      const int64_t m = mb + q_row + (256 / QV) * i;
      const int j = j0 + q_j;
      f32x4_t v = f32x4_t{0.f, 0.f, 0.f, 0.f};
      if (m < m_end) {
        const float* qp = Q + m * r + j;
        if (qvec && j + 4 <= r) {
          v = *reinterpret_cast<const f32x4_t*>(qp);
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] = j + e < r ? qp[e] : 0.f;
        }
      }
      qr[i] = v;
    }
  };
  auto store = [&]() {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      *reinterpret_cast<u32x4_t*>(sP + (p_row + 16 * i) * LDP + p_col) = pr[i];
#pragma unroll
    for (int i = 0; i < QPASS; ++i) {
      const f32x4_t v = qr[i];
      const uint32_t h01 = pack16x2<F16>(v[0], v[1]), h23 = pack16x2<F16>(v[2], v[3]);
      const uint32_t l01 = pack16x2<F16>(v[0] - lo16<F16>(h01), v[1] - hi16<F16>(h01));
      const uint32_t l23 = pack16x2<F16>(v[2] - lo16<F16>(h23), v[3] - hi16<F16>(h23));
      const int o = (q_row + (256 / QV) * i) * LDQ + q_j;
      *reinterpret_cast<u32x2_t*>(sQh + o) = u32x2_t{h01, h23};
      *reinterpret_cast<u32x2_t*>(sQl + o) = u32x2_t{l01, l23};
    }
  };

  f32x16_t acc[JT];
#pragma unroll
  for (int t = 0; t < JT; ++t)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[t][i] = 0.f;

  // transposing fragment read: contraction rows 16 kk .. +15, 32 columns
  // from `col`
  const int G16 = lane >> 4, i16 = lane & 15;
  auto frag = [&](const uint16_t* st, int ld, int kk, int col) {
    const int row = 16 * kk + 8 * (G16 >> 1) + (i16 >> 2);
    const int cc = col + 16 * (G16 & 1) + 4 * (i16 & 3);
    const u32x2_t lo = ds_tr16(st + row * ld + cc);
    const u32x2_t hi = ds_tr16(st + (row + 4) * ld + cc);
    return u32x4_t{lo[0], lo[1], hi[0], hi[1]};
  };

  if (m_begin < m_end) load(m_begin);
  for (int64_t mb = m_begin; mb < m_end; mb += WG_CHUNK) {
    store();
    __syncthreads();
    if (mb + WG_CHUNK < m_end) load(mb + WG_CHUNK);
#pragma unroll
    for (int kk = 0; kk < WG_CHUNK / 16; ++kk) {
      const u32x4_t b = frag(sP, LDP, kk, 32 * wave);
#pragma unroll
      for (int t = 0; t < JT; ++t) {
        acc[t] = mfma32x32x16<F16>(frag(sQh, LDQ, kk, 32 * t), b, acc[t]);
        acc[t] = mfma32x32x16<F16>(frag(sQl, LDQ, kk, 32 * t), b, acc[t]);
      }
    }
    __syncthreads();
  }

  // D[8(i/4) + 4(l/32) + i%4][l%32]: rank rows, column lanes
  const int64_t c = c0 + 32 * wave + (lane & 31);
#pragma unroll
  for (int t = 0; t < JT; ++t)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int j = j0 + 32 * t + 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3);
      if (j >= r || c >= C) continue;
      const float v = acc[t][i];
      if (msplit > 1)
        part[((int64_t)split * r + j) * C + c] = v;
      else if (transpose_out)
        out[c * r + j] = scaling * v;
      else
        out[(int64_t)j * C + c] = scaling * v;
    }
}

// out of both jobs = scaling * (sum of the msplit partials, in split order)
__global__ __launch_bounds__(256) void k_wgrad_reduce(const float* __restrict__ part, int msplit,
                                                      int r, float scaling, WgradJob ja,
                                                      WgradJob jb) {
  int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;   // = j * C + c within its job
  const int64_t na = (int64_t)r * ja.C;
  if (idx >= na + (int64_t)r * jb.C) return;
  const bool second = idx >= na;
  if (second) {
    idx -= na;
    part += (int64_t)msplit * na;
  }
  const int64_t C = second ? jb.C : ja.C;
  float* __restrict__ out = second ? jb.out : ja.out;
  const int transpose_out = second ? jb.transpose_out : ja.transpose_out;
  // partials added in split order; eight loads in flight at a time
  const int64_t stride = (int64_t)r * C;
  float v = 0.f;
  int s = 0;
  for (; s + 8 <= msplit; s += 8) {
    float t[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) t[u] = part[(int64_t)(s + u) * stride + idx];
#pragma unroll
    for (int u = 0; u < 8; ++u) v += t[u];
  }
  for (; s < msplit; ++s) v += part[(int64_t)s * stride + idx];
  const int64_t j = idx / C, c = idx % C;
  if (transpose_out)
    out[c * r + j] = scaling * v;
  else
    out[idx] = scaling * v;
}

template <bool GROUPED, bool VEC, bool F16>
static void rowdot_launch(int max_r, dim3 grid, hipStream_t s, const uint16_t* P, const uint16_t* Q,
                          int64_t M, int64_t C, int r, float* out, const RowdotJob* jobs, int rows) {
  if constexpr (VEC && !GROUPED) {
    if (rows == 8 && max_r <= 8) {
      hipLaunchKernelGGL((k_rowdot<1, false, true, F16, true>), grid, dim3(64 * RD_WAVES), 0, s, P, Q,
                         M, C, r, out, jobs, rows);
      return;
    }
  }
#define QL_RD(RT) \
  hipLaunchKernelGGL((k_rowdot<RT, GROUPED, VEC, F16>), grid, dim3(64 * RD_WAVES), 0, s, P, Q, M, C, r, out, jobs, rows)
  if (max_r <= 16) QL_RD(1);
  else if (max_r <= 32) QL_RD(2);
  else if (max_r <= 64) QL_RD(4);
  else QL_RD(8);
#undef QL_RD
}

template <bool F16, bool QT>
static hipError_t rowdot_any(const uint16_t* P, const uint16_t* Q, int64_t M, int64_t C, int r,
                             float* out, float* part, hipStream_t s) {
  const bool vec = C % 8 == 0 && (reinterpret_cast<uintptr_t>(P) & 15) == 0 &&
                   (reinterpret_cast<uintptr_t>(Q) & 15) == 0;
  const int ns = rowdot_splits(M, C, r, QT);
  const bool split = vec && rowdot_uses_split_path(M, r, QT) && (ns == 1 || part);
  // transposed Q only on the split path (rowdot_t_supported, partials given)
  if (QT && (!split || r % 8 != 0)) return hipErrorInvalidValue;
  if (split) {
    const int64_t tiles = (M + RS_ROWS - 1) / RS_ROWS;
    const int ch = r <= 32 ? RsGeo<2>::CH : RsGeo<4>::CH;
    const int64_t chunks = (C + ch - 1) / ch;
    const int per = (int)((chunks + ns - 1) / ns);
    const dim3 grid((unsigned)tiles, (unsigned)ns);
    if (r <= 16)
      hipLaunchKernelGGL((k_rowdot_sk<1, F16, QT>), grid, dim3(512), 0, s, P, Q, M, C, r, out, part, ns, per);
    else if (r <= 32)
      hipLaunchKernelGGL((k_rowdot_sk<2, F16, QT>), grid, dim3(512), 0, s, P, Q, M, C, r, out, part, ns, per);
    else
      hipLaunchKernelGGL((k_rowdot_sk<4, F16, QT>), grid, dim3(512), 0, s, P, Q, M, C, r, out, part, ns, per);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || ns == 1) return e;
    const int64_t n = M * r;
    hipLaunchKernelGGL(k_rowdot_reduce, dim3((unsigned)((n + 1023) / 1024)), dim3(256), 0, s, part, ns,
                       n, out);
    return hipGetLastError();
  }
  // 8-row tiles when 16-row tiles would leave compute units idle
  const int rows = (M + 15) / 16 < 256 ? 8 : 16;
  const dim3 grid((unsigned)((M + rows - 1) / rows));
  // 16-byte rows: both operands start 16-byte aligned (checked by the caller
  // for X and dY; A and the transposed B are C-element rows)
  if (vec)
    rowdot_launch<false, true, F16>(r, grid, s, P, Q, M, C, r, out, nullptr, rows);
  else
    rowdot_launch<false, false, F16>(r, grid, s, P, Q, M, C, r, out, nullptr, rows);
  return hipGetLastError();
}

hipError_t launch_rowdot(const uint16_t* P, const uint16_t* Q, int64_t M, int64_t C, int r,
                         float* out, float* part, bool f16, hipStream_t s) {
  return f16 ? rowdot_any<true, false>(P, Q, M, C, r, out, part, s)
             : rowdot_any<false, false>(P, Q, M, C, r, out, part, s);
}

hipError_t launch_rowdot_t(const uint16_t* P, const uint16_t* Qs, int64_t M, int64_t C, int r,
                           float* out, float* part, bool f16, hipStream_t s) {
  return f16 ? rowdot_any<true, true>(P, Qs, M, C, r, out, part, s)
             : rowdot_any<false, true>(P, Qs, M, C, r, out, part, s);
}

hipError_t launch_rowdot_grouped(const RowdotJob* jobs, int njobs, int64_t M, int max_r,
                                 bool f16, hipStream_t s) {
  // the jobs' contraction lengths are whole 64-blocks; X and A are 16-byte aligned
  const dim3 grid((unsigned)((M + 15) / 16), 1, (unsigned)njobs);
  if (f16)
    rowdot_launch<true, true, true>(max_r, grid, s, nullptr, nullptr, M, int64_t(0), 0, nullptr, jobs, 16);
  else
    rowdot_launch<true, true, false>(max_r, grid, s, nullptr, nullptr, M, int64_t(0), 0, nullptr, jobs, 16);
  return hipGetLastError();
}

hipError_t launch_transpose_bf16(const uint16_t* Q, int64_t N, int r, uint16_t* Qt, hipStream_t s) {
  hipLaunchKernelGGL(k_transpose_bf16, dim3((unsigned)((N + 255) / 256), (unsigned)r), dim3(256), 0,
                     s, Q, (int)N, r, Qt);
  return hipGetLastError();
}

int wgrad_rows_per_split(int64_t M, int msplit) {
  const int64_t per = (M + msplit - 1) / msplit;
  return (int)((per + WG_CHUNK - 1) / WG_CHUNK * WG_CHUNK);
}

hipError_t launch_wgrad(const WgradJob& a, const WgradJob& b, int64_t M, int r, float scaling,
                        float* part, int msplit, bool f16, hipStream_t s, bool reduce) {
  // splits of whole 64-row chunks; a split past the rows writes a zero partial
  const int rows = wgrad_rows_per_split(M, msplit);
  const int jt = r <= 32 ? 1 : 2;
  const int tiles_a = (int)((a.C + 127) / 128), tiles_b = (int)((b.C + 127) / 128);
  dim3 grid((unsigned)(tiles_a + tiles_b), (unsigned)msplit, (unsigned)((r + 32 * jt - 1) / (32 * jt)));
#define QL_WG(JT, H)                                                                           \
  hipLaunchKernelGGL((k_wgrad<JT, H>), grid, dim3(256), 0, s, a, b, tiles_a, M, r, scaling, part, \
                     msplit, rows)
  if (jt == 1) {
    if (f16) QL_WG(1, true); else QL_WG(1, false);
  } else {
    if (f16) QL_WG(2, true); else QL_WG(2, false);
  }
#undef QL_WG
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || msplit == 1 || !reduce) return e;
  const int64_t total = (int64_t)r * (a.C + b.C);
  hipLaunchKernelGGL(k_wgrad_reduce, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s, part,
                     msplit, r, scaling, a, b);
  return hipGetLastError();
}

// Row m of a rank projection, L[m][j] = sum_c P[m][c] Q_j(c), formed by a
// whole workgroup of 256 threads into lrow[0 .. r) (LDS; www.lqnn.cn/news/
// 228537 §3.2: the low-rank branch).  Thread t takes the 8-column pieces
// 8 t + 2048 i, two pieces' loads issued before their products (16-byte loads;
// rank-major Q: the piece of each rank's row; contraction-major Q: the eight
// 16-byte rows of the piece's columns, eight ranks each), eight ranks at a
// time; products of 16-bit values are exact in fp32; a thread adds its pieces
// in order, a wave's 64 sums are added by a butterfly and the four waves'
// sums in wave order, so the value depends only on the row, Q and C.  red:
// LDS scratch of 32 floats.  Ends with the workgroup synchronized.
template <bool F16>
QL_DEV void rank_row(const RankRow& f, int64_t m, float* lrow, float* red) {
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const bool rank_major = f.qs_c == 1;
  const QL_GLOBAL uint16_t* prow = gptr(f.P + m * f.C);
  for (int jb = 0; jb < f.r; jb += 8) {
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    auto piece = [&](int64_t c, u32x4_t (&qv)[8]) {
#pragma unroll
      for (int i = 0; i < 8; ++i)
        qv[i] = *reinterpret_cast<const QL_GLOBAL u32x4_t*>(
            gptr(rank_major ? f.Q + (jb + i) * f.qs_j + c : f.Q + (c + i) * f.qs_c + jb));
      return *reinterpret_cast<const QL_GLOBAL u32x4_t*>(prow + c);
    };
    auto products = [&](const u32x4_t& pv, const u32x4_t (&qv)[8]) {
      float p[8];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        p[2 * e] = lo16<F16>(pv[e]);
        p[2 * e + 1] = hi16<F16>(pv[e]);
      }
      if (rank_major) {
#pragma unroll
        for (int jj = 0; jj < 8; ++jj)
#pragma unroll
          for (int e = 0; e < 4; ++e)
            acc[jj] += p[2 * e] * lo16<F16>(qv[jj][e]) + p[2 * e + 1] * hi16<F16>(qv[jj][e]);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            acc[2 * q] += p[e] * lo16<F16>(qv[e][q]);
            acc[2 * q + 1] += p[e] * hi16<F16>(qv[e][q]);
          }
      }
    };
    for (int64_t c = 8 * t; c < f.C; c += 4096) {
      u32x4_t q0[8], q1[8];
      const bool two = c + 2048 < f.C;
      const u32x4_t p0 = piece(c, q0);
      u32x4_t p1 = p0;
      if (two) p1 = piece(c + 2048, q1);
      products(p0, q0);
      if (two) products(p1, q1);
    }
#pragma unroll
    for (int jj = 0; jj < 8; ++jj) {
      float v = acc[jj];
#pragma unroll
      for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
      acc[jj] = v;
    }
    if (lane == 0) {
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) red[wave * 8 + jj] = acc[jj];
    }
    __syncthreads();
    if (t < 8) lrow[jb + t] = ((red[t] + red[8 + t]) + red[16 + t]) + red[24 + t];
    __syncthreads();
  }
}

// The split reduce of the small-m streaming paths when the LoRA factor is a
// rank projection formed here: out[m][c] = sum_s part[s][m][c] (split order)
// + scaling sum_j L[m][j] R[c][j], with L = P Q^T.  With C >= 256 a
// workgroup's 256 outputs lie in at most two rows, whose factor rows it forms
// first (rank_row); the workgroup holding column 0 of a row writes that row
// to rank.out when given (T saved by the forward, U for the adapter
// gradients).  16-bit R and out in fp16 when F16, else bf16.
template <bool F16>
__global__ __launch_bounds__(256) void k_reduce_rows(const float* __restrict__ part, int nsplit,
                                                     int64_t M, int64_t C, LoraTerm lora,
                                                     void* __restrict__ out, int out16, RankRow rank) {
  __shared__ float s_l[2 * 64];
  __shared__ float s_red[32];
  const int64_t idx0 = (int64_t)blockIdx.x * 256, idx = idx0 + threadIdx.x;
  const int r = lora.r;
  const int64_t m_first = idx0 / C, m_last = min(M - 1, (idx0 + 255) / C);
  // this output's first eight split partials are loaded before the factor
  // rows are formed (their latency overlaps those loads), then added in
  // split order
  const bool live = idx < M * C;
  const float* pp = part + (live ? idx : 0);
  const int64_t ps = M * C;
  const int n8 = min(nsplit, 8);
  float t[8];
#pragma unroll
  for (int u = 0; u < 8; ++u) t[u] = u < n8 ? pp[u * ps] : 0.f;
  for (int64_t m = m_first; m <= m_last; ++m) {
    float* lrow = s_l + (m - m_first) * r;
    rank_row<F16>(rank, m, lrow, s_red);
    if (rank.out && m * C >= idx0 && threadIdx.x < r) rank.out[m * r + threadIdx.x] = lrow[threadIdx.x];
  }
  if (!live) return;
  float v = 0.f;
#pragma unroll
  for (int u = 0; u < 8; ++u)
    if (u < n8) v += t[u];
  for (int sp = 8; sp < nsplit; ++sp) v += pp[sp * ps];
  const int64_t m = idx / C, c = idx % C;
  const float* lrow = s_l + (m - m_first) * r;
  float acc = 0.f;
  for (int j = 0; j < r; ++j) acc += lrow[j] * w16<F16>(lora.R[c * lora.rs_c + j * lora.rs_j]);
  v += lora.scaling * acc;
  if (out16)
    gptr_w(reinterpret_cast<uint16_t*>(out))[idx] = to16<F16>(v);
  else
    gptr_w(reinterpret_cast<float*>(out))[idx] = v;
}

// rank.out = P Q^T, row blockIdx.x formed by rank_row as the reduce forms it.
template <bool F16>
__global__ __launch_bounds__(256) void k_rank_rows(RankRow rank) {
  __shared__ float s_l[64];
  __shared__ float s_red[32];
  const int64_t m = blockIdx.x;
  rank_row<F16>(rank, m, s_l, s_red);
  if (threadIdx.x < rank.r) rank.out[m * rank.r + threadIdx.x] = s_l[threadIdx.x];
}

hipError_t launch_reduce_rows(const float* part, int nsplit, int64_t M, int64_t C, const LoraTerm& lora,
                              void* out, bool out16, bool f16, hipStream_t s, const RankRow& rank) {
  const dim3 grid((unsigned)((M * C + 255) / 256));
  if (f16)
    hipLaunchKernelGGL(k_reduce_rows<true>, grid, dim3(256), 0, s, part, nsplit, M, C, lora, out,
                       (int)out16, rank);
  else
    hipLaunchKernelGGL(k_reduce_rows<false>, grid, dim3(256), 0, s, part, nsplit, M, C, lora, out,
                       (int)out16, rank);
  return hipGetLastError();
}

hipError_t launch_rank_rows(const RankRow& rank, int64_t M, bool f16, hipStream_t s) {
  if (f16)
    hipLaunchKernelGGL(k_rank_rows<true>, dim3((unsigned)M), dim3(256), 0, s, rank);
  else
    hipLaunchKernelGGL(k_rank_rows<false>, dim3((unsigned)M), dim3(256), 0, s, rank);
  return hipGetLastError();
}

}  // namespace ql
