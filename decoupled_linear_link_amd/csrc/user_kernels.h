// User side of the hot path on the matrix cores (bf16, d_h = 32): the
// LIME-XOR layer stack (LIME notes, "Key design 2": history -> links and
// links -> history cross attention, residual + gated MLP; LN before the
// projections per the training-strategy section).
//
// Row space: [B*ell link rows ; total_N history rows].  Intermediates use
//   QK [rows, 2d]      Q in columns [0, d), K in [d, 2d), row-major
//   Vp [rows/8][d][8]  V "row-octet packed": one column of 8 consecutive
//                      rows is contiguous, the operand layout of the
//                      contractions over rows (no transposes needed).
// The device functions below work on either global or LDS pointers; they
// are shared by the streaming kernels (any history length, one launch per
// step of a layer) and the user-resident kernel (one workgroup per user,
// all layers in one launch, for histories that fit in LDS).
#pragma once

#include <type_traits>

#include "mfma_kernels.h"

namespace lime {
namespace mfma {

__device__ __forceinline__ int64_t vp_index(int64_t row, int col, int D) {
  return (row >> 3) * static_cast<int64_t>(D) * 8 + static_cast<int64_t>(col) * 8 + (row & 7);
}

// Layout of a buffer of 32-column head slices: slice p of row `row` starts
// at element p * ps + row * rs.  For Q|K the slice index is part * H + h
// (part 0 = Q, 1 = K); for Y it is h.  Row-major rows: rs = row stride,
// ps = 32.  Head-planar (every slice of every row contiguous by rows, as the
// streaming kernels use in HBM): rs = 32, ps = rows * 32.
struct Lay {
  int64_t rs, ps;
};

// Pairwise (tree) sum of N values: a log-depth dependency chain instead of
// a serial one.
template <int N>
__device__ __forceinline__ float tree_sum(const float* v) {
  if constexpr (N == 1) {
    return v[0];
  } else {
    return tree_sum<N / 2>(v) + tree_sum<N - N / 2>(v + N / 2);
  }
}

// Sum over each group of N consecutive lanes (N a power of two up to 64).
template <int N>
__device__ __forceinline__ float span_sum(float x) {
#pragma unroll
  for (int o = 1; o < N; o <<= 1) x += __shfl_xor(x, o);
  return x;
}

// LayerNorm (no affine, eps 1e-5) of the row a lane group holds: v[] are
// this lane's values of the row; the other values are in lanes ^16, ^32.
template <int N>
__device__ __forceinline__ void ln_rows(float* v, int D) {
  float s = tree_sum<N>(v);
  s = rows_sum(s);
  const float mu = s / D;
  float t[N];
#pragma unroll
  for (int i = 0; i < N; ++i) {
    const float u = v[i] - mu;
    t[i] = u * u;
  }
  float q = tree_sum<N>(t);
  q = rows_sum(q);
  const float rs = rsqrtf(q / D + 1e-5f);
#pragma unroll
  for (int i = 0; i < N; ++i) v[i] = (v[i] - mu) * rs;
}

__device__ __forceinline__ bf16x8 pack8(const float* v) {
  bf16x8 o;
#pragma unroll
  for (int j = 0; j < 8; ++j) o[j] = static_cast<__bf16>(v[j]);
  return o;
}

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// The one-pass variance E[x^2] - E[x]^2 cancels float32 bits in proportion
// to mean^2 / variance.  While mean^2 <= 64 variance its error stays below
// about 3e-4 of the variance (E[x^2] <= 65 variance, summed in float32); a
// row past that bound is a row whose values sit far from zero relative to
// their spread.  If any row of the wave is past it, the whole wave (so that
// the cross-lane sums see only active lanes) recomputes the variance from
// centred values, which has no cancellation.
__device__ __forceinline__ bool wave_needs_centred_var(float mu, float var) {
  return __builtin_amdgcn_ballot_w64(mu * mu > 64.f * var) != 0;
}

// LayerNorm (no affine, eps 1e-5) of the bf16 row a lane group holds
// (x[kb]: this lane's values, the rest in lanes ^16, ^32), straight to bf16
// operands.  The statistics come from bf16 pair dot products (sum and sum
// of squares, one instruction per pair each, float32 accumulation), the
// variance as E[x^2] - E[x]^2, recomputed from centred values when the
// mean dwarfs the spread (wave_needs_centred_var).
template <int KB>
__device__ __forceinline__ void ln_bf16(const bf16x8 (&x)[KB], int D, bf16x8 (&out)[KB]) {
  const bf16x2 one = {static_cast<__bf16>(1.f), static_cast<__bf16>(1.f)};
  float s[2] = {0.f, 0.f}, q[2] = {0.f, 0.f};
#pragma unroll
  for (int kb = 0; kb < KB; ++kb)
#pragma unroll
    for (int pp = 0; pp < 4; ++pp) {
      const bf16x2 v = {x[kb][2 * pp], x[kb][2 * pp + 1]};
      s[pp & 1] = __builtin_amdgcn_fdot2_f32_bf16(v, one, s[pp & 1], false);
      q[pp & 1] = __builtin_amdgcn_fdot2_f32_bf16(v, v, q[pp & 1], false);
    }
  const float sum = rows_sum(s[0] + s[1]), sq = rows_sum(q[0] + q[1]);
  const float inv_d = 1.f / static_cast<float>(D);
  const float mu = sum * inv_d;
  float var = sq * inv_d - mu * mu;
  if (wave_needs_centred_var(mu, var)) {
    float c[2] = {0.f, 0.f};
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float u = static_cast<float>(x[kb][j]) - mu;
        c[j & 1] = fmaf(u, u, c[j & 1]);
      }
    var = rows_sum(c[0] + c[1]) * inv_d;
  }
  const float rs = rsqrtf(fmaxf(var, 0.f) + 1e-5f);
  const float nb = -mu * rs;
#pragma unroll
  for (int kb = 0; kb < KB; ++kb) {
    float v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = fmaf(static_cast<float>(x[kb][j]), rs, nb);
    out[kb] = pack8(v);
  }
}


// ---------------------------------------------------------------------------
// QKV projection of one 32-row chunk.  hb[rb][kb] are LN(X) operands: lane
// (r, g) of row block rb carries chunk row 8*(r/4) + 4*rb + r%4, columns
// kb*32 + 8g .. +8.  Q and K (transposed form) land as 16-byte row pieces;
// V (operands swapped) lands as one 16-byte column piece of 8 rows.
// QK and Vp are addressed with chunk-local row `row0` (multiple of 8).
// ---------------------------------------------------------------------------
template <int D>
__device__ __forceinline__ void qk_part(const bf16x8 (&hb)[2][D / 32], const bf16_t* __restrict__ W,
                                        int ldw, bf16_t* QK, int64_t row0, int r, int g, float qs,
                                        Lay L, bool with_q = true) {
  constexpr int KB = D / 32;
#pragma unroll 2
  for (int p = with_q ? 0 : D / 32; p < 2 * D / 32; ++p) {
    floatx4 acc[2][2] = {};
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const bf16_t* wr = W + static_cast<int64_t>(32 * p + 8 * (r >> 2) + 4 * c + (r & 3)) * ldw + 8 * g;
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        const bf16x8 a = ld16(wr + kb * 32);
        acc[c][0] = mma(a, hb[0][kb], acc[c][0]);
        acc[c][1] = mma(a, hb[1][kb], acc[c][1]);
      }
    }
    const float f = p < D / 32 ? qs : 1.f;  // Q columns carry the logit scale
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
      const int64_t row = row0 + 8 * (r >> 2) + 4 * rb + (r & 3);
      const float v[8] = {acc[0][rb][0] * f, acc[0][rb][1] * f, acc[0][rb][2] * f, acc[0][rb][3] * f,
                          acc[1][rb][0] * f, acc[1][rb][1] * f, acc[1][rb][2] * f, acc[1][rb][3] * f};
      st8h(QK + p * L.ps + row * L.rs + 8 * g, v);
    }
  }
}

template <int D>
__device__ __forceinline__ void v_part(const bf16x8 (&hb)[2][D / 32], const bf16_t* __restrict__ W,
                                       int ldw, bf16_t* Vp, int64_t row0, int r, int g) {
  constexpr int KB = D / 32;
#pragma unroll 2
  for (int n = 0; n < D / 16; ++n) {
    const bf16_t* wr = W + static_cast<int64_t>(2 * D + 16 * n + r) * ldw + 8 * g;
    floatx4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      const bf16x8 b = ld16(wr + kb * 32);
      acc0 = mma(hb[0][kb], b, acc0);
      acc1 = mma(hb[1][kb], b, acc1);
    }
    const float v[8] = {acc0[0], acc0[1], acc0[2], acc0[3], acc1[0], acc1[1], acc1[2], acc1[3]};
    st8h(Vp + vp_index(row0 + 8 * g, 16 * n + r, D), v);
  }
}

template <int D>
__device__ __forceinline__ void qkv_chunk(const bf16x8 (&hb)[2][D / 32], const bf16_t* __restrict__ W,
                                          int ldw, bf16_t* QK, bf16_t* Vp, int64_t row0, int r, int g, float qs,
                                          Lay L, bool with_q = true) {
  qk_part<D>(hb, W, ldw, QK, row0, r, g, qs, L, with_q);
  v_part<D>(hb, W, ldw, Vp, row0, r, g);
}

// LN + QKV of RB 16-row blocks: lane (r, g) of block rb holds row
// row0 + 16 rb + r, columns 32 kb + 8 g .. +8 (the post block's layout) in
// x[rb].  Q|K land as 16-byte row pieces; V (operands swapped) as 8-byte
// pieces of 4 rows of one column in the packed layout (row0 a multiple of 8).
template <int D, int RB>
__device__ __forceinline__ void qkv_rows(const float (&x)[RB][D / 4], const bf16_t* __restrict__ W, int ldw,
                                         bf16_t* QK, bf16_t* Vp, int64_t row0, int r, int g, Lay L, float qs,
                                         bool with_q = true) {
  constexpr int KB = D / 32;
  bf16x8 hb[RB][KB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    float v[8 * KB];
#pragma unroll
    for (int i = 0; i < 8 * KB; ++i) v[i] = x[rb][i];
    ln_rows<8 * KB>(v, D);
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) hb[rb][kb] = pack8(v + 8 * kb);
  }
#pragma unroll 2
  for (int p = with_q ? 0 : D / 32; p < 2 * D / 32; ++p) {
    floatx4 acc[2][RB] = {};
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const bf16_t* wr = W + static_cast<int64_t>(32 * p + 8 * (r >> 2) + 4 * c + (r & 3)) * ldw + 8 * g;
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        const bf16x8 a = ld16(wr + kb * 32);
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) acc[c][rb] = mma(a, hb[rb][kb], acc[c][rb]);
      }
    }
    const float f = p < D / 32 ? qs : 1.f;  // Q columns carry the logit scale
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      const float o[8] = {acc[0][rb][0] * f, acc[0][rb][1] * f, acc[0][rb][2] * f, acc[0][rb][3] * f,
                          acc[1][rb][0] * f, acc[1][rb][1] * f, acc[1][rb][2] * f, acc[1][rb][3] * f};
      st8h(QK + p * L.ps + (row0 + 16 * rb + r) * L.rs + 8 * g, o);
    }
  }
#pragma unroll 2
  for (int nn = 0; nn < D / 16; ++nn) {
    const bf16_t* wr = W + static_cast<int64_t>(2 * D + 16 * nn + r) * ldw + 8 * g;
    floatx4 acc[RB] = {};
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      const bf16x8 b = ld16(wr + kb * 32);
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) acc[rb] = mma(hb[rb][kb], b, acc[rb]);
    }
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) st4h(Vp + vp_index(row0 + 16 * rb + 4 * g, 16 * nn + r, D), acc[rb]);
  }
}

// ---------------------------------------------------------------------------
// XOR attention pieces for one (user, head h).  Link rows start at `lrow`,
// history row j is row `hrow + j` of QK / Vp / Y.
// Link order of the score blocks: M-block c, row 4*g + q -> link
// (c/2)*32 + 8*g + 4*(c%2) + q, so each lane's 8 links per 32 are the K
// slice of the P^T operand of the value product.
// ---------------------------------------------------------------------------
template <int ELL>
struct HeadOps {
  static constexpr int MB = ELL / 16, KBL = ELL / 32;
  f16x8 kl[MB];       // A: K_L, rows = links (ordered as above), k = d_h
  f16x8 qlt[MB];      // B: Q_L^T, cols = links 16*c + r, k = d_h
  f16x8 vlt[2][KBL];  // A: V_L^T, rows = 8*(r/4) + 4*c2 + r%4, k = links
};

template <int ELL, int D>
__device__ __forceinline__ void load_head_ops(HeadOps<ELL>& o, const bf16_t* QK, const bf16_t* Vp,
                                              int64_t lrow, int h, int r, int g, Lay L) {
  constexpr int H = D / 32;
#pragma unroll
  for (int c = 0; c < HeadOps<ELL>::MB; ++c) {
    const int link = (c >> 1) * 32 + 8 * (r >> 2) + 4 * (c & 1) + (r & 3);
    o.kl[c] = ldh16(QK + (H + h) * L.ps + (lrow + link) * L.rs + 8 * g);
    o.qlt[c] = ldh16(QK + h * L.ps + (lrow + 16 * c + r) * L.rs + 8 * g);
  }
#pragma unroll
  for (int c2 = 0; c2 < 2; ++c2)
#pragma unroll
    for (int kb = 0; kb < HeadOps<ELL>::KBL; ++kb)
      o.vlt[c2][kb] = ldh16(Vp + vp_index(lrow + kb * 32 + 8 * g, h * 32 + 8 * (r >> 2) + 4 * c2 + (r & 3), D));
}

// Operands of one 32-row chunk of history rows c0 + [0, 32) for head h:
// Q rows (E-branch B operands), K rows in the L-branch row order (A
// operands) and two packed V column blocks (A operands of V^T P^T).
struct ChunkOps {
  f16x8 qe[2], ke[2], ve[2];
};

template <int D>
__device__ __forceinline__ void load_chunk(ChunkOps& c, const bf16_t* QK, const bf16_t* Vp, int64_t hrow,
                                           int64_t c0, int h, bool with_q, int r, int g, Lay L) {
  constexpr int H = D / 32;
  if (with_q) {
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) c.qe[rb] = ldh16(QK + h * L.ps + (hrow + c0 + 16 * rb + r) * L.rs + 8 * g);
  }
#pragma unroll
  for (int k = 0; k < 2; ++k)
    c.ke[k] = ldh16(QK + (H + h) * L.ps + (hrow + c0 + 8 * (r >> 2) + 4 * k + (r & 3)) * L.rs + 8 * g);
  c.ve[0] = ldh16(Vp + vp_index(hrow + c0 + 8 * g, h * 32 + r, D));
  c.ve[1] = ldh16(Vp + vp_index(hrow + c0 + 8 * g, h * 32 + 16 + r, D));
}

// LIME-XOR+Window (LIME notes, "Key design 3"): history row j also attends
// the rows q of its user with 1 <= |q - j| <= half.  For a 32-row chunk at
// c0 the keys of both 16-row blocks lie in [c0 - ceil8(half), +NKW) when
// NKW >= 32 + 2 ceil8(half); NKW = 64 serves half <= 16 (ell = 32) and
// NKW = 96 serves half <= 32 (ell = 64).
struct WinArgs {
  int64_t u0 = 0, u1 = 0;        // the user's history rows (history index space)
  int64_t rmax = 0;              // rows of the QK / packed-V buffers (multiple of 8)
  int half = 0;                  // neighbours on each side
  const bf16_t* Vp = nullptr;    // packed V, read for the value product
  int64_t hrow = 0;              // buffer row of history row 0
};

template <int NKW>
struct WinOps {
  static constexpr int MBW = NKW / 16, KBW = NKW / 32;
  f16x8 kw[MBW];      // A: window keys, rows in the link-block order
};
template <>
struct WinOps<0> {};

constexpr int win_nkw(int ell) { return ell == 32 ? 64 : 96; }

__device__ __forceinline__ int64_t win_key0(int64_t c0, int half) { return c0 - ((half + 7) & ~7); }

// Window operands of the chunk at c0 (history index) for head h.  Buffer
// rows outside [0, rmax) are clamped: such keys are always masked, and
// every buffer row holds finite values.
template <int NKW, int D>
__device__ __forceinline__ void load_window(WinOps<NKW>& w, const bf16_t* QK, const bf16_t* Vp, int64_t hrow,
                                            int64_t key0, int64_t rmax, int h, int r, int g, Lay L) {
  constexpr int H = D / 32;
#pragma unroll
  for (int c = 0; c < WinOps<NKW>::MBW; ++c) {
    const int t = (c >> 1) * 32 + 8 * (r >> 2) + 4 * (c & 1) + (r & 3);
    const int64_t row = clamp64(hrow + key0 + t, 0, rmax - 1);
    w.kw[c] = ldh16(QK + (H + h) * L.ps + row * L.rs + 8 * g);
  }
  (void)Vp;
}

// A operand of the window's value product for 32 keys kb (V transposed):
// loaded where it is used, so it is not live through the scores.
template <int D>
__device__ __forceinline__ f16x8 window_v(const WinArgs& wa, int64_t key0, int kb, int c2, int h, int r, int g) {
  const int64_t row = clamp64(wa.hrow + key0 + 32 * kb + 8 * g, 0, wa.rmax - 8);
  return ldh16(wa.Vp + vp_index(row, h * 32 + 8 * (r >> 2) + 4 * c2 + (r & 3), D));
}

// phi in log2 units (exp2_f, silu2 and silu2_div are defined with the
// cache kernels): the projections store Q multiplied by scale*log2(e), so a
// score y is the logit x in log2 units.

// E-branch: history rows c0 + [0, 32) attend to the ell links (and, with
// NKW > 0, to their window); rows in [lo, hi) are written to Y.  Row order
// of the Q operands: qe[rb] lane r holds chunk row 16*rb + r, or with RHO
// the projection's order 8*(r/4) + 4*rb + r%4.
template <int ELL, int D, bool SM, int NKW = 0, bool RHO = false>
__device__ __forceinline__ void e_branch(const HeadOps<ELL>& o, const ChunkOps& ci, bf16_t* Y,
                                         int64_t hrow, int64_t c0, int64_t lo, int64_t hi, int h,
                                         int r, int g, Lay yl,
                                         const WinOps<NKW>* wo = nullptr, const WinArgs* wa = nullptr) {
  constexpr int MB = HeadOps<ELL>::MB, KBL = HeadOps<ELL>::KBL;
  constexpr int NWS = NKW > 0 ? NKW / 4 : 1;  // window scores per lane
#pragma unroll
  for (int rb = 0; rb < 2; ++rb) {
    const int64_t j = c0 + (RHO ? 8 * (r >> 2) + 4 * rb + (r & 3) : 16 * rb + r);
    float v[4 * MB];
#pragma unroll
    for (int c = 0; c < MB; ++c) {
      const floatx4 st = mma(o.kl[c], ci.qe[rb], floatx4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
      for (int q = 0; q < 4; ++q) v[4 * c + q] = st[q];
    }
    float ws[NWS];
    int nwin = 0;  // this row's window size (its own row excluded)
    if constexpr (NKW > 0) {
      const int64_t key0 = win_key0(c0, wa->half);
#pragma unroll
      for (int c = 0; c < NKW / 16; ++c) {
        const floatx4 sw = mma(wo->kw[c], ci.qe[rb], floatx4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int64_t kq = key0 + (c >> 1) * 32 + 8 * g + 4 * (c & 1) + q;
          const int64_t dist = kq > j ? kq - j : j - kq;
          const bool ok = kq >= wa->u0 && kq < wa->u1 && dist >= 1 && dist <= wa->half;
          ws[4 * c + q] = ok ? sw[q] : -INFINITY;
        }
      }
      const int64_t a = j - wa->half > wa->u0 ? j - wa->half : wa->u0;
      const int64_t e = j + wa->half < wa->u1 - 1 ? j + wa->half : wa->u1 - 1;
      nwin = e > a ? static_cast<int>(e - a) : 0;
    }
    if constexpr (SM) {
      float mx = v[0];
#pragma unroll
      for (int q = 1; q < 4 * MB; ++q) mx = fmaxf(mx, v[q]);
      if constexpr (NKW > 0) {
#pragma unroll
        for (int q = 0; q < NWS; ++q) mx = fmaxf(mx, ws[q]);
      }
      mx = rows_max(mx);
      float sum = 0.f;
#pragma unroll
      for (int q = 0; q < 4 * MB; ++q) {
        v[q] = exp2_f(v[q] - mx);
        sum += v[q];
      }
      if constexpr (NKW > 0) {
#pragma unroll
        for (int q = 0; q < NWS; ++q) {
          ws[q] = exp2_f(ws[q] - mx);  // 0 for masked keys
          sum += ws[q];
        }
      }
      sum = rows_sum(sum);
      const float inv = __builtin_amdgcn_rcpf(sum);  // sum >= 1 (the max term)
#pragma unroll
      for (int q = 0; q < 4 * MB; ++q) v[q] *= inv;
      if constexpr (NKW > 0) {
#pragma unroll
        for (int q = 0; q < NWS; ++q) ws[q] *= inv;
      }
    } else {
      // silu2 * ln 2 / |keys|
      const float c = NKW > 0 ? static_cast<float>(ELL + nwin) * LOG2E : ELL * LOG2E;
#pragma unroll
      for (int q = 0; q < 4 * MB; ++q) v[q] = silu2_div(v[q], c);
      if constexpr (NKW > 0) {
#pragma unroll
        for (int q = 0; q < NWS; ++q) ws[q] = ws[q] == -INFINITY ? 0.f : silu2_div(ws[q], c);
      }
    }
    floatx4 y0 = {0.f, 0.f, 0.f, 0.f}, y1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kb = 0; kb < KBL; ++kb) {
      const f16x8 pb = packh8(v + 8 * kb);
      y0 = mma(o.vlt[0][kb], pb, y0);
      y1 = mma(o.vlt[1][kb], pb, y1);
    }
    if constexpr (NKW > 0) {
      const int64_t key0 = win_key0(c0, wa->half);
#pragma unroll
      for (int kb = 0; kb < NKW / 32; ++kb) {
        const f16x8 pb = packh8(ws + 8 * kb);
        y0 = mma(window_v<D>(*wa, key0, kb, 0, h, r, g), pb, y0);
        y1 = mma(window_v<D>(*wa, key0, kb, 1, h, r, g), pb, y1);
      }
    }
    if (j >= lo && j < hi) {
      const float out[8] = {y0[0], y0[1], y0[2], y0[3], y1[0], y1[1], y1[2], y1[3]};
      st8(Y + h * yl.ps + (hrow + j) * yl.rs + 8 * g, out);
    }
  }
}

// L-branch running state: per link block nb, running max m / denominator l
// and acc, all for the link 16*nb + r of this lane (acc: columns
// 16*c2 + 4*g + q), so the rescaling of acc by the new max stays in the lane.
template <int ELL>
struct LState {
  static constexpr int MB = ELL / 16;
  float m[MB], l[MB];
  floatx4 acc[MB][2];
  __device__ __forceinline__ void init() {
#pragma unroll
    for (int c = 0; c < MB; ++c) {
      m[c] = -INFINITY;
      l[c] = 0.f;
      acc[c][0] = floatx4{0.f, 0.f, 0.f, 0.f};
      acc[c][1] = floatx4{0.f, 0.f, 0.f, 0.f};
    }
  }
};

// L-branch: the links attend to history rows c0 + [0, 32) (those in
// [lo, hi)); c0 + hrow must be a multiple of 8.  Scores are in log2 units;
// with silu the accumulators hold sum silu2 * v (the ln 2 factor is applied
// where they are normalised).  MASK = false: every row of the chunk is in
// [lo, hi).
template <int ELL, bool MASK, bool SM>
__device__ __forceinline__ void l_branch_rows(LState<ELL>& st, const HeadOps<ELL>& o, const ChunkOps& ci,
                                              int64_t c0, int64_t lo, int64_t hi, int r, int g) {
  constexpr int MB = HeadOps<ELL>::MB;
  bool valid[8];
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    const int64_t j = c0 + 8 * g + q;  // q = 4*c + jj
    valid[q] = !MASK || ((j >= lo) && (j < hi));
  }
  // V of rows outside [lo, hi) (another user's, or past the history end) is
  // zeroed, not only their weights: a non-finite value there must not reach
  // this split through 0 * inf
  f16x8 ve[2] = {ci.ve[0], ci.ve[1]};
  if constexpr (MASK) {
#pragma unroll
    for (int q = 0; q < 8; ++q)
      if (!valid[q]) {
        ve[0][q] = static_cast<_Float16>(0.f);
        ve[1][q] = static_cast<_Float16>(0.f);
      }
  }
#pragma unroll
  for (int nb = 0; nb < MB; ++nb) {
    float p[8];
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const floatx4 sv = mma(ci.ke[c], o.qlt[nb], floatx4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
      for (int q = 0; q < 4; ++q) p[4 * c + q] = sv[q];
    }
    if constexpr (SM) {
      float mc = -INFINITY;
#pragma unroll
      for (int q = 0; q < 8; ++q)
        if (valid[q]) mc = fmaxf(mc, p[q]);
      mc = rows_max(mc);
      const float mn = fmaxf(st.m[nb], mc);
      const float alpha = (st.m[nb] == -INFINITY) ? 0.f : exp2_f(st.m[nb] - mn);
      float ls = 0.f;
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        p[q] = valid[q] ? exp2_f(p[q] - mn) : 0.f;
        ls += p[q];
      }
      ls = rows_sum(ls);
      st.l[nb] = st.l[nb] * alpha + ls;
      st.m[nb] = mn;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        st.acc[nb][0][q] *= alpha;
        st.acc[nb][1][q] *= alpha;
      }
    } else {
#pragma unroll
      for (int q = 0; q < 8; ++q) p[q] = valid[q] ? silu2(p[q]) : 0.f;
    }
    // (V^T P^T): P's lane layout (link r, rows 8g..8g+7) is the B operand as
    // it stands, and the product's columns are the links
    const f16x8 pb = packh8(p);
    st.acc[nb][0] = mma(ve[0], pb, st.acc[nb][0]);
    st.acc[nb][1] = mma(ve[1], pb, st.acc[nb][1]);
  }
}

template <int ELL, bool SM>
__device__ __forceinline__ void l_branch(LState<ELL>& st, const HeadOps<ELL>& o, const ChunkOps& ci,
                                         int64_t c0, int64_t lo, int64_t hi, int r, int g) {
  if (c0 >= lo && c0 + 32 <= hi)
    l_branch_rows<ELL, false, SM>(st, o, ci, c0, lo, hi, r, g);
  else
    l_branch_rows<ELL, true, SM>(st, o, ci, c0, lo, hi, r, g);
}

// Runs f(std::true_type) for softmax and f(std::false_type) otherwise, so
// each phi gets straight-line code.
template <typename F>
__device__ __forceinline__ void with_phi(bool softmax, F&& f) {
  if (softmax)
    f(std::true_type{});
  else
    f(std::false_type{});
}

// The same for any runtime flag.
template <typename F>
__device__ __forceinline__ void with_flag(bool b, F&& f) {
  with_phi(b, static_cast<F&&>(f));
}

// ---------------------------------------------------------------------------
// Post-attention block on RB row blocks of 16 rows (lane (r, g) of block rb
// carries one row, columns 32*p + 8*g .. +8 of every 32-column block):
//   x1 += Y Wo^T ;  G = LN(x1) ;  M = SiLU(G Wg^T) * (G Wu^T) ;  x1 += M Wd^T
// x1 holds the residual on entry and the layer output on exit (float32);
// with xres the residual comes as bf16 from xres instead and is first read
// in the W_o epilogue (so its loads can still be in flight through W_o).
// Each product's output is the next product's B operand as it stands.
// ---------------------------------------------------------------------------
template <int D, int DFF, int RB, bool XB = false, bool SB = true>
__device__ __forceinline__ void post_rows(const bf16x8 (&yb)[RB][D / 32], float (&x1)[RB][D / 4],
                                          const bf16_t* __restrict__ Wo, const bf16_t* __restrict__ Wg,
                                          const bf16_t* __restrict__ Wu, const bf16_t* __restrict__ Wd,
                                          int ldd, int ldf, int r, int g,
                                          const bf16x8 (*xres)[D / 32] = nullptr) {
  constexpr int KB = D / 32, KF = DFF / 32;
#pragma unroll
  for (int p = 0; p < KB; ++p) {
    floatx4 acc[2][RB] = {};
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const bf16_t* wr = Wo + static_cast<int64_t>(32 * p + 8 * (r >> 2) + 4 * c + (r & 3)) * ldd + 8 * g;
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        const bf16x8 a = ld16(wr + kb * 32);
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) acc[c][rb] = mma(a, yb[rb][kb], acc[c][rb]);
      }
    }
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float r0 = XB ? static_cast<float>(xres[rb][p][q]) : x1[rb][8 * p + q];
        const float r1 = XB ? static_cast<float>(xres[rb][p][4 + q]) : x1[rb][8 * p + 4 + q];
        x1[rb][8 * p + q] = r0 + acc[0][rb][q];
        x1[rb][8 * p + 4 + q] = r1 + acc[1][rb][q];
      }
    // keep the scheduler from hoisting every block's weight loads at once
    if constexpr (SB) __builtin_amdgcn_sched_barrier(0);
  }
  bf16x8 gb[RB][KB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    float t[8 * KB];
#pragma unroll
    for (int i = 0; i < 8 * KB; ++i) t[i] = x1[rb][i];
    ln_rows<8 * KB>(t, D);
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) gb[rb][kb] = pack8(t + 8 * kb);
  }
  bf16x8 mb[RB][KF];
#pragma unroll
  for (int q2 = 0; q2 < KF; ++q2) {
    floatx4 ag[2][RB] = {}, au[2][RB] = {};
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const int64_t orow = 32 * q2 + 8 * (r >> 2) + 4 * c + (r & 3);
      const bf16_t* gr = Wg + orow * ldd + 8 * g;
      const bf16_t* ur = Wu + orow * ldd + 8 * g;
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        const bf16x8 a1 = ld16(gr + kb * 32);
        const bf16x8 a2 = ld16(ur + kb * 32);
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
          ag[c][rb] = mma(a1, gb[rb][kb], ag[c][rb]);
          au[c][rb] = mma(a2, gb[rb][kb], au[c][rb]);
        }
      }
    }
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      float v[8];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        v[q] = silu_f(ag[0][rb][q]) * au[0][rb][q];
        v[4 + q] = silu_f(ag[1][rb][q]) * au[1][rb][q];
      }
      mb[rb][q2] = pack8(v);
    }
    if constexpr (SB) __builtin_amdgcn_sched_barrier(0);
  }
#pragma unroll
  for (int p = 0; p < KB; ++p) {
    floatx4 acc[2][RB] = {};
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const bf16_t* wr = Wd + static_cast<int64_t>(32 * p + 8 * (r >> 2) + 4 * c + (r & 3)) * ldf + 8 * g;
#pragma unroll
      for (int kf = 0; kf < KF; ++kf) {
        const bf16x8 a = ld16(wr + kf * 32);
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) acc[c][rb] = mma(a, mb[rb][kf], acc[c][rb]);
      }
    }
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        x1[rb][8 * p + q] += acc[0][rb][q];
        x1[rb][8 * p + 4 + q] += acc[1][rb][q];
      }
    // keep the scheduler from hoisting every block's weight loads at once
    if constexpr (SB) __builtin_amdgcn_sched_barrier(0);
  }
}

// ===========================================================================
// Streaming kernels (any history length)
// ===========================================================================

// Splits of the streaming attention.  User b's history rows [u0, u1) are
// cut at a grid of chunk rows anchored at the 8-aligned row below u0
// (a = u0 & ~7): split s is [max(u0, a + s chunk), min(u1, a + (s+1) chunk)),
// S_b = max(1, ceil((u1 - a) / chunk)) of them.  Every split but the tails
// then carries the same work however ragged the histories are, and, since
// the attention walks 32-row chunks from the 8-aligned row at or below a
// split's start, a chunk that is a multiple of 32 takes chunk / 32 steps for
// every split (cut at u0 itself, a misaligned user would take one more).
// split_off[b] = sum of S_b' over b' < b (split_off[B] = the number of
// splits) and split_user[x] = the user of split x, -1 for x >= split_off[B]
// up to G.  One workgroup of 1024 threads.
constexpr int SPLIT_PLAN_NT = 1024;
constexpr int PART_LD = 36;  // floats per partial row: m, l, 2 spare, acc[32]

__device__ __forceinline__ int64_t split_count(int64_t u0, int64_t u1, int64_t chunk) {
  const int64_t sb = (u1 - (u0 & ~int64_t(7)) + chunk - 1) / chunk;
  return sb > 1 ? sb : 1;
}

// rows [lo, hi) of split s of the user owning [u0, u1)
__device__ __forceinline__ void split_rows(int64_t u0, int64_t u1, int64_t s, int64_t chunk, int64_t* lo,
                                           int64_t* hi) {
  const int64_t a = u0 & ~int64_t(7);
  *lo = clamp64(a + s * chunk, u0, u1);
  *hi = clamp64(a + (s + 1) * chunk, *lo, u1);
}

__global__ __launch_bounds__(SPLIT_PLAN_NT) void split_plan(const int64_t* __restrict__ off, int B,
                                                            int64_t total_N, int64_t chunk,
                                                            int32_t* __restrict__ split_off,
                                                            int32_t* __restrict__ split_user, int G) {
  __shared__ int32_t wsum[SPLIT_PLAN_NT / 64];
  __shared__ int32_t carry_s;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  if (tid == 0) {
    carry_s = 0;
    split_off[0] = 0;
  }
  __syncthreads();
  for (int base = 0; base < B; base += SPLIT_PLAN_NT) {
    const int b = base + tid;
    int32_t cnt = 0;
    if (b < B) {
      const int64_t u0 = clamp64(off[b], 0, total_N);
      const int64_t u1 = clamp64(off[b + 1], u0, total_N);
      cnt = static_cast<int32_t>(split_count(u0, u1, chunk));
    }
    // inclusive scan: within the wave, then over the waves
    int32_t v = cnt;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int32_t t = __shfl_up(v, o);
      if (lane >= o) v += t;
    }
    if (lane == 63) wsum[wv] = v;
    __syncthreads();
    int32_t before = carry_s;
    for (int w = 0; w < wv; ++w) before += wsum[w];
    // capped at G, which bounds the splits of non-decreasing offsets; with
    // offsets out of order the users past the cap get no splits
    const int32_t first = before + v - cnt < G ? before + v - cnt : G;
    const int32_t last = before + v < G ? before + v : G;
    if (b < B) {
      split_off[b + 1] = last;
      for (int32_t x = first; x < last; ++x) split_user[x] = b;
    }
    __syncthreads();
    if (tid == SPLIT_PLAN_NT - 1) carry_s = last;
    __syncthreads();
  }
  for (int x = carry_s + tid; x < G; x += SPLIT_PLAN_NT) split_user[x] = -1;
}

// XOR attention: one workgroup per (split x, head group) with one wave per
// head, so the waves of a workgroup read the same rows at the same time and
// share each cache line (HB heads per workgroup: all of them, or at most 4
// for the windowed form, whose registers need the room).  Writes the
// E-branch rows of Y and the L-branch partial rows [ell][PART_LD] (max,
// denominator, 2 spare, acc) of (split x, head h).
template <int ELL, int H, int NKW = 0, int HB = H>
__global__ __launch_bounds__(64 * HB) void xor_attn(const bf16_t* __restrict__ QK,
                                                    const bf16_t* __restrict__ Vp,
                                                    bf16_t* __restrict__ Y, float* __restrict__ part,
                                                    const int64_t* __restrict__ off,
                                                    const int32_t* __restrict__ split_off,
                                                    const int32_t* __restrict__ split_user, int B,
                                                    int64_t chunk, int64_t total_N,
                                                    int phi, int do_e, int half, int64_t rmax) {
  static_assert(H % HB == 0, "head groups");
  constexpr int D = 32 * H, MB = ELL / 16;
  const int lane = threadIdx.x & 63;
  const int g = lane >> 4, r = lane & 15;
  const int64_t x = blockIdx.x / (H / HB);  // split
  const int h = static_cast<int>(blockIdx.x % (H / HB)) * HB + (threadIdx.x >> 6);
  const int b = split_user[x];
  if (b < 0) return;  // past the last split
  const int64_t s = x - split_off[b];
  const int64_t nlr = static_cast<int64_t>(B) * ELL;
  const int64_t u0 = clamp64(off[b], 0, total_N);
  const int64_t u1 = clamp64(off[b + 1], u0, total_N);
  int64_t lo, hi;
  split_rows(u0, u1, s, chunk, &lo, &hi);
  const bool softmax = (phi == PHI_SOFTMAX);

  HeadOps<ELL> o;
  // Q|K and Y are head-planar in HBM: a wave's 16-row slice of one head is
  // one contiguous 1 KB piece
  const Lay qkl{32, rmax * 32}, yl{32, (nlr + total_N) * 32};
  load_head_ops<ELL, D>(o, QK, Vp, static_cast<int64_t>(b) * ELL, h, r, g, qkl);
  LState<ELL> st;
  st.init();
  // phi and the E-branch switch as compile-time flags: straight-line chunk
  // loops with no conditional loads
  with_phi(softmax, [&](auto phi_tag) {
    with_flag(do_e != 0, [&](auto e_tag) {
      constexpr bool SM = decltype(phi_tag)::value, DO_E = decltype(e_tag)::value;
      int64_t c0 = lo & ~int64_t(7);
      if (c0 >= hi) return;
      // chunk loads past the last chunk re-read the last one (never used),
      // so every step issues the same loads and the waits on them are exact
      const int64_t clast = c0 + ((hi - 1 - c0) >> 5) * 32;
      auto ld = [&](ChunkOps& c, int64_t at) {
        load_chunk<D>(c, QK, Vp, nlr, at < clast ? at : clast, h, DO_E, r, g, qkl);
      };
      ChunkOps cur;
      ld(cur, c0);
      if constexpr (NKW == 0) {
        // the next chunk's operands load while a chunk is computed; pairs
        // of steps swap the two buffers by name, and the loop has a single
        // exit, so the waits on the loads stay exact
        const int nch = static_cast<int>((clast - c0) >> 5) + 1;
        ChunkOps nxt;
        auto step = [&](const ChunkOps& ci, ChunkOps& ahead) {
          ld(ahead, c0 + 32);
          if constexpr (DO_E) e_branch<ELL, D, SM>(o, ci, Y, nlr, c0, lo, hi, h, r, g, yl);
          l_branch<ELL, SM>(st, o, ci, c0, lo, hi, r, g);
          c0 += 32;
        };
        for (int k = 2; k <= nch; k += 2) {
          step(cur, nxt);
          step(nxt, cur);
        }
        if (nch & 1) step(cur, nxt);
      } else {
        // the windowed form's own operands take the registers: one chunk at
        // a time
        for (; c0 < hi; c0 += 32) {
          if constexpr (DO_E) {
            WinOps<NKW> wo;
            load_window<NKW, D>(wo, QK, Vp, nlr, win_key0(c0, half), rmax, h, r, g, qkl);
            const WinArgs wa{u0, u1, rmax, half, Vp, nlr};
            e_branch<ELL, D, SM, NKW>(o, cur, Y, nlr, c0, lo, hi, h, r, g, yl, &wo, &wa);
          }
          l_branch<ELL, SM>(st, o, cur, c0, lo, hi, r, g);
          if (c0 + 32 < hi) ld(cur, c0 + 32);
        }
      }
    });
  });
  float* p0 = part + ((x * H + h) * ELL) * PART_LD;
#pragma unroll
  for (int nb = 0; nb < MB; ++nb) {
    // partials in natural units: max * ln 2; silu sums * ln 2
    float* pl = p0 + (16 * nb + r) * PART_LD;
    if (g == 0) {
      pl[0] = softmax ? st.m[nb] * LN2 : 0.f;
      pl[1] = softmax ? st.l[nb] : static_cast<float>(hi - lo);
    }
    const float f = softmax ? 1.f : LN2;
#pragma unroll
    for (int c2 = 0; c2 < 2; ++c2)
      *reinterpret_cast<floatx4*>(pl + 4 + 16 * c2 + 4 * g) =
          floatx4{st.acc[nb][c2][0] * f, st.acc[nb][c2][1] * f, st.acc[nb][c2][2] * f, st.acc[nb][c2][3] * f};
  }
}

// Merge of the split partials into the link rows of Y (head-planar, row
// stride 32, head stride yps).  CSG consecutive threads share one output
// octet (b, h, link k, columns 8 cq ..): thread t folds the splits
// x0 + t, x0 + t + CSG, ... of user b (four per round, with a running max),
// then the group merges its CSG partial states by lane exchanges.
constexpr int CSG = 8;

template <int ELL>
__global__ __launch_bounds__(256) void xor_combine(const float* __restrict__ part,
                                                   const int32_t* __restrict__ split_off,
                                                   bf16_t* __restrict__ Y, int B, int H, int64_t yps) {
  const int64_t gid = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  const int t = static_cast<int>(gid % CSG);
  const int64_t oi = gid / CSG;
  // a group's CSG lanes leave together (the block size is a multiple of CSG)
  if (oi >= static_cast<int64_t>(B) * H * ELL * 4) return;
  const int cq = static_cast<int>(oi & 3);
  const int k = static_cast<int>((oi >> 2) % ELL);
  const int h = static_cast<int>((oi / (4 * ELL)) % H);
  const int b = static_cast<int>(oi / (4 * ELL * static_cast<int64_t>(H)));
  const int32_t x0 = split_off[b], x1 = split_off[b + 1];
  const int64_t xs = static_cast<int64_t>(H) * ELL * PART_LD;  // split stride
  const float* p = part + (static_cast<int64_t>(h) * ELL + k) * PART_LD;
  float M = -INFINITY, den = 0.f;
  float num[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  auto fold = [&](float m2, float d2, const float* n2) {
    const float mn = fmaxf(M, m2);
    const float f1 = M == -INFINITY ? 0.f : __expf(M - mn);
    const float f2 = m2 == -INFINITY ? 0.f : __expf(m2 - mn);
    M = mn;
    den = den * f1 + d2 * f2;
#pragma unroll
    for (int q = 0; q < 8; ++q) num[q] = num[q] * f1 + n2[q] * f2;
  };
  for (int32_t xb = x0 + t; xb < x1; xb += 4 * CSG) {
    float2 ml[4];
    float a[4][8];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int32_t x = xb + u * CSG;
      const int64_t xx = x < x1 ? x : x1 - 1;  // repeats are masked below
      const float* pu = p + xx * xs;
      ml[u] = *reinterpret_cast<const float2*>(pu);
      const floatx4 a0 = *reinterpret_cast<const floatx4*>(pu + 4 + 8 * cq);
      const floatx4 a1 = *reinterpret_cast<const floatx4*>(pu + 8 + 8 * cq);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        a[u][q] = a0[q];
        a[u][4 + q] = a1[q];
      }
    }
#pragma unroll
    for (int u = 0; u < 4; ++u)
      if (xb + u * CSG < x1) fold(ml[u].x, ml[u].y, a[u]);
  }
#pragma unroll
  for (int o = 1; o < CSG; o <<= 1) {
    float n2[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) n2[q] = __shfl_xor(num[q], o);
    const float m2 = __shfl_xor(M, o), d2 = __shfl_xor(den, o);
    fold(m2, d2, n2);
  }
  if (t == 0) {
    const float inv = den > 0.f ? 1.f / den : 0.f;
    float o[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) o[q] = num[q] * inv;
    st8(Y + h * yps + (static_cast<int64_t>(b) * ELL + k) * 32 + 8 * cq, o);
  }
}

// ---------------------------------------------------------------------------
// Persistent variants with the weights staged once per workgroup in LDS
// (rows padded by 16 bytes).  NW waves per workgroup; each wave walks
// 32-row blocks strided by the whole grid.
// ---------------------------------------------------------------------------
// Copies rows x K bf16 from global memory into LDS rows padded by PAD
// elements (16 or 32 bytes; see wqkv_slot for what each costs in bank
// conflicts).
// SU loads per thread are issued before their LDS stores (indexes past the
// end re-read the last chunk and are not stored), so a thread waits on one
// round trip per batch rather than one per chunk.
constexpr int SU = 8;

// Where row `row` sits when staged for the projection helpers below (w_qkv
// rows, and the fused kernels' LN chunk rows): inside each 32-row block,
// bit 2 of the row index is flipped when bit 4 is set.  A fragment read
// (ds_read_b128: 16 rows, 4 adjacent 16-byte columns per row) touches 16
// consecutive rows, or rows {0-3, 8-11, 16-19, 24-27} (or those plus 4).
// Measured with the LDS bank-conflict counter on gfx950: with rows padded by
// 16 bytes every one of these reads conflicts (half of its LDS cycles);
// with 32 bytes of padding consecutive rows are conflict-free, and so are
// the strided sets once permuted by this slot map.  Rows are permuted inside
// 32-row blocks only.
__device__ __forceinline__ int wqkv_slot(int row) { return row ^ ((row >> 2) & 4); }

// PAD: elements of padding per staged row (8 = 16 bytes, 16 = 32 bytes)
template <bool WQKV = false, int PAD = 8>
__device__ __forceinline__ void stage_rows(bf16_t* dst, const bf16_t* __restrict__ src, int rows, int K,
                                           int tid, int nthreads) {
  const int c8n = K / 8, total = rows * c8n;
  for (int e0 = tid; e0 < total; e0 += SU * nthreads) {
    bf16x8 v[SU];
#pragma unroll
    for (int u = 0; u < SU; ++u) {
      int e = e0 + u * nthreads;
      e = e < total ? e : total - 1;
      v[u] = ld16(src + static_cast<int64_t>(e / c8n) * K + 8 * (e % c8n));
    }
#pragma unroll
    for (int u = 0; u < SU; ++u) {
      const int e = e0 + u * nthreads;
      const int row = WQKV ? wqkv_slot(e / c8n) : e / c8n;
      if (e < total) *reinterpret_cast<bf16x8*>(dst + row * (K + PAD) + 8 * (e % c8n)) = v[u];
    }
  }
}

template <int D>
struct QkvLds {
  static constexpr int NW = 8;
  static constexpr size_t lds_bytes = static_cast<size_t>(3) * D * (D + 8) * 2;
};

template <int D>
__global__ __launch_bounds__(64 * QkvLds<D>::NW) void qkv_proj_lds(Rows X, int64_t R, int64_t R_pad,
                                                    int64_t nproj, const bf16_t* __restrict__ W,
                                                    bf16_t* __restrict__ QK, bf16_t* __restrict__ Vp,
                                                    float qs, int64_t q_rows) {
  constexpr int KB = D / 32, NW = QkvLds<D>::NW;
  extern __shared__ __attribute__((aligned(16))) char smem[];
  bf16_t* Wl = reinterpret_cast<bf16_t*>(smem);
  stage_rows(Wl, W, 3 * D, D, threadIdx.x, NW * 64);
  lds_barrier();
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int g = lane >> 4, r = lane & 15;
  const int64_t nblk = nproj / 32;  // rows [0, nproj) are projected
  // whole rounds of 32-row blocks over all the waves; after at least one
  // such round a short remainder (its 16-row halves fit one round) is taken
  // as halves by twice as many waves, spread over the workgroups, so no wave
  // runs a lone extra full block (a half costs most of a block: the chain is
  // latency-bound, so a split pays only there)
  const int64_t nw = static_cast<int64_t>(gridDim.x) * NW;
  int64_t nfull = nblk / nw * nw;
  if (nfull == 0 || 2 * (nblk - nfull) > nw) nfull = nblk;
  for (int64_t blk = static_cast<int64_t>(blockIdx.x) * NW + w; blk < nfull; blk += nw) {
    const int64_t row0 = blk * 32;
    bf16x8 hb[2][KB];
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
      const int64_t row = row0 + 8 * (r >> 2) + 4 * rb + (r & 3);
      float v[8 * KB];
      if (row < R) {
        const bf16_t* xr = row_in<bf16_t>(X, row) + 8 * g;
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
          const bf16x8 x = ld16(xr + kb * 32);
#pragma unroll
          for (int j = 0; j < 8; ++j) v[8 * kb + j] = static_cast<float>(x[j]);
        }
      } else {
#pragma unroll
        for (int i = 0; i < 8 * KB; ++i) v[i] = 0.f;
      }
      ln_rows<8 * KB>(v, D);
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) hb[rb][kb] = pack8(v + 8 * kb);
    }
    // Q only for rows below q_rows (a multiple of 32): the rest need K and V
    qkv_chunk<D>(hb, Wl + opaque_zero(), D + 8, QK, Vp, row0, r, g, qs, Lay{32, R_pad * 32}, row0 < q_rows);
  }
  for (int64_t hid = static_cast<int64_t>(w) * gridDim.x + blockIdx.x; hid < 2 * (nblk - nfull); hid += nw) {
    const int64_t row0 = nfull * 32 + 16 * hid;
    const int64_t row = row0 + r;
    float x[1][D / 4];
    const bf16_t* xr = row < R ? row_in<bf16_t>(X, row) + 8 * g : nullptr;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      const bf16x8 v = xr ? ld16(xr + kb * 32) : zero8();
#pragma unroll
      for (int j = 0; j < 8; ++j) x[0][8 * kb + j] = static_cast<float>(v[j]);
    }
    qkv_rows<D, 1>(x, Wl + opaque_zero(), D + 8, QK, Vp, row0, r, g, Lay{32, R_pad * 32}, qs, row0 < q_rows);
  }
}

// LN(X) operands of two 16-row blocks: lane (r, g) of block rb holds row
// row_of(rb) of X, columns 32*kb + 8*g .. +8, as bf16 after the LN.
template <int D, typename F>
__device__ __forceinline__ void ln_operands(const Rows& X, F&& row_of, int g, bf16x8 (&hb)[2][D / 32]) {
  constexpr int KB = D / 32;
  bf16x8 xv[2][KB];
#pragma unroll
  for (int rb = 0; rb < 2; ++rb) {
    const bf16_t* xr = row_in<bf16_t>(X, row_of(rb)) + 8 * g;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) xv[rb][kb] = ld16(xr + kb * 32);
  }
#pragma unroll
  for (int rb = 0; rb < 2; ++rb) ln_bf16<KB>(xv[rb], D, hb[rb]);
}

// The products of the two projections below, with the weight fragments
// from wf: wf(c, kb) for Q or K (row 8 (r / 4) + 4 c + r % 4 of the head
// part, columns 32 kb + 8 g ..), wf(kb) for V.  FENCE keeps the fragments
// in flight bounded at d = 256 (registers) where wf loads them.
template <int D, bool FENCE, typename WF>
__device__ __forceinline__ void qk_products(const bf16x8 (&hb)[2][D / 32], WF&& wf, float f, f16x8 (&out)[2]) {
  constexpr int KB = D / 32;
  floatx4 acc[2][2] = {};
#pragma unroll
  for (int c = 0; c < 2; ++c) {
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      const bf16x8 a = wf(c, kb);
      acc[c][0] = mma(a, hb[0][kb], acc[c][0]);
      acc[c][1] = mma(a, hb[1][kb], acc[c][1]);
      if constexpr (KB > 4 && FENCE) {
        if (kb % 2 == 1) __builtin_amdgcn_sched_barrier(0);
      }
    }
  }
#pragma unroll
  for (int rb = 0; rb < 2; ++rb) {
    const float v[8] = {acc[0][rb][0] * f, acc[0][rb][1] * f, acc[0][rb][2] * f, acc[0][rb][3] * f,
                        acc[1][rb][0] * f, acc[1][rb][1] * f, acc[1][rb][2] * f, acc[1][rb][3] * f};
    out[rb] = packh8(v);
  }
}

template <int D, bool FENCE, typename WF>
__device__ __forceinline__ f16x8 v_products(const bf16x8 (&hb)[2][D / 32], WF&& wf) {
  constexpr int KB = D / 32;
  floatx4 a0 = {0.f, 0.f, 0.f, 0.f}, a1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int kb = 0; kb < KB; ++kb) {
    const bf16x8 bq = wf(kb);
    a0 = mma(hb[0][kb], bq, a0);
    a1 = mma(hb[1][kb], bq, a1);
    if constexpr (KB > 4 && FENCE) {
      if (kb % 2 == 1) __builtin_amdgcn_sched_barrier(0);
    }
  }
  const float v[8] = {a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
  return packh8(v);
}

// Q or K of head part p (p < H: Q, else K), multiplied by f, for the two row
// blocks of hb, in the transposed form: out[rb] lane (r, g) holds features
// 8g .. 8g+7 of the row that hb[rb] lane r carries.  W: w_qkv rows in LDS
// with row stride ldw, placed by wqkv_slot.
template <int D>
__device__ __forceinline__ void proj_qk_regs(const bf16x8 (&hb)[2][D / 32], const bf16_t* W, int ldw, int p,
                                             float f, int r, int g, f16x8 (&out)[2]) {
  qk_products<D, true>(hb, [&](int c, int kb) {
    return ld16(W + wqkv_slot(32 * p + 8 * (r >> 2) + 4 * c + (r & 3)) * ldw + 8 * g + kb * 32);
  }, f, out);
}

// V of two 16-row blocks whose rows are in the projection order (block rb,
// lane r: row 8*(r/4) + 4*rb + r%4), operands swapped: lane (r, g) ends with
// V of rows 8g .. 8g+7 for column `col_of(r)` of w_qkv's V part.
template <int D, typename F>
__device__ __forceinline__ f16x8 proj_v_regs(const bf16x8 (&hb)[2][D / 32], const bf16_t* W, int ldw,
                                              F&& col_of, int r, int g, int vrow0 = 2 * D) {
  const bf16_t* wr = W + wqkv_slot(vrow0 + col_of(r)) * ldw + 8 * g;
  return v_products<D, true>(hb, [&](int kb) { return ld16(wr + kb * 32); });
}

// The link operands of user b and head h (the HeadOps layouts) computed
// from the link rows of X: K and V from rows in the projection order, Q
// from rows in natural order.  Both Q_L and K_L carry the logit scale qs:
// each branch's scores then come out in log2 units with the history rows'
// Q and K left unscaled.
template <int ELL, int D>
__device__ __forceinline__ void link_ops(HeadOps<ELL>& o, const Rows& X, const bf16_t* W, int ldw, int b, int h,
                                         int r, int g, float qs) {
  constexpr int H = D / 32;
  const int64_t l0 = static_cast<int64_t>(b) * ELL;
#pragma unroll
  for (int kb2 = 0; kb2 < ELL / 32; ++kb2) {
    bf16x8 hb[2][D / 32];
    ln_operands<D>(X, [&](int rb) { return l0 + kb2 * 32 + 8 * (r >> 2) + 4 * rb + (r & 3); }, g, hb);
    f16x8 k2[2];
    proj_qk_regs<D>(hb, W, ldw, H + h, qs, r, g, k2);
    o.kl[2 * kb2] = k2[0];
    o.kl[2 * kb2 + 1] = k2[1];
#pragma unroll
    for (int c2 = 0; c2 < 2; ++c2)
      o.vlt[c2][kb2] = proj_v_regs<D>(hb, W, ldw, [&](int rr) { return 32 * h + 8 * (rr >> 2) + 4 * c2 + (rr & 3); },
                                      r, g);
    ln_operands<D>(X, [&](int rb) { return l0 + kb2 * 32 + 16 * rb + r; }, g, hb);
    f16x8 q2[2];
    proj_qk_regs<D>(hb, W, ldw, h, qs, r, g, q2);
    o.qlt[2 * kb2] = q2[0];
    o.qlt[2 * kb2 + 1] = q2[1];
  }
}

// XOR attention with the history rows' LN + QKV projection fused in, for
// d <= 128 (w_qkv fits LDS).  A history row's Q, K and V feed only the
// attention of its own chunk (there are no history-to-history terms), so
// they stay in registers, already in the attention's operand layouts: the
// kernel reads the residual rows X and writes Y, where a separate projection
// would write Q|K and V to HBM and read them back.  Each wave also projects
// its user's link rows for its head (K_L, V_L, Q_L: the HeadOps operands),
// so a layer needs no projection launch.
// A workgroup of 8 waves holds w_qkv in LDS (rows padded by 32 bytes) and
// runs SPW = 8 / H splits with one wave per (split, head); splits and
// partials as in xor_attn.  The H waves of a split share each chunk's LN:
// every wave normalizes 32 / H of its rows into an LDS chunk buffer (two per
// split, alternating), and after one workgroup barrier per chunk each wave
// reads the rows it needs as projection operands.  The splits of a
// workgroup run the same number of barrier steps (the most chunks of any of
// them); a split out of chunks only joins the barriers.
template <int ELL, int H>
struct FusedCfg {
  // rows padded by 32 bytes (LDW): with the wqkv_slot row order, fragment
  // reads of the staged weights and of the LN chunk rows are conflict-free
  static constexpr int D = 32 * H, NW = 8, SPW = NW / H, LDW = D + 16;
  static constexpr int RPWV = 32 / H;  // chunk rows each wave normalizes
  static constexpr size_t w_elems = static_cast<size_t>(3) * D * LDW;
  static constexpr size_t buf_elems = static_cast<size_t>(32) * LDW;
  static constexpr size_t lds_bytes = (w_elems + 2 * SPW * buf_elems) * 2 + 4 * SPW;
};

// Sum over the lanes of a wave that share lane % N (N = 8 or 16): xor
// steps of N (a row rotation by 8 within 16 lanes when N = 8), 16 and 32.
template <int N>
__device__ __forceinline__ float group_sum(float x) {
  static_assert(N == 8 || N == 16, "group");
  if constexpr (N == 8) {
    // row_ror:8 within each 16-lane row: lane i reads lane i ^ 8
    const int o = __builtin_amdgcn_mov_dpp(__float_as_int(x), 0x128, 0xf, 0xf, false);
    x += __int_as_float(o);
  }
  return rows_sum(x);
}

template <int ELL, int H>
__global__ __launch_bounds__(512) void xor_attn_qkv(Rows X, const bf16_t* __restrict__ W,
                                                    bf16_t* __restrict__ Y, float* __restrict__ part,
                                                    const int64_t* __restrict__ off,
                                                    const int32_t* __restrict__ split_off,
                                                    const int32_t* __restrict__ split_user, int B, int G,
                                                    int64_t chunk, int64_t total_N, int phi, int do_e,
                                                    float qs) {
  using C = FusedCfg<ELL, H>;
  constexpr int D = C::D, KB = D / 32, MB = ELL / 16, LDW = C::LDW, RPWV = C::RPWV, SPW = C::SPW;
  // splits are numbered without gaps, so a workgroup whose first slot holds
  // none has nothing to do (slots past the last split: the grid covers G,
  // an upper bound); it leaves before staging the weights
  {
    const int64_t x0 = static_cast<int64_t>(blockIdx.x) * SPW;
    if (x0 >= G || split_user[x0] < 0) return;
  }
  extern __shared__ __attribute__((aligned(16))) char smem[];
  bf16_t* Wl = reinterpret_cast<bf16_t*>(smem);
  bf16_t* hbuf = Wl + C::w_elems;  // [SPW][2][32][LDW]
  int* nchs = reinterpret_cast<int*>(hbuf + 2 * SPW * C::buf_elems);
  stage_rows<true, LDW - D>(Wl, W, 3 * D, D, threadIdx.x, C::NW * 64);
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int g = lane >> 4, r = lane & 15;
  const int sidx = w / H, h = w % H;
  const int64_t x = static_cast<int64_t>(blockIdx.x) * SPW + sidx;  // split
  const int b = x < G ? split_user[x] : -1;
  const bool has = b >= 0;  // uniform over the split's waves
  const int64_t nlr = static_cast<int64_t>(B) * ELL;
  int64_t lo = 0, hi = 0;
  if (has) {
    const int64_t sx = x - split_off[b];
    const int64_t u0 = clamp64(off[b], 0, total_N);
    const int64_t u1 = clamp64(off[b + 1], u0, total_N);
    split_rows(u0, u1, sx, chunk, &lo, &hi);
  }
  const int64_t c0s = lo & ~int64_t(7);
  const int nch = c0s < hi ? static_cast<int>((hi - 1 - c0s) >> 5) + 1 : 0;
  if (h == 0 && lane == 0) nchs[sidx] = nch;
  lds_barrier();
  int nmax = 0;
#pragma unroll
  for (int q = 0; q < SPW; ++q) nmax = nchs[q] > nmax ? nchs[q] : nmax;
  const bool softmax = (phi == PHI_SOFTMAX);

  HeadOps<ELL> o;
  const Lay yl{32, (nlr + total_N) * 32};
  if (has) link_ops<ELL, D>(o, X, Wl + opaque_zero(), LDW, b, h, r, g, qs);
  LState<ELL> st;
  st.init();
  // LN lanes: chunk row crow = RPWV*h + lr, features 16*fg .. +16
  const int lr = lane % RPWV, fg = lane / RPWV, crow = RPWV * h + lr;
  with_phi(softmax, [&](auto phi_tag) {
    with_flag(do_e != 0, [&](auto e_tag) {
      constexpr bool SM = decltype(phi_tag)::value, DO_E = decltype(e_tag)::value;
      // this lane's X row of chunk i (clamped: past the history end or past
      // the split's chunks it is read but not used)
      auto ldx = [&](bf16x8(&xv)[2], int i) {
        int64_t j = c0s + 32 * i + crow;
        j = j < total_N ? j : total_N - 1;
        const bf16_t* p = row_in<bf16_t>(X, nlr + j) + 16 * fg;
        xv[0] = ld16(p);
        xv[1] = ld16(p + 8);
      };
      auto step = [&](const bf16x8(&xc)[2], bf16x8(&xn)[2], int i, int par) {
        ldx(xn, i + 1);
        const bool active = i < nch;
        bf16_t* buf = hbuf + (sidx * 2 + par) * C::buf_elems;
        if (active) {
          // LN of this lane's 16 values of row crow; the row's other values
          // are in the lanes with the same lr
          const bf16x2 one = {static_cast<__bf16>(1.f), static_cast<__bf16>(1.f)};
          float sm[2] = {0.f, 0.f}, sq[2] = {0.f, 0.f};
#pragma unroll
          for (int u = 0; u < 2; ++u)
#pragma unroll
            for (int pp = 0; pp < 4; ++pp) {
              const bf16x2 v = {xc[u][2 * pp], xc[u][2 * pp + 1]};
              sm[u] = __builtin_amdgcn_fdot2_f32_bf16(v, one, sm[u], false);
              sq[u] = __builtin_amdgcn_fdot2_f32_bf16(v, v, sq[u], false);
            }
          const float sum = group_sum<RPWV>(sm[0] + sm[1]), ssq = group_sum<RPWV>(sq[0] + sq[1]);
          constexpr float inv_d = 1.f / static_cast<float>(D);
          const float mu = sum * inv_d;
          float var = ssq * inv_d - mu * mu;
          if (wave_needs_centred_var(mu, var)) {
            float c[2] = {0.f, 0.f};
#pragma unroll
            for (int u = 0; u < 2; ++u)
#pragma unroll
              for (int jj = 0; jj < 8; ++jj) {
                const float dv = static_cast<float>(xc[u][jj]) - mu;
                c[u] = fmaf(dv, dv, c[u]);
              }
            var = group_sum<RPWV>(c[0] + c[1]) * inv_d;
          }
          const float rs = rsqrtf(fmaxf(var, 0.f) + 1e-5f);
          const float nb = -mu * rs;
#pragma unroll
          for (int u = 0; u < 2; ++u) {
            float v[8];
#pragma unroll
            for (int jj = 0; jj < 8; ++jj) v[jj] = fmaf(static_cast<float>(xc[u][jj]), rs, nb);
            *reinterpret_cast<bf16x8*>(buf + wqkv_slot(crow) * LDW + 16 * fg + 8 * u) = pack8(v);
          }
        }
        lds_barrier();
        if (active) {
          const int64_t c0 = c0s + 32 * i;
          // the chunk's LN rows in the projection order
          bf16x8 hb[2][KB];
#pragma unroll
          for (int rb = 0; rb < 2; ++rb)
#pragma unroll
            for (int kb = 0; kb < KB; ++kb)
              hb[rb][kb] = *reinterpret_cast<const bf16x8*>(
                  buf + wqkv_slot(8 * (r >> 2) + 4 * rb + (r & 3)) * LDW + 32 * kb + 8 * g);
          const bf16_t* Wb = Wl + opaque_zero();
          ChunkOps ci;
          // (the logit scale is on the link side)
          if constexpr (DO_E) proj_qk_regs<D>(hb, Wb, LDW, h, 1.f, r, g, ci.qe);
          proj_qk_regs<D>(hb, Wb, LDW, H + h, 1.f, r, g, ci.ke);
#pragma unroll
          for (int c2 = 0; c2 < 2; ++c2)
            ci.ve[c2] = proj_v_regs<D>(hb, Wb, LDW, [&](int rr) { return 32 * h + 16 * c2 + rr; }, r, g);
          if constexpr (DO_E) e_branch<ELL, D, SM, 0, true>(o, ci, Y, nlr, c0, lo, hi, h, r, g, yl);
          l_branch<ELL, SM>(st, o, ci, c0, lo, hi, r, g);
        }
      };
      bf16x8 xa[2], xb[2];
      ldx(xa, 0);
      for (int i = 0; i + 2 <= nmax; i += 2) {
        step(xa, xb, i, 0);
        step(xb, xa, i + 1, 1);
      }
      if (nmax & 1) step(xa, xb, nmax - 1, 0);
    });
  });
  if (!has) return;
  float* p0 = part + ((x * H + h) * ELL) * PART_LD;
#pragma unroll
  for (int nb = 0; nb < MB; ++nb) {
    // partials in natural units: max * ln 2; silu sums * ln 2
    float* pl = p0 + (16 * nb + r) * PART_LD;
    if (g == 0) {
      pl[0] = softmax ? st.m[nb] * LN2 : 0.f;
      pl[1] = softmax ? st.l[nb] : static_cast<float>(hi - lo);
    }
    const float f = softmax ? 1.f : LN2;
#pragma unroll
    for (int c2 = 0; c2 < 2; ++c2)
      *reinterpret_cast<floatx4*>(pl + 4 + 16 * c2 + 4 * g) =
          floatx4{st.acc[nb][c2][0] * f, st.acc[nb][c2][1] * f, st.acc[nb][c2][2] * f, st.acc[nb][c2][3] * f};
  }
}

// ---------------------------------------------------------------------------
// XOR attention with the history rows' QKV projection fused in, for d = 256,
// whose w_qkv (384 KB) LDS cannot hold: a workgroup serves SPW = 4 splits
// and a group of HG = 2 heads, with those heads' 192 rows of w_qkv staged in
// LDS (Q rows, then K rows, then V rows, 32 per head); one wave per (split,
// head) loads its user's link operands (projected once per user and head by
// link_qkv_h) and projects each 32-row chunk of its split itself, so the
// history rows' Q, K and V never leave the registers.  The rows come from Hs,
// LayerNorm(X) of every row that the previous layer's post block stored as
// bf16 (LNX = false), or, in the first layer, from X normalised here
// (LNX = true).  Each head group reads a split's rows once; block indices
// are laid out so that the NHG head groups of a split run on one XCD close
// together and share its rows in L2.  The next chunk's rows load into the
// operand registers as soon as the projection has used them, while the
// attention of the current chunk runs.
// ---------------------------------------------------------------------------
template <int ELL>
struct FusedHCfg {
  static constexpr int D = 256, H = 8, HG = 2, NW = 8, SPW = NW / HG, NHG = H / HG, LDW = D + 16;
  static constexpr size_t w_elems = static_cast<size_t>(3) * HG * 32 * LDW;
  static constexpr size_t lds_bytes = w_elems * 2;
  // workgroups for G split slots: split groups rounded up to a multiple of
  // the 8 XCDs, times the head groups
  static constexpr int64_t grid(int64_t G) { return ((G + SPW - 1) / SPW + 7) / 8 * 8 * NHG; }
};

// Operands of two 16-row blocks (lane (r, g) of block rb: row row_of(rb) of
// src, columns 32 kb + 8 g .. +8): the rows as stored (H rows), or their
// LayerNorm (X rows, LNX).
template <int D, bool LNX, typename F>
__device__ __forceinline__ void row_operands(const Rows& src, F&& row_of, int g, bf16x8 (&hb)[2][D / 32]) {
  if constexpr (LNX) {
    ln_operands<D>(src, row_of, g, hb);
  } else {
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
      const bf16_t* xr = row_in<bf16_t>(src, row_of(rb)) + 8 * g;
#pragma unroll
      for (int kb = 0; kb < D / 32; ++kb) hb[rb][kb] = ld16(xr + kb * 32);
    }
  }
}

// Link operands of xor_attn_h, projected once per (user, head) instead of
// by every split of the user: the HeadOps registers of one wave, stored
// lane-major.  Register k of lane t of (user b, head h) is element
// ((b H + h) NREG + k) 64 + t, in the order kl[0..MB), qlt[0..MB),
// vlt[0][0..KBL), vlt[1][0..KBL): each split's waves then load them with one
// coalesced 16-byte load per register.
template <int ELL>
struct LinkOpsLayout {
  static constexpr int MB = ELL / 16, KBL = ELL / 32, NREG = 2 * MB + 2 * KBL;
  static constexpr int KL = 0, QLT = MB, VLT = 2 * MB;
};

// One wave per (user, head, job), each job one 32-link block: K_L and V_L
// from its rows in the projection order, or Q_L from its rows in natural
// order (without DO_E, a last layer, only Q_L is used).  The weight
// fragments come straight from w_qkv in global memory (384 KB, read into
// each XCD's L2 once): a workgroup that staged them in LDS first would
// spend most of its time on that.  Both Q_L and K_L carry
// the logit scale qs (the history rows' Q and K are left unscaled, and
// each branch's scores come out in log2 units).
template <int ELL, bool DO_E>
struct LinkQkvCfg {
  static constexpr int KBL = ELL / 32, JOBS = DO_E ? 2 * KBL : KBL;
  static constexpr int64_t grid(int B) { return static_cast<int64_t>(B) * FusedHCfg<ELL>::H * JOBS; }
};

template <int ELL, bool DO_E>
__global__ __launch_bounds__(64) void link_qkv_h(Rows src, const bf16_t* __restrict__ W, void* __restrict__ ops_,
                                                 float qs) {
  using LO = LinkOpsLayout<ELL>;
  constexpr int D = FusedHCfg<ELL>::D, H = FusedHCfg<ELL>::H, KBL = LO::KBL, JOBS = LinkQkvCfg<ELL, DO_E>::JOBS;
  const int job = static_cast<int>(blockIdx.x % JOBS) + (DO_E ? 0 : KBL);
  const int h = static_cast<int>((blockIdx.x / JOBS) % H), b = static_cast<int>(blockIdx.x / (JOBS * H));
  const int lane = threadIdx.x, g = lane >> 4, r = lane & 15;
  f16x8* rec = static_cast<f16x8*>(ops_) + (static_cast<int64_t>(b) * H + h) * LO::NREG * 64 + lane;
  // jobs [0, KBL): K_L and V_L of link block kb2 = job; [KBL, 2 KBL): Q_L.
  // Every operand is loaded before the first product (one memory latency;
  // the fused kernels load weight fragments as they go, from LDS).
  constexpr int KB = D / 32;
  const int kb2 = job < KBL ? job : job - KBL;
  const int64_t l0 = static_cast<int64_t>(b) * ELL + 32 * kb2;
  bf16x8 hb[2][KB];
  bf16x8 wa[2][KB];
  const int p = job < KBL ? H + h : h;
#pragma unroll
  for (int c = 0; c < 2; ++c)
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
      wa[c][kb] = ld16(W + static_cast<int64_t>(32 * p + 8 * (r >> 2) + 4 * c + (r & 3)) * D + 8 * g + 32 * kb);
  if (job < KBL) {
    row_operands<D, false>(src, [&](int rb) { return l0 + 8 * (r >> 2) + 4 * rb + (r & 3); }, g, hb);
    bf16x8 wv[2][KB];
#pragma unroll
    for (int c2 = 0; c2 < 2; ++c2)
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
        wv[c2][kb] = ld16(W + static_cast<int64_t>(2 * D + 32 * h + 8 * (r >> 2) + 4 * c2 + (r & 3)) * D + 8 * g +
                          32 * kb);
    __builtin_amdgcn_sched_barrier(0);
    f16x8 k2[2];
    qk_products<D, false>(hb, [&](int c, int kb) { return wa[c][kb]; }, qs, k2);
    rec[(LO::KL + 2 * kb2) * 64] = k2[0];
    rec[(LO::KL + 2 * kb2 + 1) * 64] = k2[1];
#pragma unroll
    for (int c2 = 0; c2 < 2; ++c2)
      rec[(LO::VLT + c2 * KBL + kb2) * 64] = v_products<D, false>(hb, [&](int kb) { return wv[c2][kb]; });
  } else {
    row_operands<D, false>(src, [&](int rb) { return l0 + 16 * rb + r; }, g, hb);
    __builtin_amdgcn_sched_barrier(0);
    f16x8 q2[2];
    qk_products<D, false>(hb, [&](int c, int kb) { return wa[c][kb]; }, qs, q2);
    rec[(LO::QLT + 2 * kb2) * 64] = q2[0];
    rec[(LO::QLT + 2 * kb2 + 1) * 64] = q2[1];
  }
}

// LayerNorm (no affine, eps 1e-5) of every row of X as bf16 [R, D]: the
// first layer's operands of xor_attn_h (later layers get theirs from the
// post block).  D / 8 lanes per row, 16 bytes each; two-pass statistics.
template <int D>
__global__ __launch_bounds__(256) void ln_rows_kernel(Rows X, int64_t R, bf16_t* __restrict__ out) {
  constexpr int LPR = D / 8;            // lanes per row
  constexpr int RPB = 256 / LPR;        // rows per block step
  static_assert(LPR == 32, "written for d = 256");
  const int tid = threadIdx.x, c8 = tid % LPR;
  for (int64_t row = static_cast<int64_t>(blockIdx.x) * RPB + tid / LPR; row < R;
       row += static_cast<int64_t>(gridDim.x) * RPB) {
    const bf16x8 x = ld16(row_in<bf16_t>(X, row) + 8 * c8);
    float v[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) v[q] = static_cast<float>(x[q]);
    float s = ((v[0] + v[1]) + (v[2] + v[3])) + ((v[4] + v[5]) + (v[6] + v[7]));
#pragma unroll
    for (int o = 1; o < LPR; o <<= 1) s += __shfl_xor(s, o);
    const float mu = s * (1.f / static_cast<float>(D));
    float t = 0.f;
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const float u = v[q] - mu;
      t = fmaf(u, u, t);
    }
#pragma unroll
    for (int o = 1; o < LPR; o <<= 1) t += __shfl_xor(t, o);
    const float rs = rsqrtf(t * (1.f / static_cast<float>(D)) + 1e-5f);
#pragma unroll
    for (int q = 0; q < 8; ++q) v[q] = (v[q] - mu) * rs;
    st8(out + row * D + 8 * c8, v);
  }
}

// DO_E: the layer also updates history rows (the E-branch).  Without it
// (a last layer) Q_E, K_L and V_L are dead, and at l = 32 the freed
// registers hold a second operand buffer: the rows are loaded two chunks
// ahead (at l = 64 the second buffer would not fit the 256 registers of a
// wave without spilling).
template <int ELL, bool LNX, bool DO_E>
__global__ __launch_bounds__(512) void xor_attn_h(Rows src, const bf16_t* __restrict__ W,
                                                  const void* __restrict__ lops, bf16_t* __restrict__ Y,
                                                  float* __restrict__ part, const int64_t* __restrict__ off,
                                                  const int32_t* __restrict__ split_off,
                                                  const int32_t* __restrict__ split_user, int B, int G,
                                                  int64_t chunk, int64_t total_N, int phi) {
  using C = FusedHCfg<ELL>;
  constexpr int D = C::D, H = C::H, HG = C::HG, SPW = C::SPW, NHG = C::NHG, MB = ELL / 16, LDW = C::LDW;
  // block -> (split group, head group): the NHG head groups of a split
  // group take consecutive slots of one XCD (blocks are spread over the 8
  // XCDs round-robin)
  const int64_t slot = blockIdx.x >> 3;
  const int hgi = static_cast<int>(slot % NHG);
  const int64_t sg = (slot / NHG) * 8 + (blockIdx.x & 7);
  {
    const int64_t x0 = sg * SPW;
    if (x0 >= G || split_user[x0] < 0) return;  // slots past the last split
  }
  extern __shared__ __attribute__((aligned(16))) char smem[];
  bf16_t* Wl = reinterpret_cast<bf16_t*>(smem);
  // the head group's rows of w_qkv: Q, K, V parts, HG * 32 rows each (the
  // history rows' Q only where they are updated)
#pragma unroll
  for (int part3 = DO_E ? 0 : 1; part3 < 3; ++part3)
    stage_rows<true, LDW - D>(Wl + part3 * HG * 32 * LDW, W + (static_cast<int64_t>(part3) * D + hgi * HG * 32) * D, HG * 32, D,
               threadIdx.x, C::NW * 64);
  lds_barrier();
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int g = lane >> 4, r = lane & 15;
  const int j = w % HG, h = hgi * HG + j;
  const int64_t x = sg * SPW + w / HG;  // split
  const int b = x < G ? split_user[x] : -1;
  if (b < 0) return;  // no barrier follows
  const int64_t nlr = static_cast<int64_t>(B) * ELL;
  int64_t lo = 0, hi = 0;
  {
    const int64_t sx = x - split_off[b];
    const int64_t u0 = clamp64(off[b], 0, total_N);
    const int64_t u1 = clamp64(off[b + 1], u0, total_N);
    split_rows(u0, u1, sx, chunk, &lo, &hi);
  }
  const int64_t c0s = lo & ~int64_t(7);
  const int nch = c0s < hi ? static_cast<int>((hi - 1 - c0s) >> 5) + 1 : 0;
  const bool softmax = (phi == PHI_SOFTMAX);
  const bf16_t* Wb = Wl + opaque_zero();

  // the user's link operands for head h, from link_qkv_h (without DO_E
  // only Q_L is live)
  HeadOps<ELL> o;
  {
    using LO = LinkOpsLayout<ELL>;
    const f16x8* rec = static_cast<const f16x8*>(lops) + (static_cast<int64_t>(b) * H + h) * LO::NREG * 64 + lane;
#pragma unroll
    for (int c = 0; c < MB; ++c) {
      if constexpr (DO_E) o.kl[c] = rec[(LO::KL + c) * 64];
      o.qlt[c] = rec[(LO::QLT + c) * 64];
    }
    if constexpr (DO_E) {
#pragma unroll
      for (int c2 = 0; c2 < 2; ++c2)
#pragma unroll
        for (int kb = 0; kb < LO::KBL; ++kb) o.vlt[c2][kb] = rec[(LO::VLT + c2 * LO::KBL + kb) * 64];
    }
  }
  LState<ELL> st;
  st.init();
  const Lay yl{32, (nlr + total_N) * 32};
  with_phi(softmax, [&](auto phi_tag) {
    constexpr bool SM = decltype(phi_tag)::value;
    using Ops = bf16x8[2][D / 32];
    // chunk i's rows in the projection order (clamped: past the history
    // end they are read but not used)
    auto load = [&](Ops& hb, int i) {
      const int64_t c0 = c0s + 32 * i;
      row_operands<D, LNX>(src, [&](int rb) {
        int64_t jj = c0 + 8 * (r >> 2) + 4 * rb + (r & 3);
        jj = jj < total_N ? jj : total_N - 1;
        return nlr + jj;
      }, g, hb);
    };
    auto project = [&](const Ops& hb, ChunkOps& ci) {
      // (the logit scale is on the link side)
      if constexpr (DO_E) proj_qk_regs<D>(hb, Wb, LDW, j, 1.f, r, g, ci.qe);
      proj_qk_regs<D>(hb, Wb, LDW, HG + j, 1.f, r, g, ci.ke);
#pragma unroll
      for (int c2 = 0; c2 < 2; ++c2)
        ci.ve[c2] = proj_v_regs<D>(hb, Wb, LDW, [&](int rr) { return 32 * j + 16 * c2 + rr; }, r, g, 2 * HG * 32);
    };
    auto attend = [&](const ChunkOps& ci, int64_t c0) {
      // the attention's dependent VALU chains take issue priority over the
      // projection products of the SIMD's other wave (3% per layer)
      __builtin_amdgcn_s_setprio(1);
      if constexpr (DO_E) e_branch<ELL, D, SM, 0, true>(o, ci, Y, nlr, c0, lo, hi, h, r, g, yl);
      l_branch<ELL, SM>(st, o, ci, c0, lo, hi, r, g);
      __builtin_amdgcn_s_setprio(0);
    };
    if constexpr (DO_E || ELL > 32) {
      // one chunk ahead, into the operand registers the projections have
      // just freed, while this chunk's attention runs
      Ops hb;
      if (nch > 0) load(hb, 0);
      for (int i = 0; i < nch; ++i) {
        ChunkOps ci;
        project(hb, ci);
        if (i + 1 < nch) load(hb, i + 1);
        attend(ci, c0s + 32 * i);
      }
    } else if (nch > 0) {
      // two chunks ahead in two buffers that alternate by name; every step
      // issues its load (past the last chunk it rereads that chunk, unused)
      // so that the waits stay exact
      Ops ha, hz;
      auto step = [&](Ops& hb, int i) {
        ChunkOps ci;
        project(hb, ci);
        load(hb, i + 2 < nch ? i + 2 : nch - 1);
        attend(ci, c0s + 32 * i);
      };
      load(ha, 0);
      load(hz, nch > 1 ? 1 : 0);
      int i = 0;
      for (; i + 2 <= nch; i += 2) {
        step(ha, i);
        step(hz, i + 1);
      }
      if (i < nch) step(ha, i);
    }
  });
  float* p0 = part + ((x * H + h) * ELL) * PART_LD;
#pragma unroll
  for (int nb = 0; nb < MB; ++nb) {
    // partials in natural units: max * ln 2; silu sums * ln 2
    float* pl = p0 + (16 * nb + r) * PART_LD;
    if (g == 0) {
      pl[0] = softmax ? st.m[nb] * LN2 : 0.f;
      pl[1] = softmax ? st.l[nb] : static_cast<float>(hi - lo);
    }
    const float f = softmax ? 1.f : LN2;
#pragma unroll
    for (int c2 = 0; c2 < 2; ++c2)
      *reinterpret_cast<floatx4*>(pl + 4 + 16 * c2 + 4 * g) =
          floatx4{st.acc[nb][c2][0] * f, st.acc[nb][c2][1] * f, st.acc[nb][c2][2] * f, st.acc[nb][c2][3] * f};
  }
}

template <int D, int DFF>
struct PostLds {
  static constexpr int NW = 8;
  static constexpr size_t lds_bytes =
      (static_cast<size_t>(D) * (D + 8) + 2 * static_cast<size_t>(DFF) * (D + 8) +
       static_cast<size_t>(D) * (DFF + 8)) * 2;
};

template <int D, int DFF, int RPW>
__global__ __launch_bounds__((64 * PostLds<D, DFF>::NW)) void post_block_lds(const bf16_t* __restrict__ Y, int64_t yR,
                                                                             Rows Xres, Rows Out, int64_t nrows,
                                                      const bf16_t* __restrict__ Wo,
                                                      const bf16_t* __restrict__ Wg,
                                                      const bf16_t* __restrict__ Wu,
                                                      const bf16_t* __restrict__ Wd) {
  constexpr int KB = D / 32, RB = RPW / 16, NW = PostLds<D, DFF>::NW;
  extern __shared__ __attribute__((aligned(16))) char smem[];
  bf16_t* Wol = reinterpret_cast<bf16_t*>(smem);
  bf16_t* Wgl = Wol + D * (D + 8);
  bf16_t* Wul = Wgl + DFF * (D + 8);
  bf16_t* Wdl = Wul + DFF * (D + 8);
  stage_rows(Wol, Wo, D, D, threadIdx.x, NW * 64);
  stage_rows(Wgl, Wg, DFF, D, threadIdx.x, NW * 64);
  stage_rows(Wul, Wu, DFF, D, threadIdx.x, NW * 64);
  stage_rows(Wdl, Wd, D, DFF, threadIdx.x, NW * 64);
  lds_barrier();
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int g = lane >> 4, r = lane & 15;
  // the post block of NB 16-row blocks from row0
  auto rows_block = [&](auto nb_tag, int64_t row0) {
    constexpr int NB = decltype(nb_tag)::value;
    // every load is issued (rows past nrows read the last row and are not
    // stored), Y's first: the W_o product waits on Y only, the residual is
    // first read in its epilogue
    bf16x8 yb[NB][KB], xb[NB][KB];
    float x1[NB][D / 4];
#pragma unroll
    for (int rb = 0; rb < NB; ++rb) {
      int64_t row = row0 + 16 * rb + r;
      row = row < nrows ? row : nrows - 1;
      const bf16_t* yr = Y + row * 32 + 8 * g;  // head-planar: head kb at kb * yR * 32
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) yb[rb][kb] = ld16(yr + kb * yR * 32);
    }
#pragma unroll
    for (int rb = 0; rb < NB; ++rb) {
      int64_t row = row0 + 16 * rb + r;
      row = row < nrows ? row : nrows - 1;
      const bf16_t* xr = row_in<bf16_t>(Xres, row) + 8 * g;
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) xb[rb][kb] = ld16(xr + kb * 32);
    }
    const int z = opaque_zero();
    post_rows<D, DFF, NB, true>(yb, x1, Wol + z, Wgl + z, Wul + z, Wdl + z, D + 8, DFF + 8, r, g, xb);
#pragma unroll
    for (int rb = 0; rb < NB; ++rb) {
      const int64_t row = row0 + 16 * rb + r;
      if (row >= nrows) continue;
      bf16_t* orow = row_out<bf16_t>(Out, row);
      if (orow == nullptr) continue;
#pragma unroll
      for (int p = 0; p < KB; ++p) st8(orow + 32 * p + 8 * g, &x1[rb][8 * p]);
    }
  };
  // whole rounds of RPW-row blocks over all the waves; after at least one
  // such round a short remainder (its 16-row blocks fit one round) is taken
  // as 16-row blocks by more waves, spread over the workgroups, so no wave
  // runs a lone extra full block
  const int64_t nblk = (nrows + RPW - 1) / RPW;
  const int64_t nw = static_cast<int64_t>(gridDim.x) * NW;
  int64_t nfull = nblk / nw * nw;
  if (nfull == 0 || (RPW / 16) * (nblk - nfull) > nw) nfull = nblk;
  for (int64_t blk = static_cast<int64_t>(blockIdx.x) * NW + w; blk < nfull; blk += nw)
    rows_block(std::integral_constant<int, RB>{}, blk * RPW);
  for (int64_t hid = static_cast<int64_t>(w) * gridDim.x + blockIdx.x; nfull * RPW + 16 * hid < nrows; hid += nw)
    rows_block(std::integral_constant<int, 1>{}, nfull * RPW + 16 * hid);
}

// ---------------------------------------------------------------------------
// Weight-streaming variants for widths whose weights do not fit in LDS
// (d = 256).  A workgroup takes a tile of rows held in registers and
// streams the weights through two LDS buffers of 64-row chunks, chunk c + 1
// loading while the waves multiply by chunk c, so weight traffic from L2 is
// one pass per tile instead of one per wave.  The projection (8 waves, 32
// rows each) loads chunks through registers into padded rows; the
// post-attention block (4 waves, 16 rows each) loads them straight into LDS
// into unpadded rows with swizzled 16-byte slots.
// ---------------------------------------------------------------------------
// ---------------------------------------------------------------------------
// Weight streaming through LDS by LDS-DMA (d = 256 kernels)
// ---------------------------------------------------------------------------
// A raw buffer descriptor over `elems` bf16 elements at p (gfx9-family
// word 3: raw 32-bit accesses, no stride); loads past the extent return 0.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t weight_rsrc(const bf16_t* p, int elems) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<bf16_t*>(p), 0, elems * 2, 0x00020000);
}

// LN + QKV projection with w_qkv streamed through LDS (d = 256: 384 KB of
// weights).  Workgroups of 4 waves, two per CU, each wave 32 rows: a tile
// is 128 rows and 12 chunks of 64 weight rows (0..7: Q|K column pairs,
// 8..11: V blocks).  Chunks travel global -> LDS directly (LDS-DMA buffer
// loads); two buffers, the next chunk in flight while one is computed, and
// the second workgroup of the CU covers the first's tile-start loads.  LDS
// rows are unpadded with their 16-byte slots XOR-swizzled by swz_qkv(row),
// which keeps both fragment patterns conflict-free: the Q|K rows
// 32 p + 8 (r / 4) + 4 c + r % 4 and the V rows 16 n + r of lanes r = 0..15.
template <int D>
struct StreamCfg {
  static constexpr int NW = 4, NT = 64 * NW;
  static constexpr int CR = 64;                       // weight rows per chunk
  static constexpr int SPR = D / 8;                   // 16-byte slots per row
  static constexpr int CPT = CR * SPR / NT;           // LDS-DMA slots per thread per chunk
  static constexpr int TILE = 32 * NW;                // rows per tile
  static constexpr size_t lds_bytes = static_cast<size_t>(2) * CR * D * 2;
  static_assert((CR * SPR) % NT == 0, "chunk split");
};

__device__ __forceinline__ int swz_qkv(int row) { return (row & 3) | ((((row >> 3) ^ (row >> 2)) & 3) << 2); }

template <int D>
__global__ __launch_bounds__(256, 2) void qkv_proj_stream(Rows X, int64_t R, int64_t R_pad,
                                                          const bf16_t* __restrict__ W,
                                                          bf16_t* __restrict__ QK, bf16_t* __restrict__ Vp,
                                                          float qs, int64_t q_rows) {
  using C = StreamCfg<D>;
  constexpr int KB = D / 32, NW = C::NW, CR = C::CR, CPT = C::CPT;
  constexpr int NCH = 3 * D / CR, NQK = 2 * D / CR;
  static_assert(C::NT / C::SPR == 8 && CPT == 8, "load pattern assumes 8 rows per step");
  extern __shared__ __attribute__((aligned(16))) char smem[];
  bf16_t* const buf0 = reinterpret_cast<bf16_t*>(smem);
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int g = lane >> 4, r = lane & 15;
  const int64_t ntiles = (R_pad + C::TILE - 1) / C::TILE;
  const int64_t my_tiles = (ntiles - blockIdx.x + gridDim.x - 1) / gridDim.x;
  const int64_t total = my_tiles * NCH;
  if (total <= 0) return;

  // chunk k: weight rows [64 k, 64 k + 64) of w_qkv.  Step i of a chunk is
  // its row 8 i + tid / 32, physical slot tid % 32, fetched by this thread
  // with one LDS-DMA load (a wave fills 1 KB of LDS in a row): the chunk
  // base is a scalar offset into one buffer descriptor, the lane's part a
  // constant per step.
  const __amdgpu_buffer_rsrc_t rsw = weight_rsrc(W, 3 * D * D);
  const int lrow = tid >> 5;
  const int wu = __builtin_amdgcn_readfirstlane(w);
  auto issue_chunk = [&](int k, bf16_t* buf) {
    const unsigned base = static_cast<unsigned>(CR * k * D * 2);
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int row = 8 * i + lrow;
      const unsigned vo = static_cast<unsigned>((row * D + 8 * ((tid & 31) ^ swz_qkv(row))) * 2);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsw, (lds_void_t*)(buf + (i * C::NT + wu * 64) * 8), 16, vo,
                                               base, 0, 0);
    }
  };
  // the fragment of chunk row `row` (lane's k-slice kb) in a chunk buffer
  auto frag = [&](const bf16_t* wb, int row, int kb) {
    return ld16(wb + row * D + 8 * ((4 * kb + g) ^ swz_qkv(row)));
  };

  issue_chunk(0, buf0);
  wait_vm<0>();
  dma_barrier();
  bf16x8 hb[2][KB];
  bool active = false;
  int64_t row0 = 0;
  for (int64_t c = 0; c < total; ++c) {
    const int k = static_cast<int>(c % NCH);
    if (k == 0) {
      const int64_t tile = blockIdx.x + (c / NCH) * gridDim.x;
      row0 = tile * C::TILE + 32 * w;
      active = row0 < R_pad;
      if (active) {
#pragma unroll
        for (int rb = 0; rb < 2; ++rb) {
          const int64_t row = row0 + 8 * (r >> 2) + 4 * rb + (r & 3);
          float v[8 * KB];
          if (row < R) {
            const bf16_t* xr = row_in<bf16_t>(X, row) + 8 * g;
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) {
              const bf16x8 x = ld16(xr + kb * 32);
#pragma unroll
              for (int j = 0; j < 8; ++j) v[8 * kb + j] = static_cast<float>(x[j]);
            }
          } else {
#pragma unroll
            for (int i = 0; i < 8 * KB; ++i) v[i] = 0.f;
          }
          ln_rows<8 * KB>(v, D);
#pragma unroll
          for (int kb = 0; kb < KB; ++kb) hb[rb][kb] = pack8(v + 8 * kb);
        }
      }
    }
    const bool more = c + 1 < total;
    if (more) issue_chunk(static_cast<int>((c + 1) % NCH), buf0 + ((c + 1) & 1) * (CR * D));
    const bf16_t* wb = buf0 + (c & 1) * (CR * D) + opaque_zero();
    // Q columns only for rows below q_rows (a multiple of 32)
    const bool work = active && (CR * k >= D || row0 < q_rows);
    if (work) {
      if (k < NQK) {
        // output columns [64k, 64k + 64) of Q|K: two 32-column pairs
#pragma unroll
        for (int pp = 0; pp < 2; ++pp) {
          floatx4 acc[2][2] = {};
#pragma unroll
          for (int cc = 0; cc < 2; ++cc) {
            const int wrow = 32 * pp + 8 * (r >> 2) + 4 * cc + (r & 3);
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) {
              const bf16x8 a = frag(wb, wrow, kb);
              acc[cc][0] = mma(a, hb[0][kb], acc[cc][0]);
              acc[cc][1] = mma(a, hb[1][kb], acc[cc][1]);
            }
          }
          const float f = CR * k < D ? qs : 1.f;  // Q columns carry the logit scale
#pragma unroll
          for (int rb = 0; rb < 2; ++rb) {
            const int64_t row = row0 + 8 * (r >> 2) + 4 * rb + (r & 3);
            const float v[8] = {acc[0][rb][0] * f, acc[0][rb][1] * f, acc[0][rb][2] * f, acc[0][rb][3] * f,
                                acc[1][rb][0] * f, acc[1][rb][1] * f, acc[1][rb][2] * f, acc[1][rb][3] * f};
            st8h(QK + ((CR * k) / 32 + pp) * (R_pad * 32) + row * 32 + 8 * g, v);  // head-planar
          }
        }
      } else {
        // V columns [64(k-NQK), +64): four 16-column blocks, operands swapped
#pragma unroll
        for (int nn = 0; nn < 4; ++nn) {
          floatx4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int kb = 0; kb < KB; ++kb) {
            const bf16x8 b = frag(wb, 16 * nn + r, kb);
            acc0 = mma(hb[0][kb], b, acc0);
            acc1 = mma(hb[1][kb], b, acc1);
          }
          const float v[8] = {acc0[0], acc0[1], acc0[2], acc0[3], acc1[0], acc1[1], acc1[2], acc1[3]};
          st8h(Vp + vp_index(row0 + 8 * g, CR * (k - NQK) + 16 * nn + r, D), v);
        }
      }
    }
    // the next chunk's loads must have landed; after them this wave issued
    // its 4 output stores of this chunk (if it had work), which may still
    // be in flight
    if (work) wait_vm<4>();
    else wait_vm<0>();
    dma_barrier();
  }
}

// The 32 products of one chunk and wave as 4 groups of 8 (fragment read
// from LDS, product): group g + 1's 8 reads are issued after group g's
// first two products, so a wave keeps 6 to 14 reads in flight while its
// products run instead of waiting one LDS round trip per product.  The
// products of a group alternate between two accumulators.
template <typename FragOf, typename Mul>
__device__ __forceinline__ void chunk_products(FragOf&& frag_of, Mul&& mul) {
  bf16x8 buf[2][8];
#pragma unroll
  for (int j = 0; j < 8; ++j) buf[0][j] = frag_of(0, j);
#pragma unroll
  for (int grp = 0; grp < 4; ++grp) {
    __builtin_amdgcn_sched_barrier(0);
    mul(grp, 0, buf[grp & 1][0]);
    mul(grp, 1, buf[grp & 1][1]);
    __builtin_amdgcn_sched_barrier(0);
    if (grp < 3) {
#pragma unroll
      for (int j = 0; j < 8; ++j) buf[(grp + 1) & 1][j] = frag_of(grp + 1, j);
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int j = 2; j < 8; ++j) mul(grp, j, buf[grp & 1][j]);
  }
  __builtin_amdgcn_sched_barrier(0);
}

// Post-attention block, weights streamed: 16 chunks of 64 weight rows per
// step: 0..3 w_o (two column pairs each), 4..11 gate/up (32 rows of each:
// one pair), 12..15 w_down (two pairs each).  One wave of eight owns a
// 16-row block per step, so each chunk in LDS feeds up to 128 rows.  Each
// workgroup takes an equal contiguous range of 16-row blocks (rounded), 8
// per step: its last step may hold fewer blocks, and the waves without one
// only stream and wait.  (Whole 128-row tiles dealt round-robin left, at
// 3.1 rounds, a fourth round of full tiles on a tenth of the CUs.)  Chunks travel global ->
// LDS directly (LDS-DMA buffer loads, 16 bytes per lane), so no registers
// carry them; three chunk buffers keep two chunks in flight while one is
// computed, and the next tile's Y and X rows are fetched during the w_down
// chunks.  LDS rows are unpadded (D bf16) with their 16-byte slots
// XOR-swizzled by swz(row): the 8 rows one fragment read touches per lane
// group land in distinct banks.
template <int D>
struct PostStreamCfg {
  static constexpr int NW = 8, NT = 64 * NW, CR = 64, NBUF = 3;
  static constexpr int SPR = D / 8;                  // 16-byte slots per row
  static constexpr int CPT = CR * SPR / NT;          // slots per thread per chunk
  static constexpr size_t lds_bytes = static_cast<size_t>(NBUF) * CR * D * 2;
};

__device__ __forceinline__ int swz(int row) { return (row & 3) | (((row >> 3) & 3) << 2); }

// Hout (Hout.a non-null): also LayerNorm(output row) as bf16, the next
// layer's attention operands.
template <int D>
__global__ __launch_bounds__(512) void post_block_stream(const bf16_t* __restrict__ Y, int64_t yR,
                                                         Rows Xres, Rows Out, int64_t nrows,
                                                         const bf16_t* __restrict__ Wo,
                                                         const bf16_t* __restrict__ Wg,
                                                         const bf16_t* __restrict__ Wu,
                                                         const bf16_t* __restrict__ Wd, Rows Hout) {
  using C = PostStreamCfg<D>;
  constexpr int KB = D / 32, NW = C::NW, CR = C::CR, NCH = 16, SPR = C::SPR, CPT = C::CPT;
  static_assert(D == 256, "chunk schedule is written for d = 256");
  static_assert(C::NT / SPR == 16 && CPT == 4, "load pattern assumes 16 rows per step");
  extern __shared__ __attribute__((aligned(16))) char smem[];
  bf16_t* const buf0 = reinterpret_cast<bf16_t*>(smem);
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int g = lane >> 4, r = lane & 15;
  // this workgroup's 16-row blocks [blk0, blk1), NW per step (block
  // indices fit 32 bits: the host caps nrows below 2^35)
  const int nblk = static_cast<int>((nrows + 15) / 16);
  const int blk0 = static_cast<int>(static_cast<int64_t>(blockIdx.x) * nblk / gridDim.x);
  const int blk1 = static_cast<int>((static_cast<int64_t>(blockIdx.x) + 1) * nblk / gridDim.x);
  const int my_tiles = (blk1 - blk0 + NW - 1) / NW;
  if (my_tiles <= 0) return;

  // Chunk step i of a chunk (CPT steps, 16 weight rows each): row 16 i +
  // tid / 32, swizzled slot tid % 32, fetched by this thread with one
  // LDS-DMA load; a wave's 64 lanes fill 1 KB of LDS in a row.  Each weight
  // matrix is one buffer descriptor, so a load is a scalar row offset (a
  // constant of the unrolled schedule) plus this lane's offset for the step
  // into a descriptor: no per-load vector address arithmetic.
  const __amdgpu_buffer_rsrc_t rs_o = weight_rsrc(Wo, D * D), rs_g = weight_rsrc(Wg, D * D),
                               rs_u = weight_rsrc(Wu, D * D), rs_d = weight_rsrc(Wd, D * D);
  const int lrow = tid >> 5;  // row within a 16-row step
  const int wu = __builtin_amdgcn_readfirstlane(w);  // wave-uniform LDS segment
  auto issue_chunk = [&](int k, bf16_t* buf) {
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      // this lane's byte offset within the step (the same for every chunk)
      const unsigned vo = static_cast<unsigned>((lrow * D + 8 * ((tid & 31) ^ swz(16 * i + lrow))) * 2);
      lds_void_t* dst = (lds_void_t*)(buf + (i * C::NT + wu * 64) * 8);
      // the first weight row of this step in its matrix, as a byte offset
      if (k < 4)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs_o, dst, 16, vo, (64 * k + 16 * i) * D * 2, 0, 0);
      else if (k < 12 && i < 2)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs_g, dst, 16, vo, (32 * (k - 4) + 16 * i) * D * 2, 0, 0);
      else if (k < 12)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs_u, dst, 16, vo, (32 * (k - 4) + 16 * (i - 2)) * D * 2, 0, 0);
      else
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs_d, dst, 16, vo, (64 * (k - 12) + 16 * i) * D * 2, 0, 0);
    }
  };
  // the A fragment of weight row `row`, k-slice kb, of a chunk buffer; every
  // row this kernel reads as lane (r, g) has swz(row) = r
  auto frag = [&](const bf16_t* wb, int row, int kb) {
    return ld16(wb + row * D + 8 * ((4 * kb + g) ^ r));
  };
  // the Y rows of step `it` (fetched during the previous step's last
  // chunks) and its X rows (fetched at the step's start, first used when
  // the w_o product is complete); rows past the end, or of a wave without
  // a block, read row 0, unused (every wave issues the same loads: the
  // counted waits below rely on it)
  auto tile_row = [&](int it) {
    const int blk = blk0 + it * NW + w;
    const int64_t row = static_cast<int64_t>(blk) * 16 + r;
    return blk < blk1 && row < nrows ? row : int64_t(0);
  };
  bf16x8 yn[KB];
  auto load_y = [&](int it) {
    const bf16_t* yr = Y + tile_row(it) * 32 + 8 * g;  // head-planar: head kb at kb * yR * 32
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) yn[kb] = ld16(yr + kb * yR * 32);
  };

  // chunk c of the whole sequence (tile c / 16, schedule step c % 16) sits
  // in buffer c % 3; chunks c + 1 and c + 2 are in flight while c is used.
  // The waits count this wave's vector memory operations, which complete in
  // issue order: after chunk c + 1's loads come chunk c + 2's (CPT) and,
  // where noted, row loads (KB each) and the previous tile's stores.
  load_y(0);
  issue_chunk(0, buf0);
  issue_chunk(1, buf0 + CR * D);
  wait_vm<CPT>();  // Y and chunk 0 have landed
  dma_barrier();
  int t3 = 0;  // (tile index) % 3: chunk k of this tile is in buffer (t3 + k) % 3
  for (int it = 0; it < my_tiles; ++it) {
    const int blk = blk0 + it * NW + w;
    const bool active = blk < blk1;  // wave-uniform
    const int64_t row = static_cast<int64_t>(blk) * 16 + r;
    const bool rowok = active && row < nrows;
    const bool next = it + 1 < my_tiles;
    bf16x8 yb[1][KB], xr[KB];
    {
      const bf16_t* xp = row_in<bf16_t>(Xres, tile_row(it)) + 8 * g;
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        yb[0][kb] = yn[kb];
        xr[kb] = ld16(xp + kb * 32);
      }
    }
    float x1[1][D / 4];
#pragma unroll
    for (int i = 0; i < D / 4; ++i) x1[0][i] = 0.f;
    bf16x8 gb[KB], mb[KB];
#pragma unroll
    for (int k = 0; k < NCH; ++k) {
      // chunk k + 2 (of this tile or the next) goes to the buffer chunk
      // k - 1 used, which every wave has left (the barrier ending step k - 1)
      const bool more2 = (k + 2 < NCH) || next;
      if (more2) issue_chunk((k + 2) % NCH, buf0 + ((t3 + k + 2) % 3) * (CR * D));
      const bf16_t* wb = buf0 + ((t3 + k) % 3) * (CR * D) + opaque_zero();
      if (!active) {
        // no block this step: stream and wait only
      } else if (k < 4 || k >= 12) {
        // x1 += (Y or M) W^T for column pairs 2k', 2k'+1.  Group (pp, kh):
        // k-slices 4 kh .. +4 of both column halves cc, alternating
        const int kk = k < 4 ? k : k - 12;
        floatx4 acc[2][2] = {};
        chunk_products(
            [&](int grp, int j) {
              return frag(wb, 32 * (grp >> 1) + 8 * (r >> 2) + 4 * (j & 1) + (r & 3), 4 * (grp & 1) + (j >> 1));
            },
            [&](int grp, int j, const bf16x8& f) {
              const int kb = 4 * (grp & 1) + (j >> 1);
              acc[grp >> 1][j & 1] = mma(f, k < 4 ? yb[0][kb] : mb[kb], acc[grp >> 1][j & 1]);
            });
#pragma unroll
        for (int pp = 0; pp < 2; ++pp) {
          const int p = 2 * kk + pp;
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            x1[0][8 * p + q] += acc[pp][0][q];
            x1[0][8 * p + 4 + q] += acc[pp][1][q];
          }
        }
        if (k == 3) {
          // the residual: x1 = X + Y W_o^T (one addition per element, the
          // same sum as starting from X)
#pragma unroll
          for (int kb = 0; kb < KB; ++kb)
#pragma unroll
            for (int q = 0; q < 8; ++q) x1[0][8 * kb + q] += static_cast<float>(xr[kb][q]);
          float t[8 * KB];
#pragma unroll
          for (int i = 0; i < 8 * KB; ++i) t[i] = x1[0][i];
          ln_rows<8 * KB>(t, D);
#pragma unroll
          for (int kb = 0; kb < KB; ++kb) gb[kb] = pack8(t + 8 * kb);
        }
      } else {
        // gate/up column pair q2 = k - 4: rows [0,32) gate, [32,64) up.
        // Group (cc, kh): k-slices 4 kh .. +4 of gate and up, alternating
        floatx4 ag[2] = {}, au[2] = {};
        chunk_products(
            [&](int grp, int j) {
              return frag(wb, 32 * (j & 1) + 8 * (r >> 2) + 4 * (grp >> 1) + (r & 3), 4 * (grp & 1) + (j >> 1));
            },
            [&](int grp, int j, const bf16x8& f) {
              const int kb = 4 * (grp & 1) + (j >> 1);
              if (j & 1)
                au[grp >> 1] = mma(f, gb[kb], au[grp >> 1]);
              else
                ag[grp >> 1] = mma(f, gb[kb], ag[grp >> 1]);
            });
        float v[8];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          v[q] = silu_f(ag[0][q]) * au[0][q];
          v[4 + q] = silu_f(ag[1][q]) * au[1][q];
        }
        mb[k - 4] = pack8(v);
      }
      // chunk k + 1 must have landed before the barrier:
      //   step 0: after it come the previous tile's stores (if any), this
      //           tile's X rows (KB) and chunk k + 2 (CPT);
      //   step 13: after it come the next tile's Y rows (KB, loaded after
      //           step 12's wait) and chunk k + 2;
      //   otherwise only chunk k + 2, or nothing once no chunk follows.
      if (!more2) wait_vm<0>();
      else if (k == 0 || (k == 13 && next)) wait_vm<CPT + KB>();
      else wait_vm<CPT>();
      if (k == 12 && next) load_y(it + 1);
      dma_barrier();
    }
    if (rowok) {
      bf16_t* orow = row_out<bf16_t>(Out, row);
      if (orow != nullptr)
#pragma unroll
        for (int p = 0; p < KB; ++p) st8(orow + 32 * p + 8 * g, &x1[0][8 * p]);
    }
    if (Hout.a != nullptr && active) {
      // (all lanes of the wave: the LN reduces over the lanes of each row)
      ln_rows<8 * KB>(x1[0], D);
      if (rowok) {
        bf16_t* hrow = row_out<bf16_t>(Hout, row);
#pragma unroll
        for (int p = 0; p < KB; ++p) st8(hrow + 32 * p + 8 * g, &x1[0][8 * p]);
      }
    }
    t3 = (t3 + 16) % 3;
  }
}

// ===========================================================================
// User-resident kernel: one workgroup (8 waves) per user, all layers in one
// launch, for users whose ell + N_b rows fit in LDS.  Local rows: [0, ell)
// links, [ell, ell + N_b) history, zero rows up to RT (multiple of 32).
//   Xs  [RT][D + 4] float32  residual stream (padded rows)
//   QKs [RT][2D + 8] bf16 (Q | K) ;  Vps [RT/8][D][8] bf16 ;  Ys [RT][D + 8] bf16
//   (D <= 64) one layer's weights, rows padded by 16 bytes:
//   Wq [3D][D+8] (w_qkv) ; Wp [4D][D+8] (w_o, w_gate, w_up, w_down)
// Phases, separated by barriers: layer 0's LN + QKV (items: 32-row chunk x
// {Q|K, V}); then per layer the attention (items: per head the L-branch and
// each 32-row E-branch chunk) and the post-attention block (items: 16-row
// blocks), each block followed in registers by the next layer's LN + QKV
// of the same rows.  The next layer's weights are loaded into registers
// while the current layer runs and written to LDS once their region is free.
// ===========================================================================
constexpr int RES_MAX_LAYERS = 16;
// per-layer weight pointers passed by value: w_qkv, w_o, w_gate, w_up, w_down
struct LayerSet {
  const bf16_t* p[RES_MAX_LAYERS][5];
};

// Candidate scoring inside the user-resident kernel (its SC form; LIME
// notes, "complete example", step 3: the cached weights of a candidate,
// looked up by id, weight the user's personalised links): the same
// operands and products as cand_score, for the candidates of the
// workgroup's own user.
struct ScoreArgs {
  const bf16_t* cache = nullptr;  // [n_items, H, ELL]
  int64_t n_items = 0;
  const int64_t* ids = nullptr;   // [total_M]
  const int64_t* coff = nullptr;  // [B + 1]
  int64_t total_M = 0;
  bf16_t* out = nullptr;          // [total_M, D]
  int* bad = nullptr;
};

// 8 consecutive floats of an LDS row as two 16-byte accesses (the row
// strides keep every such piece 16-byte aligned)
__device__ __forceinline__ void lds_ld8f(const float* p, float* v) {
  const float4 a = *reinterpret_cast<const float4*>(p);
  const float4 b = *reinterpret_cast<const float4*>(p + 4);
  v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
  v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}

__device__ __forceinline__ void lds_st8f(float* p, const float* v) {
  *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
  *reinterpret_cast<float4*>(p + 4) = make_float4(v[4], v[5], v[6], v[7]);
}

template <int ELL, int D>
struct ResCfg {
  static constexpr int NW = 8;
  static constexpr int NT = 64 * NW;
  static constexpr int XS = D + 4;  // float32 row stride of the residual stream
  // bf16 row strides of QK and Y padded by 16 bytes
  static constexpr int LQK = 2 * D + 8, LY = D + 8;
  static constexpr size_t bytes_per_row = static_cast<size_t>(XS) * 4 + LQK * 2 + D * 2 + LY * 2;
  static constexpr bool WL = D <= 64;  // weights staged in LDS
  static constexpr int PRB = 1;        // 16-row blocks per post-phase item
  static constexpr int LDW = D + 8;
  static constexpr int QCH = 3 * D * (D / 8);  // 16-byte chunks of w_qkv
  static constexpr int PCH = 4 * D * (D / 8);  // 16-byte chunks of the post weights
  static constexpr int QPT = (QCH + NT - 1) / NT, PPT = (PCH + NT - 1) / NT;
  static constexpr size_t w_elems = static_cast<size_t>(7) * D * LDW;
  static constexpr size_t lds_bytes(int RT) {
    return bytes_per_row * RT + (WL ? w_elems * 2 : 0);
  }
};

// chunk e of a weight set -> (source pointer, LDS row) ; set 0 = w_qkv,
// set 1 = w_o, w_gate, w_up, w_down stacked.  A thread's i-th chunk lies in
// one matrix for all threads (the chunks per matrix are a multiple of the
// threads), so the matrix index is a constant and its pointer is read once
// per wave, not per lane.
template <int D, int NT>
__device__ __forceinline__ const bf16_t* wsrc(const LayerSet& w, int l, int set, int i, int e, int* row_out) {
  constexpr int CPM = D * (D / 8);  // 16-byte chunks per matrix
  static_assert(CPM % NT == 0, "weight chunks per matrix");
  const int row = e / (D / 8), c8 = e % (D / 8);
  *row_out = row;
  if (set == 0) return w.p[l][0] + static_cast<int64_t>(row) * D + 8 * c8;
  const int m = (i * NT) / CPM;  // 0..3: w_o, w_gate, w_up, w_down
  return w.p[l][1 + m] + static_cast<int64_t>(row - m * D) * D + 8 * c8;
}

template <int ELL, int D, int NKW = 0, bool SC = false>
__global__ __launch_bounds__(512) void xor_fwd_resident(
    const bf16_t* __restrict__ links_ctx, const bf16_t* __restrict__ hist,
    const int64_t* __restrict__ off, int64_t total_N, int RT, int layers, LayerSet w, float scale, int phi,
    bf16_t* __restrict__ links_pers, bf16_t* __restrict__ hist_out, int links_only, int half, ScoreArgs sa) {
  using C = ResCfg<ELL, D>;
  constexpr int H = D / 32, KB = D / 32, XS = C::XS, NW = C::NW, NT = C::NT;
  constexpr bool WL = C::WL;
  constexpr int LDW = C::LDW;
  extern __shared__ __attribute__((aligned(16))) char smem[];
  float* Xs = reinterpret_cast<float*>(smem);
  constexpr int LQK = C::LQK, LY = C::LY;
  bf16_t* QKs = reinterpret_cast<bf16_t*>(smem + static_cast<size_t>(RT) * XS * 4);
  bf16_t* Vps = QKs + static_cast<size_t>(RT) * LQK;
  bf16_t* Ys = Vps + static_cast<size_t>(RT) * D;
  bf16_t* Wq = Ys + static_cast<size_t>(RT) * LY;  // [3D][LDW]
  bf16_t* Wp = Wq + 3 * D * LDW;                  // [4D][LDW]

  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int g = lane >> 4, r = lane & 15;
  const int b = blockIdx.x;
  const int64_t u0 = clamp64(off[b], 0, total_N);
  int64_t u1 = clamp64(off[b + 1], u0, total_N);
  if (u1 - u0 > RT - ELL) u1 = u0 + (RT - ELL);  // never beyond the planned rows
  const int n = static_cast<int>(u1 - u0);
  const int rows = ELL + n;
  const bool softmax = (phi == PHI_SOFTMAX);
  const float qs = scale * LOG2E;  // Q carries the logit scale in log2 units
  const Lay qkl{LQK, 32}, yl{LY, 32};   // row-major LDS rows
  const int nchunks = RT / 32;

  // weight prefetch registers: set 0 (w_qkv) and set 1 (post weights)
  bf16x8 pq[C::QPT], pp[C::PPT];
  auto load_set = [&](int l, int set) {
    if constexpr (WL) {
      const int cnt = set == 0 ? C::QCH : C::PCH;
#pragma unroll
      for (int i = 0; i < (set == 0 ? C::QPT : C::PPT); ++i) {
        const int e = tid + i * NT;
        int row;
        if (e < cnt) {
          const bf16x8 v = ld16(wsrc<D, NT>(w, l, set, i, e, &row));
          if (set == 0) pq[i] = v; else pp[i] = v;
        }
      }
    }
  };
  auto store_set = [&](int set) {
    if constexpr (WL) {
      const int cnt = set == 0 ? C::QCH : C::PCH;
      bf16_t* dst = set == 0 ? Wq : Wp;
#pragma unroll
      for (int i = 0; i < (set == 0 ? C::QPT : C::PPT); ++i) {
        const int e = tid + i * NT;
        if (e < cnt) {
          const int row = e / (D / 8), c8 = e % (D / 8);
          *reinterpret_cast<bf16x8*>(dst + row * LDW + 8 * c8) = set == 0 ? pq[i] : pp[i];
        }
      }
    }
  };

  // residual stream <- [L^C_b ; E_b], zero padding.  Every load is issued
  // (padding rows read the user's first link row, then zeroed), the first
  // batch before the weight loads, so converting it waits on it alone.
  constexpr int XU = 4;  // chunks per thread and batch
  auto x_load = [&](int e0, bf16x8 (&xv)[XU]) {
#pragma unroll
    for (int u = 0; u < XU; ++u) {
      const int e = e0 + u * NT, row = e / (D / 8), c8 = e % (D / 8);
      const bool link = row < ELL, hrow = !link && row < rows;
      const bf16_t* src = hrow ? hist + (u0 + row - ELL) * D + 8 * c8
                               : links_ctx + (static_cast<int64_t>(b) * ELL + (link ? row : 0)) * D + 8 * c8;
      xv[u] = ld16(src);
    }
  };
  // Each row's D/8 chunks sit in D/8 consecutive lanes, so the store also
  // takes the row's LN (layer 0's pre-attention LN) and writes it as bf16
  // into the Y rows, which hold nothing before the first attention.
  auto x_store = [&](int e0, const bf16x8 (&xv)[XU]) {
#pragma unroll
    for (int u = 0; u < XU; ++u) {
      const int e = e0 + u * NT, row = e / (D / 8), c8 = e % (D / 8);
      const bool real = row < rows;
      float v[8];
#pragma unroll
      for (int q = 0; q < 8; ++q) v[q] = real ? static_cast<float>(xv[u][q]) : 0.f;
      const float mu = span_sum<D / 8>(tree_sum<8>(v)) * (1.f / static_cast<float>(D));
      float t[8];
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const float dv = v[q] - mu;
        t[q] = dv * dv;
      }
      const float rs = rsqrtf(span_sum<D / 8>(tree_sum<8>(t)) * (1.f / static_cast<float>(D)) + 1e-5f);
      if (row < RT) {
        lds_st8f(Xs + row * XS + 8 * c8, v);
#pragma unroll
        for (int q = 0; q < 8; ++q) t[q] = (v[q] - mu) * rs;
        *reinterpret_cast<bf16x8*>(Ys + row * LY + 8 * c8) = pack8(t);
      }
    }
  };
  {
    bf16x8 xv[XU];
    x_load(tid, xv);
    load_set(0, 0);
    load_set(0, 1);
    x_store(tid, xv);
    for (int e0 = tid + XU * NT; e0 < RT * (D / 8); e0 += XU * NT) {
      x_load(e0, xv);
      x_store(e0, xv);
    }
  }
  store_set(0);
  store_set(1);
  lds_barrier();

  const int ldd = WL ? LDW : D;
  // ---- layer 0: LN + QKV over chunk items (chunk, part); later layers get
  // their projection from the previous layer's post phase
  {
    if (layers > 1) load_set(1, 0);
    const bf16_t* lq = WL ? Wq : w.p[0][0];
    for (int it = wv; it < 2 * nchunks; it += NW) {
      const int row0 = (it >> 1) * 32;
      // the LN rows the staging wrote into Y
      bf16x8 hb[2][KB];
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) {
        const int row = row0 + 8 * (r >> 2) + 4 * rb + (r & 3);
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
          hb[rb][kb] = *reinterpret_cast<const bf16x8*>(Ys + row * LY + kb * 32 + 8 * g);
      }
      if (it & 1) v_part<D>(hb, lq + opaque_zero(), ldd, Vps, row0, r, g);
      else qk_part<D>(hb, lq + opaque_zero(), ldd, QKs, row0, r, g, qs, qkl);
    }
    lds_barrier();
  }

  // scoring form: this user's candidate range; waves idle in the last post
  // phase take the first tiles and gather them during that phase (PF)
  constexpr int KBL = ELL / 32;
  constexpr bool PF = SC && D <= 64;
  int64_t m0 = 0, m1 = 0, ntile = 0;
  int sw = wv;  // this wave's first scoring tile
  bf16x8 bw_pf[H][KBL];
  int64_t i_pf = 0;
  bool ok_pf = false, have_pf = false;
  if constexpr (SC) {
    m0 = clamp64(sa.coff[b], 0, sa.total_M);
    m1 = clamp64(sa.coff[b + 1], m0, sa.total_M);
    ntile = (m1 - m0 + 15) >> 4;
    const bool full_last = !links_only && hist_out != nullptr;
    const int pl = ((full_last ? rows : ELL) + 15) / 16;  // items of the last post phase
    sw = (wv + NW - pl % NW) % NW;
  }
  auto gather_tile = [&](int64_t t, int64_t& i, bool& okid, bf16x8 (&bw)[H][KBL]) {
    i = m0 + 16 * t + r;
    const bool valid = i < m1;
    const int64_t id = valid ? sa.ids[i] : int64_t(-1);
    okid = id >= 0 && id < sa.n_items;
    if (valid && !okid && g == 0 && sa.bad != nullptr) atomicAdd(sa.bad, 1);
    const int64_t idc = okid ? id : 0;
#pragma unroll
    for (int hh = 0; hh < H; ++hh)
#pragma unroll
      for (int kb = 0; kb < KBL; ++kb)
        bw[hh][kb] = okid ? ld16(sa.cache + (idc * H + hh) * ELL + 8 * g + kb * 32) : zero8();
  };

  for (int l = 0; l < layers; ++l) {
    const bool last = (l == layers - 1);
    // history rows get attention and the post block unless nothing can
    // read them (links-only variant; last layer without hist_out)
    const bool full = !links_only && (!last || hist_out != nullptr);
    // ---- attention: items = per head, the L-branch and the E-branch chunks.
    // The weight regions are free here: stage layer l's post weights (from
    // layer 1 on) and layer l+1's projection weights.
    if (l > 0) store_set(1);
    if (!last) store_set(0);
    const int echunks = full ? (n + 31) / 32 : 0;
    const int items = H * (1 + echunks);
    for (int it = wv; it < items; it += NW) {
      const int h = it % H, k = it / H;
      HeadOps<ELL> o;
      load_head_ops<ELL, D>(o, QKs, Vps, 0, h, r, g, qkl);
      if (k == 0) {
        LState<ELL> st;
        st.init();
        with_phi(softmax, [&](auto phi_tag) {
          for (int c0 = 0; c0 < n; c0 += 32) {
            ChunkOps ci;
            load_chunk<D>(ci, QKs, Vps, ELL, c0, h, false, r, g, qkl);
            l_branch<ELL, decltype(phi_tag)::value>(st, o, ci, c0, 0, n, r, g);
          }
        });
        // normalise and write the link rows of Y
#pragma unroll
        for (int nb = 0; nb < HeadOps<ELL>::MB; ++nb) {
          const float den = softmax ? st.l[nb] : static_cast<float>(n);
          const float inv = den > 0.f ? (softmax ? 1.f : LN2) / den : 0.f;
          bf16_t* yr = Ys + (16 * nb + r) * LY + h * 32 + 4 * g;
#pragma unroll
          for (int c2 = 0; c2 < 2; ++c2)
#pragma unroll
            for (int q = 0; q < 4; ++q) yr[16 * c2 + q] = f32_to_bf16(st.acc[nb][c2][q] * inv);
        }
      } else {
        ChunkOps ci;
        load_chunk<D>(ci, QKs, Vps, ELL, 32 * (k - 1), h, true, r, g, qkl);
        with_phi(softmax, [&](auto phi_tag) {
          constexpr bool SM = decltype(phi_tag)::value;
          if constexpr (NKW > 0) {
            WinOps<NKW> wo;
            load_window<NKW, D>(wo, QKs, Vps, ELL, win_key0(32 * (k - 1), half), RT, h, r, g, qkl);
            const WinArgs wa{0, n, RT, half, Vps, ELL};
            e_branch<ELL, D, SM, NKW>(o, ci, Ys, ELL, 32 * (k - 1), 0, n, h, r, g, yl, &wo, &wa);
          } else {
            e_branch<ELL, D, SM>(o, ci, Ys, ELL, 32 * (k - 1), 0, n, h, r, g, yl);
          }
        });
      }
    }
    lds_barrier();
    // ---- post-attention block per 16-row block, and in every layer but the
    // last the next layer's LN + QKV of the same rows, straight from the
    // registers (rows the post block skips are re-projected as they are)
    if (!last) {
      load_set(l + 1, 1);
      if (l + 2 < layers) load_set(l + 2, 0);
    }
    const bf16_t* lo_w = WL ? Wp : w.p[l][1];
    const bf16_t* lg_w = WL ? Wp + D * LDW : w.p[l][2];
    const bf16_t* lu_w = WL ? Wp + 2 * D * LDW : w.p[l][3];
    const bf16_t* ld_w = WL ? Wp + 3 * D * LDW : w.p[l][4];
    const bf16_t* lq_next = last ? nullptr : (WL ? Wq : w.p[l + 1][0]);
    constexpr int PRB = ResCfg<ELL, D>::PRB;  // 16-row blocks per post item
    constexpr int PR = 16 * PRB;
    const int prow_end = full ? rows : ELL;  // a multiple of PR when not every row
    const int pitems = ((last ? prow_end : rows) + PR - 1) / PR;
    if constexpr (PF) {
      if (last && wv >= pitems && sw < ntile) {
        gather_tile(sw, i_pf, ok_pf, bw_pf);
        have_pf = true;
      }
    }
    for (int it = wv; it < pitems; it += NW) {
      const int row0 = it * PR;
      const bool do_post = row0 < prow_end;
      float x1[PRB][D / 4];
#pragma unroll
      for (int rb = 0; rb < PRB; ++rb)
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
          lds_ld8f(Xs + (row0 + 16 * rb + r) * XS + kb * 32 + 8 * g, &x1[rb][8 * kb]);
      if (do_post) {
        bf16x8 yb[PRB][KB];
#pragma unroll
        for (int rb = 0; rb < PRB; ++rb) {
          const int row = row0 + 16 * rb + r;
#pragma unroll
          for (int kb = 0; kb < KB; ++kb) yb[rb][kb] = row < rows ? ld16(Ys + row * LY + kb * 32 + 8 * g) : zero8();
        }
        const int z = opaque_zero();
        post_rows<D, D, PRB, false, false>(yb, x1, lo_w + z, lg_w + z, lu_w + z, ld_w + z, ldd, ldd, r, g);
#pragma unroll
        for (int rb = 0; rb < PRB; ++rb) {
          const bool real = row0 + 16 * rb + r < rows;
#pragma unroll
          for (int i = 0; i < D / 4; ++i) x1[rb][i] = real ? x1[rb][i] : 0.f;
        }
      }
      if (!last) {
        if (do_post) {
#pragma unroll
          for (int rb = 0; rb < PRB; ++rb)
#pragma unroll
            for (int kb = 0; kb < KB; ++kb)
              lds_st8f(Xs + (row0 + 16 * rb + r) * XS + kb * 32 + 8 * g, &x1[rb][8 * kb]);
        }
        // history rows need Q next layer only for their own attention
        const bool next_full = !links_only && (l + 2 < layers || hist_out != nullptr);
        qkv_rows<D, PRB>(x1, lq_next + opaque_zero(), ldd, QKs, Vps, row0, r, g, qkl, qs, row0 < ELL || next_full);
      } else if (do_post) {
#pragma unroll
        for (int rb = 0; rb < PRB; ++rb) {
          const int row = row0 + 16 * rb + r;
          if (row < rows) {
            bf16_t* dst = row < ELL ? links_pers + (static_cast<int64_t>(b) * ELL + row) * D
                                    : (hist_out ? hist_out + (u0 + row - ELL) * D : nullptr);
            if (dst)
#pragma unroll
              for (int kb = 0; kb < KB; ++kb) st8(dst + kb * 32 + 8 * g, &x1[rb][8 * kb]);
            // scoring reads the user's L^P from the Y rows (this item has
            // already read its own)
            if (SC && row < ELL)
#pragma unroll
              for (int kb = 0; kb < KB; ++kb) st8(Ys + row * LY + kb * 32 + 8 * g, &x1[rb][8 * kb]);
          }
        }
      }
    }
    lds_barrier();
  }

  // ---- candidate scoring of this user's candidates: 16-candidate tiles
  // round-robin over the waves; per head O^T = L^P_h^T (cache rows)^T, the
  // operand layout, products and output rounding of cand_score
  if constexpr (SC) {
    if (sw < ntile) {
      bf16x8 a[H][2][KBL];
#pragma unroll
      for (int hh = 0; hh < H; ++hh)
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          const int col = hh * 32 + 8 * (r >> 2) + 4 * c + (r & 3);
#pragma unroll
          for (int kb = 0; kb < KBL; ++kb)
#pragma unroll
            for (int j = 0; j < 8; ++j) a[hh][c][kb][j] = __builtin_bit_cast(__bf16, Ys[(kb * 32 + 8 * g + j) * LY + col]);
        }
      for (int64_t t = sw; t < ntile; t += NW) {
        int64_t i;
        bool okid;
        bf16x8 bw[H][KBL];
        if (PF && have_pf && t == sw) {
          i = i_pf;
          okid = ok_pf;
#pragma unroll
          for (int hh = 0; hh < H; ++hh)
#pragma unroll
            for (int kb = 0; kb < KBL; ++kb) bw[hh][kb] = bw_pf[hh][kb];
        } else {
          gather_tile(t, i, okid, bw);
        }
        const bool valid = i < m1;
#pragma unroll
        for (int hh = 0; hh < H; ++hh) {
          floatx4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int kb = 0; kb < KBL; ++kb) {
            acc0 = mma(a[hh][0][kb], bw[hh][kb], acc0);
            acc1 = mma(a[hh][1][kb], bw[hh][kb], acc1);
          }
          if (valid) {
            const float v[8] = {acc0[0], acc0[1], acc0[2], acc0[3], acc1[0], acc1[1], acc1[2], acc1[3]};
            st8_stream(sa.out + i * D + hh * 32 + 8 * g, v);
          }
        }
      }
    }
  }
}

}  // namespace mfma
}  // namespace lime
