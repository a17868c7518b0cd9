// Matrix-core (MFMA, gfx950) kernels of the hot path, bf16 in / fp32 accumulate.
//
// All contractions use v_mfma_f32_16x16x32_bf16 in the "transposed" form
// D[m][n] = sum_k A[m][k] B[k][n] with lane l holding
//   A: row m = l%16, k = 8*(l/16) .. +7        (16 contiguous bytes)
//   B: col n = l%16, k = 8*(l/16) .. +7        (16 contiguous bytes)
//   D: col n = l%16, rows 4*(l/16) .. +3
// The order of k inside a lane is the same for A and B, so the contraction
// does not depend on it.  Which output column a D row stands for is free:
// the kernels map rows so that every lane ends with 8 consecutive outputs
// of one item / candidate and stores them as one 16-byte vector.
#pragma once

#include "common.h"

namespace lime {
namespace mfma {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ floatx4 mma(const bf16x8& a, const bf16x8& b, const floatx4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 ld16(const bf16_t* p) {
  return *reinterpret_cast<const bf16x8*>(p);
}

__device__ __forceinline__ bf16x8 zero8() {
  bf16x8 z;
#pragma unroll
  for (int j = 0; j < 8; ++j) z[j] = static_cast<__bf16>(0.f);
  return z;
}

__device__ __forceinline__ void st8(bf16_t* p, const float* v) {
  bf16x8 o;
#pragma unroll
  for (int j = 0; j < 8; ++j) o[j] = static_cast<__bf16>(v[j]);
  *reinterpret_cast<bf16x8*>(p) = o;
}

// ---------------------------------------------------------------------------
// QK cache build.  Per item m and head h:  cache[m,h,:] = phi(scale * K_h T_m)
// GEMM in transposed form: A = link keys (rows = links of a head, K = d),
// B = item rows (cols = 16 items, K = d), D = logits [links x items].
// Row mapping: M-block c of a head, row 4*g + j  ->  link g*(4*MB) + 4*c + j,
// so lane group g holds links [g*4*MB, (g+1)*4*MB) of its item.
//
// Work: a workgroup takes tiles of TI items (persistent, grid-stride).  The
// tile is staged once in LDS (rows padded by 16 bytes against bank
// conflicts) and shared by all waves; each wave keeps the keys of its heads
// in registers for the whole kernel.  The next tile's rows are prefetched
// into registers while the current tile is computed.
// ---------------------------------------------------------------------------
template <int ELL, int D, int H>
struct QkCfg {
  static constexpr int NW = H >= 8 ? 8 : 4;               // waves per workgroup
  static constexpr int HPW = H > NW ? H / NW : 1;         // heads per wave
  static constexpr int WPH = NW > H ? NW / H : 1;         // waves per head
  static constexpr int MB = ELL / 16;                     // M-blocks per head
  static constexpr int KB = D / 32;                       // K-blocks
  static constexpr int TI = 64;                           // items per tile
  static constexpr int NB = TI / 16;                      // 16-item blocks per tile
  static constexpr int NBW = NB / WPH;                    // item blocks per wave
  static constexpr int STRIDE = D * 2 + 16;               // LDS bytes per item row
  static constexpr int NT = NW * 64;                      // threads
  static constexpr int CPR = D / 8;                       // 16-byte chunks per row
  static constexpr int CPT = TI * CPR / NT;               // chunks per thread
  static_assert(ELL % 16 == 0 && D % 32 == 0, "shape");
  static_assert(H % NW == 0 || NW % H == 0, "heads vs waves");
  static_assert(NB % WPH == 0, "item blocks per wave");
  static_assert((TI * CPR) % NT == 0, "tile load split");
};

template <int ELL, int D, int H>
__global__ __launch_bounds__((QkCfg<ELL, D, H>::NT)) void qk_cache(
    const bf16_t* __restrict__ items, const bf16_t* __restrict__ keys, bf16_t* __restrict__ cache,
    int64_t n_items, float scale, int phi, int64_t ntiles) {
  using C = QkCfg<ELL, D, H>;
  __shared__ __attribute__((aligned(16))) char lds[C::TI * C::STRIDE];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int g = lane >> 4, r = lane & 15;
  const int head0 = (C::WPH > 1) ? (w / C::WPH) : w * C::HPW;
  const int nb0 = (C::WPH > 1) ? (w % C::WPH) * C::NBW : 0;

  // link keys of this wave's heads, as A fragments
  bf16x8 a[C::HPW][C::MB][C::KB];
#pragma unroll
  for (int hh = 0; hh < C::HPW; ++hh)
#pragma unroll
    for (int c = 0; c < C::MB; ++c) {
      const int link = (r >> 2) * (4 * C::MB) + 4 * c + (r & 3);
      const bf16_t* kr = keys + (static_cast<int64_t>(head0 + hh) * ELL + link) * D + 8 * g;
#pragma unroll
      for (int kb = 0; kb < C::KB; ++kb) a[hh][c][kb] = ld16(kr + kb * 32);
    }

  uint4 pf[C::CPT];
  auto gload = [&](int64_t t) {
#pragma unroll
    for (int i = 0; i < C::CPT; ++i) {
      const int e = tid + i * C::NT;
      const int row = e / C::CPR, col = e % C::CPR;
      const int64_t item = t * C::TI + row;
      pf[i] = item < n_items ? *reinterpret_cast<const uint4*>(items + item * D + col * 8)
                             : make_uint4(0, 0, 0, 0);
    }
  };

  int64_t tile = blockIdx.x;
  if (tile < ntiles) gload(tile);
  for (; tile < ntiles; tile += gridDim.x) {
#pragma unroll
    for (int i = 0; i < C::CPT; ++i) {
      const int e = tid + i * C::NT;
      const int row = e / C::CPR, col = e % C::CPR;
      *reinterpret_cast<uint4*>(lds + row * C::STRIDE + col * 16) = pf[i];
    }
    __syncthreads();
    const int64_t nxt = tile + gridDim.x;
    if (nxt < ntiles) gload(nxt);

#pragma unroll
    for (int nbi = 0; nbi < C::NBW; ++nbi) {
      const int nb = nb0 + nbi;
      bf16x8 b[C::KB];
#pragma unroll
      for (int kb = 0; kb < C::KB; ++kb)
        b[kb] = *reinterpret_cast<const bf16x8*>(lds + (nb * 16 + r) * C::STRIDE + (kb * 32 + 8 * g) * 2);
      const int64_t item = tile * C::TI + nb * 16 + r;
#pragma unroll
      for (int hh = 0; hh < C::HPW; ++hh) {
        floatx4 acc[C::MB];
#pragma unroll
        for (int c = 0; c < C::MB; ++c) {
          acc[c] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int kb = 0; kb < C::KB; ++kb) acc[c] = mma(a[hh][c][kb], b[kb], acc[c]);
        }
        float v[4 * C::MB];
#pragma unroll
        for (int c = 0; c < C::MB; ++c)
#pragma unroll
          for (int j = 0; j < 4; ++j) v[4 * c + j] = acc[c][j] * scale;
        if (phi == PHI_SOFTMAX) {
          float mx = v[0];
#pragma unroll
          for (int q = 1; q < 4 * C::MB; ++q) mx = fmaxf(mx, v[q]);
          mx = fmaxf(mx, __shfl_xor(mx, 16));
          mx = fmaxf(mx, __shfl_xor(mx, 32));
          float s = 0.f;
#pragma unroll
          for (int q = 0; q < 4 * C::MB; ++q) {
            v[q] = __expf(v[q] - mx);
            s += v[q];
          }
          s += __shfl_xor(s, 16);
          s += __shfl_xor(s, 32);
          const float inv = 1.f / s;
#pragma unroll
          for (int q = 0; q < 4 * C::MB; ++q) v[q] *= inv;
        } else {
          constexpr float inv = 1.f / ELL;
#pragma unroll
          for (int q = 0; q < 4 * C::MB; ++q) v[q] = silu_f(v[q]) * inv;
        }
        if (item < n_items) {
          bf16_t* o = cache + (item * H + head0 + hh) * ELL + g * 4 * C::MB;
#pragma unroll
          for (int q = 0; q < C::MB / 2; ++q) st8(o + 8 * q, v + 8 * q);
        }
      }
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------
// Candidate scoring, d_h = 32.  Per head, transposed form:
//   A = L^P_b head slice transposed (rows = 32 output columns, K = ell)
//   B = gathered cache rows (cols = 16 candidates, K = ell)
// Row mapping: M-block c, row 4*g + j -> column 8*g + 4*c + j, so lane group g
// ends with columns [8g, 8g+8) of its candidate: one 16-byte store per head.
// Each wave walks a contiguous range of 16-candidate tiles, so the A
// fragments (one user's links) are reloaded only when the user changes.
// ---------------------------------------------------------------------------
template <int ELL, int H>
struct CsCfg {
  static constexpr int D = 32 * H;
  static constexpr int KB = ELL / 32;
  static constexpr int MAXB = 1024;  // users whose offsets are cached in LDS
  static_assert(ELL % 32 == 0, "ell");
};

template <int ELL, int H>
__global__ __launch_bounds__(256) void cand_score(const bf16_t* __restrict__ cache, int64_t n_items,
                                                  const bf16_t* __restrict__ lp,
                                                  const int64_t* __restrict__ ids,
                                                  const int64_t* __restrict__ off_g, int B,
                                                  int64_t total_M, bf16_t* __restrict__ out,
                                                  int* bad, int64_t tiles_per_wave) {
  using C = CsCfg<ELL, H>;
  constexpr int D = C::D, KB = C::KB;
  __shared__ int64_t off_s[C::MAXB + 1];
  const int tid = threadIdx.x, lane = tid & 63;
  const int g = lane >> 4, r = lane & 15;
  const bool in_lds = B <= C::MAXB;
  if (in_lds)
    for (int i = tid; i <= B; i += 256) off_s[i] = off_g[i];
  __syncthreads();
  const int64_t* off = in_lds ? off_s : off_g;

  const int64_t ntiles = (total_M + 15) >> 4;
  const int64_t gw = static_cast<int64_t>(blockIdx.x) * 4 + (tid >> 6);
  const int64_t t0 = gw * tiles_per_wave;
  const int64_t t1 = t0 + tiles_per_wave < ntiles ? t0 + tiles_per_wave : ntiles;
  if (t0 >= t1) return;

  bf16x8 a[H][2][KB];
  int cur = -1;
  int u = find_owner(off, B, t0 * 16);

  for (int64_t t = t0; t < t1; ++t) {
    const int64_t i = t * 16 + r;
    const bool valid = i < total_M;
    int ul = u;
    if (valid)
      while (ul + 1 < B && off[ul + 1] <= i) ++ul;
    const int64_t id = valid ? ids[i] : -1;
    const bool okid = valid && id >= 0 && id < n_items;
    if (valid && !okid && g == 0 && bad != nullptr) atomicAdd(bad, 1);

    bf16x8 bw[H][KB];
#pragma unroll
    for (int h = 0; h < H; ++h)
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
        bw[h][kb] = okid ? ld16(cache + (id * H + h) * ELL + kb * 32 + 8 * g) : zero8();

    const int last = static_cast<int>((total_M - 1 - t * 16) < 15 ? (total_M - 1 - t * 16) : 15);
    const int ufirst = __shfl(ul, 0);
    const int ulast = __shfl(ul, last);
    for (int uu = ufirst; uu <= ulast; ++uu) {
      if (!__any(valid && ul == uu)) continue;
      if (uu != cur) {
        const bf16_t* lb = lp + static_cast<int64_t>(uu) * ELL * D;
#pragma unroll
        for (int h = 0; h < H; ++h)
#pragma unroll
          for (int c = 0; c < 2; ++c) {
            const int col = h * 32 + 8 * (r >> 2) + 4 * c + (r & 3);
#pragma unroll
            for (int kb = 0; kb < KB; ++kb)
#pragma unroll
              for (int j = 0; j < 8; ++j)
                a[h][c][kb][j] = __builtin_bit_cast(__bf16, lb[static_cast<int64_t>(kb * 32 + 8 * g + j) * D + col]);
          }
        cur = uu;
      }
      const bool mine = valid && ul == uu;
#pragma unroll
      for (int h = 0; h < H; ++h) {
        floatx4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
          acc0 = mma(a[h][0][kb], bw[h][kb], acc0);
          acc1 = mma(a[h][1][kb], bw[h][kb], acc1);
        }
        if (mine) {
          const float v[8] = {acc0[0], acc0[1], acc0[2], acc0[3], acc1[0], acc1[1], acc1[2], acc1[3]};
          st8(out + i * D + h * 32 + 8 * g, v);
        }
      }
    }
    u = __shfl(ul, last);
  }
}

}  // namespace mfma
}  // namespace lime

namespace lime {
namespace mfma {

// ===========================================================================
// User side (d_h = 32).  Layout in the workspace, rows = [B*ell link rows ;
// total_N history rows], padded with zero rows to R_pad (multiple of 32):
//   QK [R_pad, 2d]  row-major, Q in columns [0, d), K in [d, 2d)
//   Vp [R_pad/8][d][8]  V "row-octet packed": the 8 values of one column
//                       for 8 consecutive rows are contiguous, which is the
//                       operand layout of the contractions over rows.
// ===========================================================================

__device__ __forceinline__ int64_t vp_index(int64_t row, int col, int D) {
  return (row >> 3) * static_cast<int64_t>(D) * 8 + static_cast<int64_t>(col) * 8 + (row & 7);
}

// LayerNorm (no affine) of the rows a lane group holds: v[k] are this lane's
// values of its row (8 per 32-column block); the other 3 lanes of the row
// are lane ^ 16 and lane ^ 32.
template <int N>
__device__ __forceinline__ void ln_rows(float* v, int D) {
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < N; ++i) s += v[i];
  s += __shfl_xor(s, 16);
  s += __shfl_xor(s, 32);
  const float mu = s / D;
  float q = 0.f;
#pragma unroll
  for (int i = 0; i < N; ++i) {
    const float t = v[i] - mu;
    q += t * t;
  }
  q += __shfl_xor(q, 16);
  q += __shfl_xor(q, 32);
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

// ---------------------------------------------------------------------------
// LN + QKV projection for 32 rows per wave.  Lane (r, g) of row block rb
// carries row row0 + 8*(r/4) + 4*rb + r%4, so that the V contraction (with
// the operands swapped) leaves each lane 8 consecutive rows of one column.
// Q and K use the transposed form: each lane ends with 8 consecutive columns.
// Rows >= R are zero.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void qkv_proj(Rows X, int64_t R, int64_t R_pad,
                                                const bf16_t* __restrict__ W,
                                                bf16_t* __restrict__ QK, bf16_t* __restrict__ Vp) {
  constexpr int KB = D / 32;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int g = lane >> 4, r = lane & 15;
  const int64_t row0 = (static_cast<int64_t>(blockIdx.x) * 4 + w) * 32;
  if (row0 >= R_pad) return;

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

  // Q and K: output column pairs of 32
  for (int p = 0; p < 2 * D / 32; ++p) {
    floatx4 acc[2][2] = {};
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const bf16_t* wr = W + static_cast<int64_t>(32 * p + 8 * (r >> 2) + 4 * c + (r & 3)) * D + 8 * g;
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        const bf16x8 a = ld16(wr + kb * 32);
        acc[c][0] = mma(a, hb[0][kb], acc[c][0]);
        acc[c][1] = mma(a, hb[1][kb], acc[c][1]);
      }
    }
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
      const int64_t row = row0 + 8 * (r >> 2) + 4 * rb + (r & 3);
      const float v[8] = {acc[0][rb][0], acc[0][rb][1], acc[0][rb][2], acc[0][rb][3],
                          acc[1][rb][0], acc[1][rb][1], acc[1][rb][2], acc[1][rb][3]};
      st8(QK + row * (2 * D) + 32 * p + 8 * g, v);
    }
  }
  // V: swapped operands, 16 output columns per block
  for (int n = 0; n < D / 16; ++n) {
    const bf16_t* wr = W + static_cast<int64_t>(2 * D + 16 * n + r) * D + 8 * g;
    floatx4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      const bf16x8 b = ld16(wr + kb * 32);
      acc0 = mma(hb[0][kb], b, acc0);
      acc1 = mma(hb[1][kb], b, acc1);
    }
    const float v[8] = {acc0[0], acc0[1], acc0[2], acc0[3], acc1[0], acc1[1], acc1[2], acc1[3]};
    st8(Vp + vp_index(row0 + 8 * g, 16 * n + r, D), v);
  }
}

// ---------------------------------------------------------------------------
// XOR attention, one wave per (user b, head h, split s), d_h = 32.
//   E-branch (history rows -> ell links), per 16 rows:
//     S^T = K_L Q_E^T (links x rows), phi over links, Y_E^T = V_L^T P^T.
//   L-branch (links -> history rows), per 32 rows:
//     S^T = K_E Q_L^T (rows x links), online softmax over rows,
//     acc (links x d_h) += P V_E with V_E from the row-octet packed buffer.
// Link rows of the mapped D blocks:  M-block c -> link (c/2)*32 + 8*g +
// 4*(c%2) + j, so each lane's 8 links per 32 are the K slice of the P^T
// operand.  History rows in the L-branch: M-block c -> row 8*g + 4*c + j.
// The partial of (b, h, s) is [ell][2 + 32]: running max, denominator, acc.
// ---------------------------------------------------------------------------
template <int ELL, int H>
__global__ __launch_bounds__(256) void xor_attn(const bf16_t* __restrict__ QK,
                                                const bf16_t* __restrict__ Vp,
                                                bf16_t* __restrict__ Y, float* __restrict__ part,
                                                const int64_t* __restrict__ off, int B, int S,
                                                int64_t chunk, int64_t total_N, float scale,
                                                int phi, int do_e) {
  constexpr int D = 32 * H, MB = ELL / 16, KBL = ELL / 32;
  const int lane = threadIdx.x & 63;
  const int g = lane >> 4, r = lane & 15;
  const int64_t gw = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (gw >= static_cast<int64_t>(B) * H * S) return;
  const int s = static_cast<int>(gw % S);
  const int h = static_cast<int>((gw / S) % H);
  const int b = static_cast<int>(gw / (static_cast<int64_t>(S) * H));
  const int64_t nlr = static_cast<int64_t>(B) * ELL;
  const int64_t u0 = clamp64(off[b], 0, total_N);
  const int64_t u1 = clamp64(off[b + 1], u0, total_N);
  const int64_t n = u1 - u0;
  const int64_t lo = u0 + clamp64(s * chunk, 0, n);
  const int64_t hi = (s == S - 1) ? u1 : u0 + clamp64((s + 1) * chunk, 0, n);
  const bool softmax = (phi == PHI_SOFTMAX);
  const int64_t lrow0 = static_cast<int64_t>(b) * ELL;  // first link row of user b

  // per (user, head) operands
  bf16x8 kl[MB], qlt[MB], vlt[2][KBL];
#pragma unroll
  for (int c = 0; c < MB; ++c) {
    const int link = (c >> 1) * 32 + 8 * (r >> 2) + 4 * (c & 1) + (r & 3);
    kl[c] = ld16(QK + (lrow0 + link) * (2 * D) + D + h * 32 + 8 * g);
    qlt[c] = ld16(QK + (lrow0 + 16 * c + r) * (2 * D) + h * 32 + 8 * g);
  }
#pragma unroll
  for (int c2 = 0; c2 < 2; ++c2)
#pragma unroll
    for (int kb = 0; kb < KBL; ++kb)
      vlt[c2][kb] = ld16(Vp + vp_index(lrow0 + kb * 32 + 8 * g, h * 32 + 8 * (r >> 2) + 4 * c2 + (r & 3), D));

  float m_run[MB], l_run[MB];
  floatx4 acc[MB][2];
#pragma unroll
  for (int c = 0; c < MB; ++c) {
    m_run[c] = -INFINITY;
    l_run[c] = 0.f;
    acc[c][0] = floatx4{0.f, 0.f, 0.f, 0.f};
    acc[c][1] = floatx4{0.f, 0.f, 0.f, 0.f};
  }

  for (int64_t c0 = lo & ~int64_t(7); c0 < hi; c0 += 32) {
    // ---------------- E-branch
    if (do_e) {
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) {
        const int64_t j = c0 + 16 * rb + r;
        const bf16x8 qe = ld16(QK + (nlr + j) * (2 * D) + h * 32 + 8 * g);
        float v[4 * MB];
#pragma unroll
        for (int c = 0; c < MB; ++c) {
          const floatx4 st = mma(kl[c], qe, floatx4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
          for (int q = 0; q < 4; ++q) v[4 * c + q] = st[q] * scale;
        }
        if (softmax) {
          float mx = v[0];
#pragma unroll
          for (int q = 1; q < 4 * MB; ++q) mx = fmaxf(mx, v[q]);
          mx = fmaxf(mx, __shfl_xor(mx, 16));
          mx = fmaxf(mx, __shfl_xor(mx, 32));
          float sum = 0.f;
#pragma unroll
          for (int q = 0; q < 4 * MB; ++q) {
            v[q] = __expf(v[q] - mx);
            sum += v[q];
          }
          sum += __shfl_xor(sum, 16);
          sum += __shfl_xor(sum, 32);
          const float inv = 1.f / sum;
#pragma unroll
          for (int q = 0; q < 4 * MB; ++q) v[q] *= inv;
        } else {
          constexpr float inv = 1.f / ELL;
#pragma unroll
          for (int q = 0; q < 4 * MB; ++q) v[q] = silu_f(v[q]) * inv;
        }
        floatx4 y0 = {0.f, 0.f, 0.f, 0.f}, y1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kb = 0; kb < KBL; ++kb) {
          const bf16x8 pb = pack8(v + 8 * kb);
          y0 = mma(vlt[0][kb], pb, y0);
          y1 = mma(vlt[1][kb], pb, y1);
        }
        if (j >= lo && j < hi) {
          const float o[8] = {y0[0], y0[1], y0[2], y0[3], y1[0], y1[1], y1[2], y1[3]};
          st8(Y + (nlr + j) * D + h * 32 + 8 * g, o);
        }
      }
    }
    // ---------------- L-branch
    bf16x8 ke[2];
#pragma unroll
    for (int c = 0; c < 2; ++c)
      ke[c] = ld16(QK + (nlr + c0 + 8 * (r >> 2) + 4 * c + (r & 3)) * (2 * D) + D + h * 32 + 8 * g);
    const bf16x8 ve0 = ld16(Vp + vp_index(nlr + c0 + 8 * g, h * 32 + r, D));
    const bf16x8 ve1 = ld16(Vp + vp_index(nlr + c0 + 8 * g, h * 32 + 16 + r, D));
    bool valid[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const int64_t j = c0 + 8 * g + q;  // q = 4*c + jj
      valid[q] = (j >= lo) && (j < hi);
    }
#pragma unroll
    for (int nb = 0; nb < MB; ++nb) {
      float p[8];
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const floatx4 st = mma(ke[c], qlt[nb], floatx4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
        for (int q = 0; q < 4; ++q) p[4 * c + q] = st[q] * scale;
      }
      if (softmax) {
        float mc = -INFINITY;
#pragma unroll
        for (int q = 0; q < 8; ++q)
          if (valid[q]) mc = fmaxf(mc, p[q]);
        mc = fmaxf(mc, __shfl_xor(mc, 16));
        mc = fmaxf(mc, __shfl_xor(mc, 32));
        const float mn = fmaxf(m_run[nb], mc);
        const float alpha = (m_run[nb] == -INFINITY) ? 0.f : __expf(m_run[nb] - mn);
        float ls = 0.f;
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          p[q] = valid[q] ? __expf(p[q] - mn) : 0.f;
          ls += p[q];
        }
        ls += __shfl_xor(ls, 16);
        ls += __shfl_xor(ls, 32);
        l_run[nb] = l_run[nb] * alpha + ls;
        m_run[nb] = mn;
        // acc rows are links 16*nb + 4*g + jj; their factor sits in lane 4*g + jj
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          const float f = __shfl(alpha, 4 * g + jj);
          acc[nb][0][jj] *= f;
          acc[nb][1][jj] *= f;
        }
      } else {
#pragma unroll
        for (int q = 0; q < 8; ++q) p[q] = valid[q] ? silu_f(p[q]) : 0.f;
      }
      const bf16x8 pa = pack8(p);
      acc[nb][0] = mma(pa, ve0, acc[nb][0]);
      acc[nb][1] = mma(pa, ve1, acc[nb][1]);
    }
  }

  // ---------------- partial of this split
  float* p0 = part + (((static_cast<int64_t>(b) * H + h) * S + s) * ELL) * 34;
#pragma unroll
  for (int nb = 0; nb < MB; ++nb) {
    if (g == 0) {
      float* pl = p0 + (16 * nb + r) * 34;
      pl[0] = softmax ? m_run[nb] : 0.f;
      pl[1] = softmax ? l_run[nb] : static_cast<float>(hi - lo);
    }
#pragma unroll
    for (int c2 = 0; c2 < 2; ++c2)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj)
        p0[(16 * nb + 4 * g + jj) * 34 + 2 + 16 * c2 + r] = acc[nb][c2][jj];
  }
}

// ---------------------------------------------------------------------------
// Post-attention block for RPW rows per wave, everything in registers:
//   X1 = Xres + Y Wo^T ;  G = LN(X1) ;  M = SiLU(G Wg^T) * (G Wu^T) ;
//   Out = X1 + M Wd^T
// Every product is in the transposed form, so the output of one is the
// B operand of the next without any data movement.
// ---------------------------------------------------------------------------
template <int D, int DFF, int RPW>
__global__ __launch_bounds__(256) void post_block(Rows Yr, Rows Xres, Rows Out, int64_t nrows,
                                                  const bf16_t* __restrict__ Wo,
                                                  const bf16_t* __restrict__ Wg,
                                                  const bf16_t* __restrict__ Wu,
                                                  const bf16_t* __restrict__ Wd) {
  constexpr int KB = D / 32, KF = DFF / 32, RB = RPW / 16;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int g = lane >> 4, r = lane & 15;
  const int64_t row0 = (static_cast<int64_t>(blockIdx.x) * 4 + w) * RPW;
  if (row0 >= nrows) return;

  bf16x8 yb[RB][KB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const int64_t row = row0 + 16 * rb + r;
    if (row < nrows) {
      const bf16_t* yr = row_in<bf16_t>(Yr, row) + 8 * g;
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) yb[rb][kb] = ld16(yr + kb * 32);
    } else {
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) yb[rb][kb] = zero8();
    }
  }

  // X1 = Xres + Y Wo^T
  float x1[RB][8 * KB];
#pragma unroll
  for (int p = 0; p < KB; ++p) {
    floatx4 acc[2][RB] = {};
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const bf16_t* wr = Wo + static_cast<int64_t>(32 * p + 8 * (r >> 2) + 4 * c + (r & 3)) * D + 8 * g;
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        const bf16x8 a = ld16(wr + kb * 32);
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) acc[c][rb] = mma(a, yb[rb][kb], acc[c][rb]);
      }
    }
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      const int64_t row = row0 + 16 * rb + r;
      bf16x8 xr = zero8();
      if (row < nrows) xr = ld16(row_in<bf16_t>(Xres, row) + 32 * p + 8 * g);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        x1[rb][8 * p + q] = acc[0][rb][q] + static_cast<float>(xr[q]);
        x1[rb][8 * p + 4 + q] = acc[1][rb][q] + static_cast<float>(xr[4 + q]);
      }
    }
  }

  // G = LN(X1) as B operands
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

  // M = SiLU(G Wg^T) * (G Wu^T)
  bf16x8 mb[RB][KF];
#pragma unroll
  for (int q2 = 0; q2 < KF; ++q2) {
    floatx4 ag[2][RB] = {}, au[2][RB] = {};
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const int64_t orow = 32 * q2 + 8 * (r >> 2) + 4 * c + (r & 3);
      const bf16_t* gr = Wg + orow * D + 8 * g;
      const bf16_t* ur = Wu + orow * D + 8 * g;
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
  }

  // Out = X1 + M Wd^T
#pragma unroll
  for (int p = 0; p < KB; ++p) {
    floatx4 acc[2][RB] = {};
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const bf16_t* wr = Wd + static_cast<int64_t>(32 * p + 8 * (r >> 2) + 4 * c + (r & 3)) * DFF + 8 * g;
#pragma unroll
      for (int kf = 0; kf < KF; ++kf) {
        const bf16x8 a = ld16(wr + kf * 32);
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) acc[c][rb] = mma(a, mb[rb][kf], acc[c][rb]);
      }
    }
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      const int64_t row = row0 + 16 * rb + r;
      if (row >= nrows) continue;
      bf16_t* orow = row_out<bf16_t>(Out, row);
      if (orow == nullptr) continue;
      float v[8];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        v[q] = x1[rb][8 * p + q] + acc[0][rb][q];
        v[4 + q] = x1[rb][8 * p + 4 + q] + acc[1][rb][q];
      }
      st8(orow + 32 * p + 8 * g, v);
    }
  }
}

}  // namespace mfma
}  // namespace lime
