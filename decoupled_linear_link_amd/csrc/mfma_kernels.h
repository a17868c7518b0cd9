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

