// Portable (VALU, any shape) kernels of the hot path.  They serve the float32
// element type and every shape the matrix-core kernels do not cover; they
// compute exactly what the MFMA kernels compute, in float32.
#pragma once

#include "common.h"

namespace lime {
namespace gen {

// ---------------------------------------------------------------------------
// Row-block GEMM with optional LayerNorm prologue and fused epilogues:
//   acc[r, c] = sum_k P(X)[r, k] * W[c, k]            (W is [NOUT, K])
//   EPI_STORE : Y[r, c] = acc
//   EPI_RESID : Y[r, c] = R[r, c] + acc
//   EPI_SWIGLU: Y[r, c] = SiLU(acc_gate) * acc_up      (W = gate, W2 = up)
// P = LayerNorm without affine when LN is set.  Rows [row0, row0 + nrows).
// ---------------------------------------------------------------------------
enum : int { EPI_STORE = 0, EPI_RESID = 1, EPI_SWIGLU = 2 };

constexpr int GB_M = 64, GB_N = 64, GB_K = 32;

template <typename T, bool LN, int EPI>
__global__ __launch_bounds__(256) void gemm_rows(Rows X, int64_t row0, int64_t nrows, int K,
                                                 const T* __restrict__ W,
                                                 const T* __restrict__ W2, int NOUT, Rows R,
                                                 Rows Y) {
  __shared__ float As[GB_K][GB_M + 1];
  __shared__ float Ws[GB_K][GB_N + 1];
  __shared__ float W2s[EPI == EPI_SWIGLU ? GB_K : 1][GB_N + 1];
  __shared__ float mean_s[GB_M], rstd_s[GB_M];

  const int tid = threadIdx.x;
  const int64_t rbase = row0 + static_cast<int64_t>(blockIdx.x) * GB_M;
  const int cbase = blockIdx.y * GB_N;
  const int64_t rend = row0 + nrows;

  if (LN) {
    // 4 threads per row: two-pass mean / variance in float32
    const int r = tid >> 2, q = tid & 3;
    const int64_t gr = rbase + r;
    float s = 0.f;
    if (gr < rend) {
      const T* xr = row_in<T>(X, gr);
      for (int k = q; k < K; k += 4) s += Elt<T>::ld(xr + k);
    }
    s += __shfl_xor(s, 1);
    s += __shfl_xor(s, 2);
    const float mu = s / K;
    float v = 0.f;
    if (gr < rend) {
      const T* xr = row_in<T>(X, gr);
      for (int k = q; k < K; k += 4) {
        float t = Elt<T>::ld(xr + k) - mu;
        v += t * t;
      }
    }
    v += __shfl_xor(v, 1);
    v += __shfl_xor(v, 2);
    if (q == 0) {
      mean_s[r] = mu;
      rstd_s[r] = rsqrtf(v / K + 1e-5f);
    }
    __syncthreads();
  }

  // each thread: 4 rows x 4 cols
  const int tr = (tid >> 4) * 4, tc = (tid & 15) * 4;
  float acc[4][4] = {}, acc2[4][4] = {};

  for (int k0 = 0; k0 < K; k0 += GB_K) {
    // load X tile (GB_M x GB_K) and W tile (GB_N x GB_K), transposed into LDS
    for (int e = tid; e < GB_M * GB_K; e += 256) {
      const int r = e / GB_K, k = e % GB_K;
      const int64_t gr = rbase + r;
      float v = 0.f;
      if (gr < rend && k0 + k < K) {
        v = Elt<T>::ld(row_in<T>(X, gr) + k0 + k);
        if (LN) v = (v - mean_s[r]) * rstd_s[r];
      }
      As[k][r] = v;
    }
    for (int e = tid; e < GB_N * GB_K; e += 256) {
      const int c = e / GB_K, k = e % GB_K;
      const int gc = cbase + c;
      const bool ok = gc < NOUT && k0 + k < K;
      Ws[k][c] = ok ? Elt<T>::ld(W + static_cast<int64_t>(gc) * K + k0 + k) : 0.f;
      if (EPI == EPI_SWIGLU)
        W2s[k][c] = ok ? Elt<T>::ld(W2 + static_cast<int64_t>(gc) * K + k0 + k) : 0.f;
    }
    __syncthreads();
#pragma unroll 8
    for (int k = 0; k < GB_K; ++k) {
      float a[4], b[4], b2[4];
      for (int i = 0; i < 4; ++i) a[i] = As[k][tr + i];
      for (int j = 0; j < 4; ++j) b[j] = Ws[k][tc + j];
      if (EPI == EPI_SWIGLU)
        for (int j = 0; j < 4; ++j) b2[j] = W2s[k][tc + j];
      for (int i = 0; i < 4; ++i)
        for (int j = 0; j < 4; ++j) {
          acc[i][j] += a[i] * b[j];
          if (EPI == EPI_SWIGLU) acc2[i][j] += a[i] * b2[j];
        }
    }
    __syncthreads();
  }

  for (int i = 0; i < 4; ++i) {
    const int64_t gr = rbase + tr + i;
    if (gr >= rend) continue;
    T* yr = row_out<T>(Y, gr);
    if (yr == nullptr) continue;
    const T* rr = (EPI == EPI_RESID) ? row_in<T>(R, gr) : nullptr;
    for (int j = 0; j < 4; ++j) {
      const int gc = cbase + tc + j;
      if (gc >= NOUT) continue;
      float v = acc[i][j];
      if (EPI == EPI_RESID) v += Elt<T>::ld(rr + gc);
      if (EPI == EPI_SWIGLU) v = silu_f(acc[i][j]) * acc2[i][j];
      Elt<T>::st(yr + gc, v);
    }
  }
}

// ---------------------------------------------------------------------------
// XOR attention, both branches, one block per (user, head, split).
// QKV is [R, 3d] row-major (Q | K | V); user b's links are rows b*ell..,
// its history rows are n_link_rows + off[b] ...  The history rows handled by
// split s are [lo, hi) of the user's history.
//   E-branch: each history row attends to the user's ell links  -> Y rows.
//   L-branch: each link attends to the split's history rows -> partial
//             (running max m, denominator l, unnormalised acc[dh]) per link,
//             merged over splits by xor_combine.
// With phi = silu_mean the partial holds m = 0, l = row count, acc = sum.
// ---------------------------------------------------------------------------
template <typename T, int DH>
__global__ __launch_bounds__(256) void xor_attn(const T* __restrict__ qkv, T* __restrict__ Y,
                                                float* __restrict__ part,
                                                const int64_t* __restrict__ off, int B, int ell,
                                                int d, int H, int S, int64_t chunk,
                                                int64_t total_N, float scale, int phi,
                                                int do_e_branch, int half) {
  const int b = blockIdx.x, h = blockIdx.y, s = blockIdx.z;
  const int tid = threadIdx.x;
  const int64_t ld = 3 * static_cast<int64_t>(d);
  const int64_t nlr = static_cast<int64_t>(B) * ell;
  const int64_t u0 = clamp64(off[b], 0, total_N);
  const int64_t u1 = clamp64(off[b + 1], u0, total_N);
  const int64_t n = u1 - u0;
  const int64_t lo = u0 + clamp64(s * chunk, 0, n);
  const int64_t hi = (s == S - 1) ? u1 : u0 + clamp64((s + 1) * chunk, 0, n);
  const T* links = qkv + static_cast<int64_t>(b) * ell * ld + h * DH;  // Q of link 0, head h

  // ---- E-branch: history rows -> links (and, with half > 0, the history
  // rows q of the same user with 1 <= |q - j| <= half: LIME-XOR+Window)
  if (do_e_branch) {
    for (int64_t j = lo + tid; j < hi; j += 256) {
      const T* row = qkv + (nlr + j) * ld + h * DH;
      float q[DH];
#pragma unroll
      for (int c = 0; c < DH; ++c) q[c] = Elt<T>::ld(row + c) * scale;
      // keys: the ell links, then the window rows (none when half = 0)
      const int64_t w0 = j - half > u0 ? j - half : u0;
      const int64_t w1 = j + half < u1 - 1 ? j + half : u1 - 1;
      const int64_t nwin = half > 0 ? w1 - w0 + 1 : 0;
      auto key_row = [&](int64_t t) -> const T* {
        if (t < ell) return links + t * ld + d;
        int64_t qr = w0 + (t - ell);
        if (qr >= j) ++qr;  // skip the row itself
        return qkv + (nlr + qr) * ld + d + h * DH;
      };
      const int64_t nkeys = ell + (nwin > 0 ? nwin - 1 : 0);
      float m = -INFINITY;
      if (phi == PHI_SOFTMAX) {
        for (int64_t k = 0; k < nkeys; ++k) {
          const T* kr = key_row(k);
          float sc = 0.f;
#pragma unroll
          for (int c = 0; c < DH; ++c) sc += q[c] * Elt<T>::ld(kr + c);
          m = fmaxf(m, sc);
        }
      }
      float l = 0.f, acc[DH];
#pragma unroll
      for (int c = 0; c < DH; ++c) acc[c] = 0.f;
      for (int64_t k = 0; k < nkeys; ++k) {
        const T* kr = key_row(k);
        float sc = 0.f;
#pragma unroll
        for (int c = 0; c < DH; ++c) sc += q[c] * Elt<T>::ld(kr + c);
        const float w = (phi == PHI_SOFTMAX) ? __expf(sc - m) : silu_f(sc);
        l += (phi == PHI_SOFTMAX) ? w : 1.f;
#pragma unroll
        for (int c = 0; c < DH; ++c) acc[c] += w * Elt<T>::ld(kr + d + c);
      }
      const float inv = 1.f / l;
      T* yr = Y + (nlr + j) * d + h * DH;
#pragma unroll
      for (int c = 0; c < DH; ++c) Elt<T>::st(yr + c, acc[c] * inv);
    }
  }

  // ---- L-branch: links -> this split's history rows.  RL lanes (a power
  // of two, an aligned group inside one wave) share each link.
  int RL = 1;
  while (RL * 2 <= 64 && RL * 2 * ell <= 256) RL *= 2;
  const int k = tid / RL, r = tid % RL;
  float m = -INFINITY, l = 0.f, acc[DH];
#pragma unroll
  for (int c = 0; c < DH; ++c) acc[c] = 0.f;
  if (k < ell) {
    float q[DH];
#pragma unroll
    for (int c = 0; c < DH; ++c) q[c] = Elt<T>::ld(links + k * ld + c) * scale;
    for (int64_t j = lo + r; j < hi; j += RL) {
      const T* row = qkv + (nlr + j) * ld + d + h * DH;
      float sc = 0.f;
#pragma unroll
      for (int c = 0; c < DH; ++c) sc += q[c] * Elt<T>::ld(row + c);
      float w;
      if (phi == PHI_SOFTMAX) {
        if (sc > m) {
          const float f = __expf(m - sc);  // 0 when m = -inf
          l *= f;
#pragma unroll
          for (int c = 0; c < DH; ++c) acc[c] *= f;
          m = sc;
        }
        w = __expf(sc - m);
        l += w;
      } else {
        w = silu_f(sc);
        l += 1.f;
      }
#pragma unroll
      for (int c = 0; c < DH; ++c) acc[c] += w * Elt<T>::ld(row + d + c);
    }
    if (phi != PHI_SOFTMAX) m = 0.f;
  }
  // merge the RL lanes of each link (every lane of the wave takes part)
  for (int o = RL >> 1; o > 0; o >>= 1) {
    const float m2 = __shfl_xor(m, o);
    const float l2 = __shfl_xor(l, o);
    const float M = fmaxf(m, m2);
    const float f1 = (m == -INFINITY) ? 0.f : __expf(m - M);
    const float f2 = (m2 == -INFINITY) ? 0.f : __expf(m2 - M);
    l = l * f1 + l2 * f2;
#pragma unroll
    for (int c = 0; c < DH; ++c) {
      const float a2 = __shfl_xor(acc[c], o);
      acc[c] = acc[c] * f1 + a2 * f2;
    }
    m = M;
  }
  if (k < ell && r == 0) {
    float* p = part + (((static_cast<int64_t>(b) * H + h) * S + s) * ell + k) * (DH + 2);
    p[0] = m;
    p[1] = l;
#pragma unroll
    for (int c = 0; c < DH; ++c) p[2 + c] = acc[c];
  }
}

// Merge split partials into the link rows of Y:  Y = sum_s acc_s e^{m_s-M} /
// sum_s l_s e^{m_s-M}; zero when the user has no history.
template <typename T, int DH>
__global__ void xor_combine(const float* __restrict__ part, T* __restrict__ Y, int B, int ell,
                            int d, int H, int S, int64_t yrs, int64_t yps) {
  const int64_t gid = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  const int64_t total = static_cast<int64_t>(B) * H * ell * DH;
  if (gid >= total) return;
  const int c = gid % DH;
  const int k = (gid / DH) % ell;
  const int h = (gid / (static_cast<int64_t>(DH) * ell)) % H;
  const int b = gid / (static_cast<int64_t>(DH) * ell * H);
  const float* p0 = part + ((static_cast<int64_t>(b) * H + h) * S) * ell * (DH + 2);
  float M = -INFINITY;
  for (int s = 0; s < S; ++s) M = fmaxf(M, p0[(static_cast<int64_t>(s) * ell + k) * (DH + 2)]);
  float num = 0.f, den = 0.f;
  for (int s = 0; s < S; ++s) {
    const float* p = p0 + (static_cast<int64_t>(s) * ell + k) * (DH + 2);
    const float f = (p[0] == -INFINITY) ? 0.f : __expf(p[0] - M);
    den += f * p[1];
    num += f * p[2 + c];
  }
  const float v = den > 0.f ? num / den : 0.f;
  // Y row b * ell + k, head h: at h * yps + row * yrs (row-major: yrs = d,
  // yps = DH; head-planar: yrs = DH, yps = rows * DH)
  Elt<T>::st(Y + h * yps + (static_cast<int64_t>(b) * ell + k) * yrs + c, v);
}

// ---------------------------------------------------------------------------
// QK cache: one thread per (item, head); logits staged in LDS.  With I8 the
// row is stored as symmetric int8 codes plus a float32 scale.
// ---------------------------------------------------------------------------
template <typename T, bool I8 = false>
__global__ __launch_bounds__(64) void qk_cache(const T* __restrict__ items,
                                               const T* __restrict__ keys, void* __restrict__ cache_out,
                                               float* __restrict__ qscale, int64_t n_items, int d,
                                               int H, int ell, float scale, int phi) {
  extern __shared__ float sbuf[];  // [64][ell]
  const int h = blockIdx.y;
  const int64_t m = static_cast<int64_t>(blockIdx.x) * 64 + threadIdx.x;
  if (m >= n_items) return;
  float* s = sbuf + threadIdx.x * ell;
  const T* t = items + m * d;
  const T* kh = keys + static_cast<int64_t>(h) * ell * d;
  float mx = -INFINITY;
  for (int k = 0; k < ell; ++k) {
    float a = 0.f;
    for (int c = 0; c < d; ++c) a += Elt<T>::ld(t + c) * Elt<T>::ld(kh + static_cast<int64_t>(k) * d + c);
    a *= scale;
    s[k] = a;
    mx = fmaxf(mx, a);
  }
  if (phi == PHI_SOFTMAX) {
    float z = 0.f;
    for (int k = 0; k < ell; ++k) {
      s[k] = __expf(s[k] - mx);
      z += s[k];
    }
    const float inv = 1.f / z;
    for (int k = 0; k < ell; ++k) s[k] *= inv;
  } else {
    const float inv = 1.f / ell;
    for (int k = 0; k < ell; ++k) s[k] = silu_f(s[k]) * inv;
  }
  if constexpr (I8) {
    float am = 0.f;
    for (int k = 0; k < ell; ++k) am = fmaxf(am, fabsf(s[k]));
    const float inv = am > 0.f ? 127.f / am : 0.f;
    int8_t* out = static_cast<int8_t*>(cache_out) + (m * H + h) * ell;
    for (int k = 0; k < ell; ++k)
      out[k] = static_cast<int8_t>(fminf(fmaxf(__builtin_rintf(s[k] * inv), -127.f), 127.f));
    qscale[m * H + h] = am / 127.f;
  } else {
    T* out = static_cast<T*>(cache_out) + (m * H + h) * ell;
    for (int k = 0; k < ell; ++k) Elt<T>::st(out + k, s[k]);
  }
}

// ---------------------------------------------------------------------------
// Candidate scoring: one thread per output element (candidate i, column c).
// ---------------------------------------------------------------------------
template <typename T, bool I8 = false>
__global__ __launch_bounds__(256) void cand_score(const void* __restrict__ cache_in,
                                                  const float* __restrict__ qscale, int64_t n_items,
                                                  const T* __restrict__ lp,
                                                  const int64_t* __restrict__ ids,
                                                  const int64_t* __restrict__ off, int B,
                                                  int ell, int d, int H, int64_t total_M,
                                                  T* __restrict__ out, int* bad) {
  const int64_t gid = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (gid >= total_M * d) return;
  const int64_t i = gid / d;
  const int c = gid % d;
  const int dh = d / H;
  const int h = c / dh;
  const int b = find_owner(off, B, i);
  const int64_t id = ids[i];
  float v = 0.f;
  if (id < 0 || id >= n_items) {
    if (c == 0 && bad != nullptr) atomicAdd(bad, 1);
  } else {
    const T* l = lp + static_cast<int64_t>(b) * ell * d + c;
    if constexpr (I8) {
      const int8_t* w = static_cast<const int8_t*>(cache_in) + (id * H + h) * ell;
      for (int k = 0; k < ell; ++k) v += static_cast<float>(w[k]) * Elt<T>::ld(l + static_cast<int64_t>(k) * d);
      v *= qscale[id * H + h];
    } else {
      const T* w = static_cast<const T*>(cache_in) + (id * H + h) * ell;
      for (int k = 0; k < ell; ++k) v += Elt<T>::ld(w + k) * Elt<T>::ld(l + static_cast<int64_t>(k) * d);
    }
  }
  Elt<T>::st(out + gid, v);
}

// ---------------------------------------------------------------------------
// Uncached scoring: one thread per (candidate, head); the candidate's
// weights for the head are computed into LDS, then the weighted sum.
// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(64) void cand_score_uncached(
    const T* __restrict__ items, int64_t n_items, const T* __restrict__ keys, const T* __restrict__ lp,
    const int64_t* __restrict__ ids, const int64_t* __restrict__ off, int B, int ell, int d, int H,
    int64_t total_M, T* __restrict__ out, int* bad, float scale, int phi) {
  extern __shared__ float sbuf[];  // [64][ell]
  const int h = blockIdx.y;
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 64 + threadIdx.x;
  if (i >= total_M) return;
  float* s = sbuf + threadIdx.x * ell;
  const int dh = d / H;
  const int64_t id = ids[i];
  T* o = out + i * d + h * dh;
  if (id < 0 || id >= n_items) {
    if (h == 0 && bad != nullptr) atomicAdd(bad, 1);
    for (int c = 0; c < dh; ++c) Elt<T>::st(o + c, 0.f);
    return;
  }
  const int b = find_owner(off, B, i);
  const T* t = items + id * d;
  const T* kh = keys + static_cast<int64_t>(h) * ell * d;
  float mx = -INFINITY;
  for (int k = 0; k < ell; ++k) {
    float a = 0.f;
    for (int c = 0; c < d; ++c) a += Elt<T>::ld(t + c) * Elt<T>::ld(kh + static_cast<int64_t>(k) * d + c);
    s[k] = a * scale;
    mx = fmaxf(mx, s[k]);
  }
  if (phi == PHI_SOFTMAX) {
    float z = 0.f;
    for (int k = 0; k < ell; ++k) {
      s[k] = __expf(s[k] - mx);
      z += s[k];
    }
    for (int k = 0; k < ell; ++k) s[k] /= z;
  } else {
    for (int k = 0; k < ell; ++k) s[k] = silu_f(s[k]) / ell;
  }
  const T* l = lp + static_cast<int64_t>(b) * ell * d + h * dh;
  for (int c = 0; c < dh; ++c) {
    float v = 0.f;
    for (int k = 0; k < ell; ++k) v += s[k] * Elt<T>::ld(l + static_cast<int64_t>(k) * d + c);
    Elt<T>::st(o + c, v);
  }
}

}  // namespace gen
}  // namespace lime
