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

// An opaque zero: offsetting an LDS operand pointer by it inside a loop keeps
// the compiler from hoisting every loop-invariant fragment load out of the
// loop (which would hold whole weight matrices in registers and spill).
__device__ __forceinline__ int opaque_zero() {
  int z = 0;
  asm volatile("" : "+v"(z));
  return z;
}

// Workgroup barrier for kernels whose waves share data through LDS only:
// it orders LDS accesses and waits for them, but leaves global loads
// (register prefetches) and global stores in flight across the barrier,
// where __syncthreads() would wait for every outstanding memory operation.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Reductions over the four 16-lane rows of a wave (lanes l, l^16, l^32,
// l^48), the lane groups that share a row of an MFMA operand.  The gfx950
// row-swap instructions give each pair's two values to both lanes, so a
// step is one VALU op instead of an LDS permute round trip; the adds pair
// the same values as a butterfly of xor-shuffles, so results are equal.
__device__ __forceinline__ float rows_sum(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

__device__ __forceinline__ float rows_max(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

__device__ __forceinline__ floatx4 mma(const bf16x8& a, const bf16x8& b, const floatx4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 ld16(const bf16_t* p) {
  return *reinterpret_cast<const bf16x8*>(p);
}

// Operands of the XOR attention's products (Q, K, V and the probabilities)
// are float16: the same matrix-core rate as bf16 with three more mantissa
// bits.  Their ranges are bounded (projections of LayerNorm rows, weights
// in [0, 1] or about the size of the logits), far inside float16's.
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ floatx4 mma(const f16x8& a, const f16x8& b, const floatx4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// 16 bytes of float16 held in a 16-bit buffer
__device__ __forceinline__ f16x8 ldh16(const bf16_t* p) {
  return *reinterpret_cast<const f16x8*>(p);
}

__device__ __forceinline__ f16x8 packh8(const float* v) {
  f16x8 o;
#pragma unroll
  for (int j = 0; j < 8; ++j) o[j] = static_cast<_Float16>(v[j]);
  return o;
}

__device__ __forceinline__ void st8h(bf16_t* p, const float* v) {
  *reinterpret_cast<f16x8*>(p) = packh8(v);
}

// 4 floats as float16 (8 bytes)
__device__ __forceinline__ void st4h(bf16_t* p, const floatx4& v) {
  typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
  f16x4 o;
#pragma unroll
  for (int j = 0; j < 4; ++j) o[j] = static_cast<_Float16>(v[j]);
  *reinterpret_cast<f16x4*>(p) = o;
}

// 4 floats as bf16 (8 bytes)
__device__ __forceinline__ void st4(bf16_t* p, const floatx4& v) {
  typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
  bf16x4 o;
#pragma unroll
  for (int j = 0; j < 4; ++j) o[j] = static_cast<__bf16>(v[j]);
  *reinterpret_cast<bf16x4*>(p) = o;
}

// The same as a streaming (non-temporal) store: for outputs written once
// and not read back by the kernel.  Scoring writes its outputs this way so
// that they do not evict the hot cache rows its gathers reuse.
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ void st8_stream(bf16_t* p, const float* v) {
  bf16x8 o;
#pragma unroll
  for (int j = 0; j < 8; ++j) o[j] = static_cast<__bf16>(v[j]);
  __builtin_nontemporal_store(__builtin_bit_cast(u32x4_t, o), reinterpret_cast<u32x4_t*>(p));
}

// phi in log2 units.  A logit x = scale * s is used as y = x log2(e):
//   softmax  2^(y - max y)                 (the same weights)
//   silu2(y) = y / (1 + 2^-y) = SiLU(x) / ln 2, the ln 2 going into the
//   normaliser.  Scaling by scale*log2(e) once replaces the scaling and the
//   base-e conversion of every exponential.
constexpr float LOG2E = 1.4426950408889634f;
constexpr float LN2 = 0.6931471805599453f;

__device__ __forceinline__ float exp2_f(float y) { return __builtin_amdgcn_exp2f(y); }

__device__ __forceinline__ float silu2(float y) {
  return y * __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(-y));
}

// silu2(y) / c in one operation fewer: y / (c + c 2^-y).  With
// c = n log2(e) this is SiLU(x) / n.
__device__ __forceinline__ float silu2_div(float y, float c) {
  return y * __builtin_amdgcn_rcpf(__builtin_fmaf(c, __builtin_amdgcn_exp2f(-y), c));
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
// LDS-DMA (global -> LDS buffer loads) and counted waits
// ---------------------------------------------------------------------------
typedef __attribute__((address_space(3))) void lds_void_t;

// wait until at most n of this wave's vector memory operations are
// outstanding (they complete in issue order)
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt");
  // gfx9 encoding: vmcnt bits [3:0] and [15:14]; expcnt (7) and lgkmcnt (15)
  // at their maxima, so only vector memory is waited for
  __builtin_amdgcn_s_waitcnt(0x0F70 | (N & 15) | ((N >> 4) << 14));
}

// Workgroup barrier for waves that only read the LDS buffers which their
// own LDS-DMA loads fill: each wave has already waited (vmcnt) for its
// loads, so the barrier needs no memory fence; a fence would make the
// compiler wait for every LDS-DMA load in flight, including chunks loaded
// ahead.  The compiler-only fences keep LDS reads on their side of it.
__device__ __forceinline__ void dma_barrier() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_barrier();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// A raw buffer descriptor over `bytes` bytes at p (raw 32-bit offsets, no
// stride): loads past the extent return 0, stores past it are dropped.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t bytes_rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), 0, static_cast<int>(bytes), 0x00020000);
}

// ---------------------------------------------------------------------------
// QK cache build.  Per item m and head h:  cache[m,h,:] = phi(scale * K_h T_m)
// GEMM in transposed form: A = link keys (rows = links of a head, K = d),
// B = item rows (cols = 16 items, K = d), D = logits [links x items].
// Row mapping: M-block c of a head, row 4*g + j  ->  link g*(4*MB) + 4*c + j,
// so lane group g holds links [g*4*MB, (g+1)*4*MB) of its item.
//
// Work: a workgroup takes tiles of TI items (persistent, grid-stride).  The
// tile is staged once in LDS (rows padded by 16 bytes) and shared by all
// waves; each wave keeps the keys of its heads
// in registers for the whole kernel.  The next tile's rows are prefetched
// into registers while the current tile is computed.
// ---------------------------------------------------------------------------
template <int ELL, int D, int H, bool I8 = false>
struct QkCfg {
  static constexpr int NW = H >= 8 ? 8 : 4;               // waves per workgroup
  static constexpr int HPW = H > NW ? H / NW : 1;         // heads per wave
  static constexpr int WPH = NW > H ? NW / H : 1;         // waves per head
  static constexpr int MB = ELL / 16;                     // M-blocks per head
  static constexpr int KB = D / 32;                       // K-blocks
  // items per tile: at d = 64 a bf16 tile of 128 items (16 KB of item rows
  // per 4-wave workgroup) beats 64 (a catalogue of 100k items: 7.7 against
  // 8.2 us); the int8 form, with its quantisation epilogue, stays at 64
  static constexpr int TI = (D <= 64 && !I8) ? 128 : 64;
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

// Symmetric int8 codes of the values a lane holds for one (item, head): the
// other values of the row are in lanes ^16, ^32.  scale = max|v| / 127,
// code = round-half-even(v * 127 / max|v|); an all-zero row gets scale 0.
// The codes come out packed, four per dword (value 4j + b in byte b of
// q[j]).  Rounding: adding 1.5 * 2^23 to a float of magnitude at most 127
// leaves round-half-even of it, two's complement, in the low byte of the
// sum's bits, so one fused multiply-add per value replaces the multiply,
// round, clamp and conversion (|v * inv| <= 127 by the choice of inv; a
// non-finite row gets inv = 0 or a NaN product, whose low byte is 0 or
// unspecified, never a fault).
template <int N>
__device__ __forceinline__ float quantize_i8(const float* v, uint32_t* q) {
  static_assert(N % 4 == 0, "codes pack four per dword");
  float m = 0.f;
#pragma unroll
  for (int i = 0; i < N; ++i) m = fmaxf(m, fabsf(v[i]));
  m = rows_max(m);
  const float inv = m > 0.f ? 127.f / m : 0.f;
  constexpr float RND = 12582912.f;  // 1.5 * 2^23
#pragma unroll
  for (int j = 0; j < N / 4; ++j) {
    const uint32_t b0 = __float_as_uint(fmaf(v[4 * j], inv, RND));
    const uint32_t b1 = __float_as_uint(fmaf(v[4 * j + 1], inv, RND));
    const uint32_t b2 = __float_as_uint(fmaf(v[4 * j + 2], inv, RND));
    const uint32_t b3 = __float_as_uint(fmaf(v[4 * j + 3], inv, RND));
    // byte selectors: 0x00 = low byte of the second operand, 0x04 = low
    // byte of the first, 0x0c = zero
    q[j] = __builtin_amdgcn_perm(b1, b0, 0x0c0c0400u) | __builtin_amdgcn_perm(b3, b2, 0x04000c0cu);
  }
  return m / 127.f;
}

// phi over the ell links of one (item, head) whose scores a lane group
// holds (lane (r, g): item r, links 4 MB g .. +4 MB in acc[c][j], link order
// of the cache kernels' A operands), into v (4 MB values per lane).
template <int ELL>
__device__ __forceinline__ void cache_phi(const floatx4 (&acc)[ELL / 16], float scale, int phi,
                                          float (&v)[ELL / 4]) {
  constexpr int MB = ELL / 16;
  // logits in log2 units
  const float k = scale * LOG2E;
#pragma unroll
  for (int c = 0; c < MB; ++c)
#pragma unroll
    for (int j = 0; j < 4; ++j) v[4 * c + j] = acc[c][j] * k;
  if (phi == PHI_SOFTMAX) {
    float mx = v[0];
#pragma unroll
    for (int q = 1; q < 4 * MB; ++q) mx = fmaxf(mx, v[q]);
    mx = rows_max(mx);
    float s = 0.f;
#pragma unroll
    for (int q = 0; q < 4 * MB; ++q) {
      v[q] = exp2_f(v[q] - mx);
      s += v[q];
    }
    s = rows_sum(s);
    const float inv = __builtin_amdgcn_rcpf(s);  // s >= 1 (the max term)
#pragma unroll
    for (int q = 0; q < 4 * MB; ++q) v[q] *= inv;
  } else {
    // SiLU(x) / ell
    constexpr float c = ELL * LOG2E;
#pragma unroll
    for (int q = 0; q < 4 * MB; ++q) v[q] = silu2_div(v[q], c);
  }
}

// cache_phi, then the store of the lane's links: bf16 weights, or int8
// codes plus the row's float32 scale.
template <int ELL, bool I8>
__device__ __forceinline__ void cache_epilogue(const floatx4 (&acc)[ELL / 16], float scale, int phi, int64_t item,
                                               int64_t n_items, int H, int head, void* __restrict__ cache_out,
                                               float* __restrict__ qscale, int g, int64_t item0,
                                               bf16_t* stage) {
  constexpr int MB = ELL / 16;
  float v[4 * MB];
  cache_phi<ELL>(acc, scale, phi, v);
  if constexpr (I8) {
    static_assert(MB % 2 == 0, "int8 codes leave in 8-byte pieces");
    uint32_t qv[MB];
    const float sc = quantize_i8<4 * MB>(v, qv);
    if (item < n_items) {
      int8_t* o = static_cast<int8_t*>(cache_out) + (item * H + head) * ELL + g * 4 * MB;
#pragma unroll
      for (int q = 0; q < MB / 2; ++q) *reinterpret_cast<uint2*>(o + 8 * q) = uint2{qv[2 * q], qv[2 * q + 1]};
      if (g == 0) qscale[item * H + head] = sc;
    }
  } else if constexpr (ELL == 64) {
    // One (item, head) row is 128 bytes, one memory line, of which this
    // lane holds 32 (links 16 g .. +16).  Written as they stand, each store
    // instruction would fill half of 16 lines; instead the 16 rows pass
    // through the wave's LDS area `stage` (16 rows, 72 bf16 apart), and each
    // store instruction then writes 8 whole lines: lane l stores piece l % 8
    // of row 8 s + l / 8 of the block.  (Within one wave: LDS accesses keep
    // their order, so no barrier is needed.)
    const int r = static_cast<int>(item - item0);
    st8(stage + r * 72 + g * 16, v);
    st8(stage + r * 72 + g * 16 + 8, v + 8);
    const int lane = 16 * g + r;
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) {
      const int row = 8 * s2 + (lane >> 3), piece = lane & 7;
      const bf16x8 o = *reinterpret_cast<const bf16x8*>(stage + row * 72 + piece * 8);
      const int64_t it = item0 + row;
      if (it < n_items)
        *reinterpret_cast<bf16x8*>(static_cast<bf16_t*>(cache_out) + (it * H + head) * ELL + piece * 8) = o;
    }
  } else {
    if (item < n_items) {
      bf16_t* o = static_cast<bf16_t*>(cache_out) + (item * H + head) * ELL + g * 4 * MB;
#pragma unroll
      for (int q = 0; q < MB / 2; ++q) st8(o + 8 * q, v + 8 * q);
    }
  }
}

template <int ELL, int D, int H, bool I8 = false>
__global__ __launch_bounds__((QkCfg<ELL, D, H, I8>::NT)) void qk_cache(
    const bf16_t* __restrict__ items, const bf16_t* __restrict__ keys, void* __restrict__ cache_out,
    float* __restrict__ qscale, int64_t n_items, float scale, int phi, int64_t ntiles) {
  using C = QkCfg<ELL, D, H, I8>;
  __shared__ __attribute__((aligned(16))) char lds[C::TI * C::STRIDE];
  // each wave's staging rows for line-sized output stores (ell = 64, bf16)
  constexpr int STG = (ELL == 64 && !I8) ? 16 * 72 : 8;
  __shared__ __attribute__((aligned(16))) bf16_t stage[C::NW * STG];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  bf16_t* const stage_w = stage + w * STG;
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
    lds_barrier();
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
        cache_epilogue<ELL, I8>(acc, scale, phi, item, n_items, H, head0 + hh, cache_out, qscale, g,
                                tile * C::TI + nb * 16, stage_w);
      }
    }
    lds_barrier();
  }
}

// The bf16 QK cache build with two item tiles in flight per workgroup: tiles
// travel global -> LDS by LDS-DMA loads (16 bytes per lane, no registers)
// into three buffers, so tiles t + 1 and t + 2 load while tile t is
// computed; one barrier per tile.  Rows are unpadded, with their 16-byte
// slots XOR-swizzled by the row's low bits, so that the 16 consecutive rows
// of a fragment read start their slot in 16 different bank groups.  Each tile has its
// own buffer descriptors for the item rows it reads and the cache rows it
// writes: rows past the catalogue load as 0 and their stores are dropped,
// so every wave issues the same loads and stores for every tile and the
// counted waits stay exact.  Products, phi and the order of the stored
// values are those of qk_cache.
template <int ELL, int D, int H>
struct QkDmaCfg {
  using C = QkCfg<ELL, D, H, false>;
  static constexpr int NBUF = 3;
  static constexpr int ROWB = D * 2;                            // bytes per item row
  static constexpr int TB = C::TI * ROWB;                       // bytes per tile
  static constexpr int SPR = ROWB / 16;                         // 16-byte slots per row
  static constexpr int LPT = TB / (16 * C::NT);                 // DMA loads per thread and tile
  static constexpr int OROWB = H * ELL * 2;                     // cache bytes per item
  // stores per wave and tile: two per (16-item block, head) at ell = 64
  // (whole lines through the wave's staging rows), MB / 2 otherwise
  static constexpr int SPW = C::NBW * C::HPW * (ELL == 64 ? 2 : C::MB / 2);
  static constexpr int STG = ELL == 64 ? 16 * 72 : 8;           // staging bf16 per wave
  static constexpr size_t lds_bytes = static_cast<size_t>(NBUF) * TB + static_cast<size_t>(C::NW) * STG * 2;
  static_assert(TB % (16 * C::NT) == 0, "tile load split");
  static_assert(2 * SPW + LPT < 64, "vmcnt");
};

__device__ __forceinline__ int qk_swz(int row, int spr) { return row & (spr < 16 ? spr - 1 : 15); }

template <int ELL, int D, int H>
__global__ __launch_bounds__((QkCfg<ELL, D, H, false>::NT)) void qk_cache_dma(
    const bf16_t* __restrict__ items, const bf16_t* __restrict__ keys, bf16_t* __restrict__ cache_out,
    int64_t n_items, float scale, int phi, int64_t ntiles) {
  using C = QkCfg<ELL, D, H, false>;
  using Q = QkDmaCfg<ELL, D, H>;
  extern __shared__ __attribute__((aligned(16))) char smem[];
  bf16_t* const stage = reinterpret_cast<bf16_t*>(smem + Q::NBUF * Q::TB);
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int wu = __builtin_amdgcn_readfirstlane(w);
  bf16_t* const stage_w = stage + w * Q::STG;
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

  // rows of tile t that exist (0 past the last tile)
  auto tile_rows = [&](int64_t t) {
    const int64_t left = n_items - t * C::TI;
    return left <= 0 ? 0 : (left < C::TI ? static_cast<int>(left) : C::TI);
  };
  // tile t into buffer b: load i of this thread fills slot e = i NT + tid
  // of the buffer (row e / SPR, swizzled slot e % SPR)
  auto issue_tile = [&](int64_t t, int b) {
    const int nrow = tile_rows(t);
    const __amdgpu_buffer_rsrc_t rs =
        bytes_rsrc(items + (nrow > 0 ? t * C::TI * D : 0), static_cast<uint32_t>(nrow) * Q::ROWB);
#pragma unroll
    for (int i = 0; i < Q::LPT; ++i) {
      const int e = i * C::NT + tid;
      const int row = e / Q::SPR, ps = e % Q::SPR;
      const unsigned vo = static_cast<unsigned>(row * Q::ROWB + (ps ^ qk_swz(row, Q::SPR)) * 16);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void_t*)(smem + b * Q::TB + (i * C::NT + wu * 64) * 16), 16,
                                               vo, 0, 0, 0);
    }
  };

  const int64_t G = gridDim.x;
  int64_t tile = blockIdx.x;
  issue_tile(tile, 0);
  issue_tile(tile + G, 1);
  int b = 0;
  for (int it = 0; tile < ntiles; tile += G, ++it) {
    // this tile's loads have landed: after them this wave issued the next
    // tile's loads and the stores of the previous two tiles (exact counts)
    if (it == 0) wait_vm<Q::LPT>();
    else if (it == 1) wait_vm<Q::LPT + Q::SPW>();
    else wait_vm<Q::LPT + 2 * Q::SPW>();
    dma_barrier();  // every wave's part of this tile; every wave has left tile - G's buffer
    issue_tile(tile + 2 * G, b == 0 ? 2 : b - 1);
    const char* const buf = smem + b * Q::TB;
    const int nrow = tile_rows(tile);
    const __amdgpu_buffer_rsrc_t ro =
        bytes_rsrc(cache_out + tile * C::TI * (H * ELL), static_cast<uint32_t>(nrow) * Q::OROWB);
#pragma unroll
    for (int nbi = 0; nbi < C::NBW; ++nbi) {
      const int nb = nb0 + nbi;
      const int row = nb * 16 + r;
      const int sw = qk_swz(row, Q::SPR);
      // all of the block's fragment reads in flight before its products
      bf16x8 bf[C::KB];
#pragma unroll
      for (int kb = 0; kb < C::KB; ++kb)
        bf[kb] = *reinterpret_cast<const bf16x8*>(buf + row * Q::ROWB + ((kb * 4 + g) ^ sw) * 16);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int hh = 0; hh < C::HPW; ++hh) {
        floatx4 acc[C::MB];
#pragma unroll
        for (int c = 0; c < C::MB; ++c) {
          acc[c] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int kb = 0; kb < C::KB; ++kb) acc[c] = mma(a[hh][c][kb], bf[kb], acc[c]);
        }
        float v[ELL / 4];
        cache_phi<ELL>(acc, scale, phi, v);
        const int head = head0 + hh;
        if constexpr (ELL == 64) {
          // whole 128-byte lines through the wave's staging rows (as in
          // qk_cache): lane l stores piece l % 8 of row 8 s + l / 8
          st8(stage_w + r * 72 + g * 16, v);
          st8(stage_w + r * 72 + g * 16 + 8, v + 8);
#pragma unroll
          for (int s2 = 0; s2 < 2; ++s2) {
            const int srow = 8 * s2 + (lane >> 3), piece = lane & 7;
            const bf16x8 o = *reinterpret_cast<const bf16x8*>(stage_w + srow * 72 + piece * 8);
            __builtin_amdgcn_raw_buffer_store_b128(
                __builtin_bit_cast(u32x4_t, o), ro,
                static_cast<unsigned>(((nb * 16 + srow) * H + head) * ELL * 2 + piece * 16), 0, 0);
          }
        } else {
#pragma unroll
          for (int q = 0; q < C::MB / 2; ++q) {
            bf16x8 o;
#pragma unroll
            for (int j = 0; j < 8; ++j) o[j] = static_cast<__bf16>(v[8 * q + j]);
            __builtin_amdgcn_raw_buffer_store_b128(
                __builtin_bit_cast(u32x4_t, o), ro,
                static_cast<unsigned>((row * H + head) * ELL * 2 + (g * 4 * C::MB + 8 * q) * 2), 0, 0);
          }
        }
      }
    }
    b = b == 2 ? 0 : b + 1;
  }
  // every wave's loads and stores finish before the workgroup exits (the
  // last two tiles' loads target no rows and move no data)
  wait_vm<0>();
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

// 8 int8 codes -> 8 bf16 values (exact: |code| <= 127)
__device__ __forceinline__ bf16x8 i8x8_to_bf16(uint2 pk) {
  bf16x8 o;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    o[j] = static_cast<__bf16>(static_cast<float>(static_cast<int8_t>((pk.x >> (8 * j)) & 0xff)));
    o[4 + j] = static_cast<__bf16>(static_cast<float>(static_cast<int8_t>((pk.y >> (8 * j)) & 0xff)));
  }
  return o;
}

template <int ELL, int H, bool I8 = false>
__global__ __launch_bounds__(256) void cand_score(const void* __restrict__ cache_in,
                                                  const float* __restrict__ qscale, int64_t n_items,
                                                  const bf16_t* __restrict__ lp,
                                                  const int64_t* __restrict__ ids,
                                                  const int64_t* __restrict__ off_g, int B,
                                                  int64_t total_M, bf16_t* __restrict__ out,
                                                  int* bad, int64_t tiles_per_wave) {
  using C = CsCfg<ELL, H>;
  constexpr int D = C::D, KB = C::KB;
  // a wave serves HG heads of its candidates: it holds the L^P operands of
  // those heads only, so large head counts do not exhaust the registers
  constexpr int HG = H < 4 ? H : 4, NG = H / HG;
  __shared__ int64_t off_s[C::MAXB + 1];
  // Output staging (HG >= 2): a candidate's HG heads are HG * 64 contiguous
  // bytes of its output row, whole memory lines, but each head's product
  // leaves a lane with 16 of them, so a store per head would fill each line
  // in pieces from separate instructions.  The tile's 16 rows are collected
  // in the wave's LDS rows (SROW bf16 apart) and stored in memory order,
  // 1 KB of whole lines per instruction, as many instructions as heads.
  constexpr bool STAGE = HG >= 2;
  constexpr int SROW = HG * 32 + 8;
  __shared__ __attribute__((aligned(16))) bf16_t stg_all[STAGE ? 4 * 16 * SROW : 8];
  const int tid = threadIdx.x, lane = tid & 63;
  const int g = lane >> 4, r = lane & 15;
  bf16_t* const stg = stg_all + (STAGE ? (tid >> 6) * 16 * SROW : 0);
  const bool in_lds = B <= C::MAXB;
  if (in_lds)
    for (int i = tid; i <= B; i += 256) off_s[i] = off_g[i];
  lds_barrier();
  const int64_t* off = in_lds ? off_s : off_g;

  const int64_t ntiles = (total_M + 15) >> 4;
  const int64_t gw_all = static_cast<int64_t>(blockIdx.x) * 4 + (tid >> 6);
  const int hg = static_cast<int>(gw_all % NG);
  const int64_t gw = gw_all / NG;
  const int hbase = hg * HG;
  const int64_t t0 = gw * tiles_per_wave;
  const int64_t t1 = t0 + tiles_per_wave < ntiles ? t0 + tiles_per_wave : ntiles;
  if (t0 >= t1) return;

  bf16x8 a[HG][2][KB];
  int cur = -1;
  int u = find_owner(off, B, t0 * 16);

  // Software pipeline over the wave's tiles (PIPE): the ids of tile t + 2
  // and the gathered cache rows of tile t + 1 are in flight while tile t is
  // computed (the row gather depends on the ids, so they go two stages).
  // It pays where the registers already limit occupancy (ell = 64) and for
  // the int8 rows; elsewhere the extra registers cost more waves than the
  // overlap gains.
  constexpr bool PIPE = I8 || ELL == 64;
  auto load_id = [&](int64_t t) -> int64_t {
    const int64_t i = t * 16 + r;
    return (t < t1 && i < total_M) ? ids[i] : int64_t(-1);
  };
  auto gather = [&](bf16x8 (&bw)[HG][KB], float (&qs)[HG], int64_t id, bool okid) {
#pragma unroll
    for (int hh = 0; hh < HG; ++hh) {
      const int h = hbase + hh;
      const int64_t idc = okid ? id : 0;
      if constexpr (I8) {
        const int8_t* row = static_cast<const int8_t*>(cache_in) + (idc * H + h) * ELL + 8 * g;
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
          bw[hh][kb] = okid ? i8x8_to_bf16(*reinterpret_cast<const uint2*>(row + kb * 32)) : zero8();
        qs[hh] = okid ? qscale[idc * H + h] : 0.f;
      } else {
        const bf16_t* row = static_cast<const bf16_t*>(cache_in) + (idc * H + h) * ELL + 8 * g;
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) bw[hh][kb] = okid ? ld16(row + kb * 32) : zero8();
        qs[hh] = 1.f;
      }
    }
  };
  auto in_range = [&](int64_t id) { return id >= 0 && id < n_items; };

  int64_t id_c = 0, id_n = 0;
  bool ok_c = false;
  bf16x8 bw_c[HG][KB];
  float qs_c[HG];
  if constexpr (PIPE) {
    id_c = load_id(t0);
    id_n = load_id(t0 + 1);
    ok_c = in_range(id_c);
    gather(bw_c, qs_c, id_c, ok_c);
  }

  for (int64_t t = t0; t < t1; ++t) {
    const int64_t i = t * 16 + r;
    const bool valid = i < total_M;
    bf16x8 bw_n[HG][KB];
    float qs_n[HG];
    int64_t id_nn = 0;
    bool ok_n = false;
    if constexpr (PIPE) {
      // next stages: ids of t + 2, rows of t + 1
      id_nn = load_id(t + 2);
      ok_n = in_range(id_n);
      gather(bw_n, qs_n, id_n, ok_n);
    } else {
      id_c = load_id(t);
      ok_c = in_range(id_c);
      gather(bw_c, qs_c, id_c, ok_c);
    }

    int ul = u;
    if (valid)
      while (ul + 1 < B && off[ul + 1] <= i) ++ul;
    if (valid && !ok_c && g == 0 && hg == 0 && bad != nullptr) atomicAdd(bad, 1);

    const int last = static_cast<int>((total_M - 1 - t * 16) < 15 ? (total_M - 1 - t * 16) : 15);
    const int ufirst = __shfl(ul, 0);
    const int ulast = __shfl(ul, last);
    for (int uu = ufirst; uu <= ulast; ++uu) {
      if (!__any(valid && ul == uu)) continue;
      if (uu != cur) {
        const bf16_t* lb = lp + static_cast<int64_t>(uu) * ELL * D;
#pragma unroll
        for (int hh = 0; hh < HG; ++hh)
#pragma unroll
          for (int c = 0; c < 2; ++c) {
            const int col = (hbase + hh) * 32 + 8 * (r >> 2) + 4 * c + (r & 3);
#pragma unroll
            for (int kb = 0; kb < KB; ++kb)
#pragma unroll
              for (int j = 0; j < 8; ++j)
                a[hh][c][kb][j] = __builtin_bit_cast(__bf16, lb[static_cast<int64_t>(kb * 32 + 8 * g + j) * D + col]);
          }
        cur = uu;
      }
      const bool mine = valid && ul == uu;
#pragma unroll
      for (int hh = 0; hh < HG; ++hh) {
        floatx4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
          acc0 = mma(a[hh][0][kb], bw_c[hh][kb], acc0);
          acc1 = mma(a[hh][1][kb], bw_c[hh][kb], acc1);
        }
        if (mine) {
          const float sc = qs_c[hh];
          const float v[8] = {acc0[0] * sc, acc0[1] * sc, acc0[2] * sc, acc0[3] * sc,
                              acc1[0] * sc, acc1[1] * sc, acc1[2] * sc, acc1[3] * sc};
          if constexpr (STAGE)
            st8(stg + r * SROW + hh * 32 + 8 * g, v);
          else
            st8_stream(out + i * D + (hbase + hh) * 32 + 8 * g, v);
        }
      }
    }
    if constexpr (STAGE) {
      // every valid row of the tile is staged (each belongs to one user);
      // store them in memory order: byte f = 1024 s + 16 lane of the tile's
      // 16 x HG * 64 bytes is row f / (HG * 64), byte f % (HG * 64) of it
#pragma unroll
      for (int s2 = 0; s2 < HG; ++s2) {
        const int f = 1024 * s2 + 16 * lane;
        const int row = f / (HG * 64), within = (f % (HG * 64)) / 2;
        const int64_t ir = t * 16 + row;
        const bf16x8 o = *reinterpret_cast<const bf16x8*>(stg + row * SROW + within);
        if (ir < total_M)
          __builtin_nontemporal_store(__builtin_bit_cast(u32x4_t, o),
                                      reinterpret_cast<u32x4_t*>(out + ir * D + hbase * 32 + within));
      }
    }
    u = __shfl(ul, last);
    if constexpr (PIPE) {
      // rotate the pipeline
#pragma unroll
      for (int hh = 0; hh < HG; ++hh) {
        qs_c[hh] = qs_n[hh];
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) bw_c[hh][kb] = bw_n[hh][kb];
      }
      ok_c = ok_n;
      id_n = id_nn;
    }
  }
}

// ---------------------------------------------------------------------------
// Uncached scoring (cold start), d_h = 32: per 16-candidate tile, gather the
// items' rows, logits S^T = K_h T^T (links x candidates) against link keys
// staged in LDS, phi over the links, then O^T = L^P_h^T P^T as in
// cand_score.  Link order of the score blocks: M-block c, row 4*g + j ->
// link (c/2)*32 + 8*g + 4*(c%2) + j, so the probabilities of each lane are
// the K slices of the value product's B operand.  A workgroup serves a
// group of HG heads (the grid's y dimension) whose keys it stages in LDS
// once, so every score product reads its key fragment from LDS; each head
// group gathers the candidates' rows itself and writes its own output
// columns.  Each wave walks its own range of tiles.
// ---------------------------------------------------------------------------
template <int ELL, int D, int H>
struct UcCfg {
  static constexpr int KB = D / 32, MB = ELL / 16, KBL = ELL / 32;
  static constexpr int LDK = D + 16;  // key row padded by 32 bytes (conflict-free fragment reads)
  // heads per workgroup: the most whose keys fit 144 KB of LDS; the head
  // groups are the grid's y dimension.  Keys over 72 KB leave one
  // workgroup per CU, which then has 8 waves instead of 4.
  static constexpr size_t KEYB = static_cast<size_t>(ELL) * LDK * 2;  // bytes per head
  static constexpr int HG = H * KEYB <= 144 * 1024 ? H : (H / 2) * KEYB <= 144 * 1024 ? H / 2 : H / 4;
  static constexpr int NHG = H / HG;
  static constexpr size_t lds_bytes = static_cast<size_t>(HG) * KEYB;
  static constexpr int NW = lds_bytes > 72 * 1024 ? 8 : 4, NT = 64 * NW;
  static_assert(D == 32 * H && ELL % 32 == 0, "shape");
  static_assert(H % HG == 0 && HG >= 1 && lds_bytes <= 144 * 1024, "head groups");
};

template <int ELL, int D, int H>
__global__ __launch_bounds__((UcCfg<ELL, D, H>::NT)) void cand_score_uncached(
    const bf16_t* __restrict__ items, int64_t n_items, const bf16_t* __restrict__ keys,
    const bf16_t* __restrict__ lp, const int64_t* __restrict__ ids, const int64_t* __restrict__ off,
    int B, int64_t total_M, bf16_t* __restrict__ out, int* bad, float scale, int phi,
    int64_t tiles_per_wave) {
  using C = UcCfg<ELL, D, H>;
  constexpr int KB = C::KB, MB = C::MB, KBL = C::KBL, LDK = C::LDK, HG = C::HG;
  extern __shared__ __attribute__((aligned(16))) char smem[];
  const int tid = threadIdx.x, lane = tid & 63;
  const int g = lane >> 4, r = lane & 15;
  // this workgroup's heads [h0, h0 + HG): their keys staged in LDS once
  const int h0 = static_cast<int>(blockIdx.y) * HG;
  {
    bf16_t* ks = reinterpret_cast<bf16_t*>(smem);
    const bf16_t* kg = keys + static_cast<int64_t>(h0) * ELL * D;
    for (int e = tid; e < HG * ELL * (D / 8); e += C::NT) {
      const int row = e / (D / 8), c8 = e % (D / 8);
      *reinterpret_cast<bf16x8*>(ks + row * LDK + 8 * c8) = ld16(kg + static_cast<int64_t>(row) * D + 8 * c8);
    }
    lds_barrier();
  }
  const bf16_t* const Ks = reinterpret_cast<const bf16_t*>(smem);
  const bool softmax = (phi == PHI_SOFTMAX);
  const float k2 = scale * LOG2E;
  const int64_t ntiles = (total_M + 15) >> 4;
  const int64_t gw = static_cast<int64_t>(blockIdx.x) * C::NW + (tid >> 6);
  const int64_t t0 = gw * tiles_per_wave;
  const int64_t t1 = t0 + tiles_per_wave < ntiles ? t0 + tiles_per_wave : ntiles;
  if (t0 >= t1) return;

  bf16x8 a[HG][2][KBL];
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
    if (valid && !okid && g == 0 && bad != nullptr && blockIdx.y == 0) atomicAdd(bad, 1);
    bf16x8 tb[KB];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) tb[kb] = okid ? ld16(items + id * D + kb * 32 + 8 * g) : zero8();

    // probabilities per head as B operands of the value product
    const bf16_t* Kt = Ks + opaque_zero();
    bf16x8 pb[HG][KBL];
#pragma unroll
    for (int h = 0; h < HG; ++h) {
      float v[4 * MB];
#pragma unroll
      for (int c = 0; c < MB; ++c) {
        const int link = (c >> 1) * 32 + 8 * (r >> 2) + 4 * (c & 1) + (r & 3);
        const bf16_t* kr = Kt + (h * ELL + link) * LDK + 8 * g;
        floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) acc = mma(ld16(kr + kb * 32), tb[kb], acc);
#pragma unroll
        for (int q = 0; q < 4; ++q) v[4 * c + q] = acc[q] * k2;  // log2 units
      }
      if (softmax) {
        float mx = v[0];
#pragma unroll
        for (int q = 1; q < 4 * MB; ++q) mx = fmaxf(mx, v[q]);
        mx = rows_max(mx);
        float sum = 0.f;
#pragma unroll
        for (int q = 0; q < 4 * MB; ++q) {
          v[q] = exp2_f(v[q] - mx);
          sum += v[q];
        }
        sum = rows_sum(sum);
        const float inv = __builtin_amdgcn_rcpf(sum);  // sum >= 1 (the max term)
#pragma unroll
        for (int q = 0; q < 4 * MB; ++q) v[q] *= inv;
      } else {
        constexpr float c = ELL * LOG2E;  // SiLU(x) / ell
#pragma unroll
        for (int q = 0; q < 4 * MB; ++q) v[q] = silu2_div(v[q], c);
      }
#pragma unroll
      for (int kb = 0; kb < KBL; ++kb) {
        bf16x8 o;
#pragma unroll
        for (int j = 0; j < 8; ++j) o[j] = static_cast<__bf16>(v[8 * kb + j]);
        pb[h][kb] = o;
      }
    }

    const int last = static_cast<int>((total_M - 1 - t * 16) < 15 ? (total_M - 1 - t * 16) : 15);
    const int ufirst = __shfl(ul, 0);
    const int ulast = __shfl(ul, last);
    for (int uu = ufirst; uu <= ulast; ++uu) {
      if (!__any(valid && ul == uu)) continue;
      if (uu != cur) {
        const bf16_t* lb = lp + static_cast<int64_t>(uu) * ELL * D;
#pragma unroll
        for (int h = 0; h < HG; ++h)
#pragma unroll
          for (int c = 0; c < 2; ++c) {
            const int col = (h0 + h) * 32 + 8 * (r >> 2) + 4 * c + (r & 3);
#pragma unroll
            for (int kb = 0; kb < KBL; ++kb)
#pragma unroll
              for (int j = 0; j < 8; ++j)
                a[h][c][kb][j] = __builtin_bit_cast(__bf16, lb[static_cast<int64_t>(kb * 32 + 8 * g + j) * D + col]);
          }
        cur = uu;
      }
      const bool mine = valid && ul == uu;
#pragma unroll
      for (int h = 0; h < HG; ++h) {
        floatx4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kb = 0; kb < KBL; ++kb) {
          acc0 = mma(a[h][0][kb], pb[h][kb], acc0);
          acc1 = mma(a[h][1][kb], pb[h][kb], acc1);
        }
        if (mine) {
          const float zf = okid ? 1.f : 0.f;  // out-of-range ids give zero rows
          const float v[8] = {acc0[0] * zf, acc0[1] * zf, acc0[2] * zf, acc0[3] * zf,
                              acc1[0] * zf, acc1[1] * zf, acc1[2] * zf, acc1[3] * zf};
          st8_stream(out + i * D + (h0 + h) * 32 + 8 * g, v);
        }
      }
    }
    u = __shfl(ul, last);
  }
}

}  // namespace mfma
}  // namespace lime

