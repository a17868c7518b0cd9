// Shared device helpers: storage types, conversions, row sources.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lime {

using bf16_t = uint16_t;  // bfloat16 bit pattern in memory

__device__ __forceinline__ float bf16_to_f32(bf16_t v) {
  return __uint_as_float(static_cast<uint32_t>(v) << 16);
}

// float -> bfloat16, round to nearest, ties to even (hardware conversion).
__device__ __forceinline__ bf16_t f32_to_bf16(float f) {
  return __builtin_bit_cast(bf16_t, static_cast<__bf16>(f));
}

template <typename T> struct Elt;
template <> struct Elt<float> {
  static __device__ __forceinline__ float ld(const float* p) { return *p; }
  static __device__ __forceinline__ void st(float* p, float v) { *p = v; }
};
template <> struct Elt<bf16_t> {
  static __device__ __forceinline__ float ld(const bf16_t* p) { return bf16_to_f32(*p); }
  static __device__ __forceinline__ void st(bf16_t* p, float v) { *p = f32_to_bf16(v); }
};

// A matrix whose rows come from two buffers: rows [0, split) from `a`,
// rows [split, ...) from `b` (row r - split).  Used so that the first layer
// reads the caller's links and history in place and the last layer writes
// the caller's outputs in place.  A null `b` on a destination drops those
// rows.
struct Rows {
  void* a;
  void* b;
  int64_t split;
  int64_t ld;  // elements per row
};

template <typename T>
__device__ __forceinline__ const T* row_in(const Rows& s, int64_t r) {
  return r < s.split ? static_cast<const T*>(s.a) + r * s.ld
                     : static_cast<const T*>(s.b) + (r - s.split) * s.ld;
}

template <typename T>
__device__ __forceinline__ T* row_out(const Rows& s, int64_t r) {
  if (r < s.split) return static_cast<T*>(s.a) + r * s.ld;
  if (s.b == nullptr) return nullptr;
  return static_cast<T*>(s.b) + (r - s.split) * s.ld;
}

// SiLU(x) = x * sigmoid(x) with the hardware reciprocal (about 1 ulp) in
// place of an IEEE division; exp(-x) = inf gives -0, exp(-x) = 0 gives x.
__device__ __forceinline__ float silu_f(float x) {
  return x * __builtin_amdgcn_rcpf(1.0f + __expf(-x));
}

__device__ __forceinline__ int64_t clamp64(int64_t v, int64_t lo, int64_t hi) {
  return v < lo ? lo : (v > hi ? hi : v);
}

// Largest b in [0, B) with off[b] <= i (off non-decreasing), i.e. the user
// that owns position i.
__device__ __forceinline__ int find_owner(const int64_t* off, int B, int64_t i) {
  int lo = 0, hi = B - 1;
  while (lo < hi) {
    int mid = (lo + hi + 1) >> 1;
    if (off[mid] <= i) lo = mid; else hi = mid - 1;
  }
  return lo;
}

enum : int { PHI_SOFTMAX = 0, PHI_SILU_MEAN = 1 };

}  // namespace lime
