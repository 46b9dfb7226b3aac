// Device-side helpers shared by the libhstu kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "../internal.h"

namespace hstu {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float bf2f(uint16_t b) { return __uint_as_float(uint32_t(b) << 16); }

// round to nearest even (lowers to v_cvt_pk_bf16_f32 on gfx950)
__device__ __forceinline__ uint16_t f2bf(float f) {
  __bf16 h = static_cast<__bf16>(f);
  return __builtin_bit_cast(uint16_t, h);
}

template <typename T>
struct Elem;
template <>
struct Elem<float> {
  static __device__ __forceinline__ float load(const float* p) { return *p; }
  static __device__ __forceinline__ void store(float* p, float v) { *p = v; }
};
template <>
struct Elem<uint16_t> {
  static __device__ __forceinline__ float load(const uint16_t* p) { return bf2f(*p); }
  static __device__ __forceinline__ void store(uint16_t* p, float v) { *p = f2bf(v); }
};

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

// Relative-position bucket floor(4 * log2(1 + delta)), exact for
// 0 <= delta < 65535: floor(4 log2 m) = floor(log2 m^4), the index of the
// highest set bit of m^4 (m = 1 + delta, m^4 < 2^64).  Sequence positions stay
// below 65535, so larger distances only arise for padding queries whose
// results are discarded; they are clamped so the table index stays in range.
__device__ __forceinline__ int rel_bucket(int delta, int num_buckets) {
  delta = delta < 0 ? 0 : (delta > 65534 ? 65534 : delta);
  uint64_t m = static_cast<uint64_t>(delta) + 1u;
  uint64_t p = m * m;
  p = p * p;
  int b = 63 - __clzll(static_cast<long long>(p));
  return b < num_buckets - 1 ? b : num_buckets - 1;
}

// SiLU(x) = x * sigmoid(x) with the hardware exp2 and reciprocal; exact
// limits: x -> -inf gives -0, x -> +inf gives x.
__device__ __forceinline__ float silu_fast(float x) {
  float e = __builtin_amdgcn_exp2f(x * -1.44269504088896340736f);
  return x * __builtin_amdgcn_rcpf(1.0f + e);
}

// first index u in [0, B) with off[u] <= r < off[u+1] (off nondecreasing)
__device__ __forceinline__ int find_segment(const int32_t* off, int B, int r) {
  int lo = 0, hi = B;  // off[lo] <= r < off[hi]
  while (hi - lo > 1) {
    int mid = (lo + hi) >> 1;
    if (off[mid] <= r) lo = mid; else hi = mid;
  }
  return lo;
}

}  // namespace hstu
