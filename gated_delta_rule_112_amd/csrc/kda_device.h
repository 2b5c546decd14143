// Device-side helpers shared by the KDA kernels (gfx950 / CDNA4 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kda {

typedef __bf16 bf16_t;
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));

// io element type traits: float32 or bfloat16 storage, float32 arithmetic.
template <typename T> struct io_traits;
template <> struct io_traits<float> {
  static __device__ __forceinline__ float to_f32(float x) { return x; }
  static __device__ __forceinline__ float from_f32(float x) { return x; }
};
template <> struct io_traits<bf16_t> {
  static __device__ __forceinline__ float to_f32(bf16_t x) { return (float)x; }
  static __device__ __forceinline__ bf16_t from_f32(float x) { return (bf16_t)x; }  // RNE
};

template <typename T> __device__ __forceinline__ float ld_f32(const T* p) {
  return io_traits<T>::to_f32(*p);
}
template <typename T> __device__ __forceinline__ void st_f32(T* p, float x) {
  *p = io_traits<T>::from_f32(x);
}

// Four consecutive io elements as float32 (p must be aligned to 4 elements).
__device__ __forceinline__ f32x4 ld4(const float* p) { return *(const f32x4*)p; }
__device__ __forceinline__ f32x4 ld4(const bf16_t* p) {
  bf16x4 v = *(const bf16x4*)p;
  return f32x4{(float)v[0], (float)v[1], (float)v[2], (float)v[3]};
}
__device__ __forceinline__ void st4(float* p, f32x4 x) { *(f32x4*)p = x; }
__device__ __forceinline__ void st4(bf16_t* p, f32x4 x) {
  bf16x4 v = {(bf16_t)x[0], (bf16_t)x[1], (bf16_t)x[2], (bf16_t)x[3]};
  *(bf16x4*)p = v;
}

__device__ __forceinline__ float sigmoidf_(float x) { return 1.0f / (1.0f + __expf(-x)); }

// Where the tokens of sequence b sit among the `total` token rows of a
// [rows, H, d] tensor: B sequences of T rows each (PACKED false, total = B T),
// or packed sequences occupying rows cu[b] .. cu[b + 1] - 1 (T is then the
// longest length).  Packed bounds are clamped into [0, total] and lengths to T,
// so every row index a kernel forms stays below `total` whatever cu holds.  A
// compile-time choice: the uniform layout keeps its plain arithmetic.
template <bool PACKED>
struct Seqs {
  const int* cu;
  int64_t T, total;

  __device__ __forceinline__ int64_t start(int64_t b) const {
    if constexpr (!PACKED) {
      return b * T;
    } else {
      const int64_t s = cu[b];
      return s < 0 ? 0 : (s > total ? total : s);
    }
  }
  __device__ __forceinline__ int64_t len(int64_t b) const {
    if constexpr (!PACKED) {
      return T;
    } else {
      const int64_t s = start(b);
      int64_t e = cu[b + 1];
      e = e < s ? s : (e > total ? total : e);
      return e - s < T ? e - s : T;
    }
  }
  // Row of token `tok` (>= 0) of sequence b, clamped into the sequence (into
  // the tensor when the sequence is empty).
  __device__ __forceinline__ int64_t row(int64_t b, int64_t tok) const {
    if constexpr (!PACKED) {
      return b * T + (tok < T ? tok : T - 1);
    } else {
      const int64_t n = len(b);
      const int64_t r = start(b) + (tok < n ? tok : n - 1);
      return r < 0 ? 0 : (r >= total ? total - 1 : r);
    }
  }
};

}  // namespace kda
