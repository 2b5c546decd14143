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

}  // namespace kda
