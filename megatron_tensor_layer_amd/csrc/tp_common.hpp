// Common types and device helpers for the gfx950 kernels of libtplayer.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tpl {

typedef uint16_t bf16_t;  // bfloat16 storage (upper half of an fp32)

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf2f(bf16_t x) { return __uint_as_float((uint32_t)x << 16); }

// round-to-nearest-even through the hardware converter (v_cvt_pk_bf16_f32)
__device__ __forceinline__ bf16_t f2bf(float f) {
  __bf16 b = (__bf16)f;
  return __builtin_bit_cast(bf16_t, b);
}

// Element traits: load / store 4 (or 8) consecutive elements as fp32.
template <typename T> struct Elt;

template <> struct Elt<float> {
  static constexpr int VEC = 4;  // elements per 16-byte chunk
  __device__ static __forceinline__ void load4(const float* p, float v[4]) {
    f32x4_t x = *reinterpret_cast<const f32x4_t*>(p);
    v[0] = x[0]; v[1] = x[1]; v[2] = x[2]; v[3] = x[3];
  }
  __device__ static __forceinline__ void store4(float* p, const float v[4]) {
    f32x4_t x = {v[0], v[1], v[2], v[3]};
    *reinterpret_cast<f32x4_t*>(p) = x;
  }
  __device__ static __forceinline__ void load8(const float* p, float v[8]) { load4(p, v); load4(p + 4, v + 4); }
  __device__ static __forceinline__ void store8(float* p, const float v[8]) { store4(p, v); store4(p + 4, v + 4); }
  __device__ static __forceinline__ float ld(const float* p) { return *p; }
  __device__ static __forceinline__ void st(float* p, float v) { *p = v; }
};

template <> struct Elt<bf16_t> {
  static constexpr int VEC = 8;
  __device__ static __forceinline__ void load4(const bf16_t* p, float v[4]) {
    uint2 u = *reinterpret_cast<const uint2*>(p);
    v[0] = __uint_as_float(u.x << 16); v[1] = __uint_as_float(u.x & 0xFFFF0000u);
    v[2] = __uint_as_float(u.y << 16); v[3] = __uint_as_float(u.y & 0xFFFF0000u);
  }
  __device__ static __forceinline__ void store4(bf16_t* p, const float v[4]) {
    f32x4_t x = {v[0], v[1], v[2], v[3]};
    bf16x4_t b = __builtin_convertvector(x, bf16x4_t);
    *reinterpret_cast<bf16x4_t*>(p) = b;
  }
  __device__ static __forceinline__ void load8(const bf16_t* p, float v[8]) {
    const uint4 u = *reinterpret_cast<const uint4*>(p);
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      v[2 * q] = __uint_as_float(w[q] << 16);
      v[2 * q + 1] = __uint_as_float(w[q] & 0xFFFF0000u);
    }
  }
  __device__ static __forceinline__ void store8(bf16_t* p, const float v[8]) {
    f32x4_t x = {v[0], v[1], v[2], v[3]}, y = {v[4], v[5], v[6], v[7]};
    const bf16x4_t a = __builtin_convertvector(x, bf16x4_t), b = __builtin_convertvector(y, bf16x4_t);
    const bf16x8_t c = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
    *reinterpret_cast<bf16x8_t*>(p) = c;
  }
  __device__ static __forceinline__ float ld(const bf16_t* p) { return bf2f(*p); }
  __device__ static __forceinline__ void st(bf16_t* p, float v) { *p = f2bf(v); }
};

// GELU(x) = x Phi(x) (erf form) and GELU'(x) = Phi(x) + x phi(x) in fp32,
// branch-free. Phi from the rational approximation of erfc in Abramowitz &
// Stegun, Handbook of Mathematical Functions, formula 7.1.26 (|error| of erf
// <= 1.5e-7): with z = |x|/sqrt(2) and t = 1/(1 + p z),
// erfc(z) = t (a1 + t (a2 + t (a3 + t (a4 + t a5)))) exp(-z^2), and
// exp(-z^2) = exp(-x^2/2) is also phi(x) sqrt(2 pi). The small tail Phi(-|x|)
// is formed directly, without the cancellation of 1 + erf(x/sqrt(2)).
// (An erff call branches on |x| per element.)
struct NormalCdf {
  float cdf, e;  // Phi(x) and exp(-x^2/2)
};
__device__ __forceinline__ NormalCdf normal_cdf(float x) {
  const float z = fabsf(x) * 0.70710678118654752f;
  const float t = __builtin_amdgcn_rcpf(__builtin_fmaf(0.3275911f, z, 1.0f));
  float q = __builtin_fmaf(t, 1.061405429f, -1.453152027f);
  q = __builtin_fmaf(t, q, 1.421413741f);
  q = __builtin_fmaf(t, q, -0.284496736f);
  q = __builtin_fmaf(t, q, 0.254829592f);
  const float e = __builtin_amdgcn_exp2f(-0.72134752044448170f * x * x);  // exp(-x^2/2) = 2^(-x^2 log2(e)/2)
  const float tail = 0.5f * t * q * e;                                     // Phi(-|x|)
  return {x >= 0.0f ? 1.0f - tail : tail, e};
}
__device__ __forceinline__ float gelu_f(float x) { return x * normal_cdf(x).cdf; }
__device__ __forceinline__ float gelu_grad_f(float x) {
  const NormalCdf n = normal_cdf(x);
  return __builtin_fmaf(x * 0.39894228040143268f, n.e, n.cdf);
}

// V consecutive elements (V = 4 or 8) as fp32.
template <typename T, int V>
__device__ __forceinline__ void loadv(const T* p, float v[V]) {
  if constexpr (V == 8) Elt<T>::load8(p, v);
  else Elt<T>::load4(p, v);
}
template <typename T, int V>
__device__ __forceinline__ void storev(T* p, const float v[V]) {
  if constexpr (V == 8) Elt<T>::store8(p, v);
  else Elt<T>::store4(p, v);
}

__host__ __device__ constexpr inline int cdiv(int a, int b) { return (a + b - 1) / b; }
__host__ __device__ constexpr inline long cdivl(long a, long b) { return (a + b - 1) / b; }

}  // namespace tpl
