// Device helpers shared by the gfx950 kernels: bf16 conversion, vector
// types for 16-byte accesses and MFMA operands, wavefront reductions.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mmdit {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;

// A launch guarded by a step-cache flag does nothing when the flag (written
// on the device by the cache decision of an earlier kernel on the stream) is
// nonzero; a null guard always runs. Uniform across the grid, so a block
// returns whole, before any barrier.
__device__ __forceinline__ bool guard_skip(const int* g) { return g != nullptr && *g != 0; }

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16 x) { return (float)x; }

template <typename T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
// round to nearest even (v_cvt_pk_bf16_f32 on gfx950)
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float x) { return (bf16)x; }

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}

// sum across aligned groups of `width` lanes (width a power of two <= 64)
template <int width>
__device__ __forceinline__ float group_sum(float v) {
#pragma unroll
  for (int o = width / 2; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

// Load 8 consecutive values of T as float.
__device__ __forceinline__ void load8(const bf16* p, float* o) {
  bf16x8 v = *reinterpret_cast<const bf16x8*>(p);
#pragma unroll
  for (int i = 0; i < 8; ++i) o[i] = (float)v[i];
}
__device__ __forceinline__ void load8(const float* p, float* o) {
  f32x4 a = *reinterpret_cast<const f32x4*>(p);
  f32x4 b = *reinterpret_cast<const f32x4*>(p + 4);
#pragma unroll
  for (int i = 0; i < 4; ++i) { o[i] = a[i]; o[4 + i] = b[i]; }
}
__device__ __forceinline__ void store8(bf16* p, const float* v) {
  bf16x8 o;
#pragma unroll
  for (int i = 0; i < 8; ++i) o[i] = (bf16)v[i];
  *reinterpret_cast<bf16x8*>(p) = o;
}
__device__ __forceinline__ void store8(float* p, const float* v) {
  f32x4 a, b;
#pragma unroll
  for (int i = 0; i < 4; ++i) { a[i] = v[i]; b[i] = v[4 + i]; }
  *reinterpret_cast<f32x4*>(p) = a;
  *reinterpret_cast<f32x4*>(p + 4) = b;
}

// Load 4 consecutive values as float.
__device__ __forceinline__ void load4(const bf16* p, float* o) {
  bf16x4 v = *reinterpret_cast<const bf16x4*>(p);
#pragma unroll
  for (int i = 0; i < 4; ++i) o[i] = (float)v[i];
}
__device__ __forceinline__ void load4(const float* p, float* o) {
  f32x4 a = *reinterpret_cast<const f32x4*>(p);
#pragma unroll
  for (int i = 0; i < 4; ++i) o[i] = a[i];
}
__device__ __forceinline__ void store4(bf16* p, const float* v) {
  bf16x4 o;
#pragma unroll
  for (int i = 0; i < 4; ++i) o[i] = (bf16)v[i];
  *reinterpret_cast<bf16x4*>(p) = o;
}
__device__ __forceinline__ void store4(float* p, const float* v) {
  f32x4 a;
#pragma unroll
  for (int i = 0; i < 4; ++i) a[i] = v[i];
  *reinterpret_cast<f32x4*>(p) = a;
}

// SiLU and GELU-tanh. Precise = true uses the library
// expf (fp32 path); false uses the hardware exp2 (bf16 path, where the
// result is rounded to bf16 anyway).
template <bool Precise>
__device__ __forceinline__ float exp_f(float x) { return Precise ? expf(x) : __expf(x); }

template <bool Precise>
__device__ __forceinline__ float silu_f(float x) { return x / (1.0f + exp_f<Precise>(-x)); }

// GELU with the tanh approximation; tanh(u) is written 1 - 2 / (exp(2u) + 1)
// so it saturates cleanly at both ends.
template <bool Precise>
__device__ __forceinline__ float gelu_tanh_f(float x) {
  const float k0 = 0.7978845608028654f;  // sqrt(2/pi)
  const float k1 = 0.044715f;
  float u = k0 * (x + k1 * x * x * x);
  float t = 1.0f - 2.0f / (exp_f<Precise>(2.0f * u) + 1.0f);
  return 0.5f * x * (1.0f + t);
}

}  // namespace mmdit
