// Shared device helpers for the gfx950 kernels (wave64, MFMA, fp16 bits).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ald {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef _Float16 v4h __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));

constexpr int WAVE = 64;

__device__ __forceinline__ float h2f(uint16_t b) {
  _Float16 h = __builtin_bit_cast(_Float16, b);
  return (float)h;
}
// round-to-nearest-even fp32 -> fp16
__device__ __forceinline__ uint16_t f2h(float f) {
  _Float16 h = (_Float16)f;
  return __builtin_bit_cast(uint16_t, h);
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, WAVE);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, WAVE));
  return v;
}

// 16-byte global load / store helpers
__device__ __forceinline__ v4i ld16(const void* p) { return *reinterpret_cast<const v4i*>(p); }
__device__ __forceinline__ void st16(void* p, v4i v) { *reinterpret_cast<v4i*>(p) = v; }

// symmetric int8 code of an fp32 value given the fp32 reciprocal 127/amax:
// one rounded product, then round-half-even, then clamp
__device__ __forceinline__ int q8_code(float u, float inv) {
  float p = u * inv;
  float r = __builtin_rintf(p);
  r = fminf(fmaxf(r, -127.0f), 127.0f);
  return (int)r;
}

__device__ __forceinline__ float gelu_erf(float x) {
  return 0.5f * x * (1.0f + erff(x * 0.70710678118654752f));
}

}  // namespace ald
