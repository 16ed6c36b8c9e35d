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

// Wave-wide reductions on DPP lane moves (no LDS round trips): butterflies
// inside each quad (quad_perm), each 8-lane half row and each 16-lane row
// (half-row and row mirrors) leave every lane with its row's result; then
// row_bcast:15 folds row 0 into row 1 and row 2 into row 3, row_bcast:31
// folds rows 0-1 into row 3, and lane 63 holds the wave's result.  Lanes a
// broadcast does not write keep `idle`, the operation's identity.
template <int CTRL, int ROWS>
__device__ __forceinline__ float dpp_mov(float idle, float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(__builtin_bit_cast(int, idle),
                                                               __builtin_bit_cast(int, v), CTRL, ROWS, 0xF, false));
}
__device__ __forceinline__ float lane63(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 63));
}
__device__ __forceinline__ float wave_sum(float v) {
  v += dpp_mov<0xB1, 0xF>(0.0f, v);   // quad_perm [1, 0, 3, 2]
  v += dpp_mov<0x4E, 0xF>(0.0f, v);   // quad_perm [2, 3, 0, 1]
  v += dpp_mov<0x141, 0xF>(0.0f, v);  // row_half_mirror
  v += dpp_mov<0x140, 0xF>(0.0f, v);  // row_mirror
  v += dpp_mov<0x142, 0xA>(0.0f, v);  // row_bcast:15 into rows 1 and 3
  v += dpp_mov<0x143, 0x8>(0.0f, v);  // row_bcast:31 into row 3
  return lane63(v);
}
// maximum of non-negative values (0 is the identity)
__device__ __forceinline__ float wave_max_nonneg(float v) {
  v = fmaxf(v, dpp_mov<0xB1, 0xF>(0.0f, v));
  v = fmaxf(v, dpp_mov<0x4E, 0xF>(0.0f, v));
  v = fmaxf(v, dpp_mov<0x141, 0xF>(0.0f, v));
  v = fmaxf(v, dpp_mov<0x140, 0xF>(0.0f, v));
  v = fmaxf(v, dpp_mov<0x142, 0xA>(0.0f, v));
  v = fmaxf(v, dpp_mov<0x143, 0x8>(0.0f, v));
  return lane63(v);
}

// 16-byte global load / store helpers
__device__ __forceinline__ v4i ld16(const void* p) { return *reinterpret_cast<const v4i*>(p); }
__device__ __forceinline__ void st16(void* p, v4i v) { *reinterpret_cast<v4i*>(p) = v; }

// Streaming (nontemporal) accesses for data a kernel touches once: on MI355X
// a read-modify-write stream reaches ~81% of HBM peak with nontemporal loads
// and stores against ~74% with ordinary ones (measured on 1 GiB buffers).
typedef int v2i __attribute__((ext_vector_type(2)));
__device__ __forceinline__ v4i ld16_nt(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const v4i*>(p));
}
__device__ __forceinline__ void st16_nt(void* p, v4i v) { __builtin_nontemporal_store(v, reinterpret_cast<v4i*>(p)); }
__device__ __forceinline__ v2i ld8_nt(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const v2i*>(p));
}
__device__ __forceinline__ void st8_nt(void* p, v2i v) { __builtin_nontemporal_store(v, reinterpret_cast<v2i*>(p)); }
__device__ __forceinline__ void st8(void* p, v2i v) { *reinterpret_cast<v2i*>(p) = v; }

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
