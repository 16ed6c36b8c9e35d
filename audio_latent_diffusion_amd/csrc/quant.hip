// Bandwidth-bound row kernels: per-token int8 quantization, fused LayerNorm
// (+ quantization), 4-bit weight packing.
//
// One wave (64 lanes) owns one row; the row is read once with 16-byte
// coalesced loads into registers, reduced with cross-lane shuffles, and
// written once.  Four rows per 256-thread workgroup.
#include "common.h"
#include "kernels.h"

namespace ald {

template <int NV>
struct RowRegs {
  v4i c[NV];  // chunk j of this lane covers elements (lane + 64 j) * 8 .. +8
};

template <int NV>
__device__ __forceinline__ void load_row(RowRegs<NV>& r, const uint16_t* row, int K, int lane) {
#pragma unroll
  for (int j = 0; j < NV; ++j) {
    int e = (lane + WAVE * j) * 8;
    if (e < K) r.c[j] = ld16(row + e);
    else r.c[j] = v4i{0, 0, 0, 0};
  }
}

__device__ __forceinline__ void unpack8(v4i c, float f[8]) {
  const uint16_t* h = reinterpret_cast<const uint16_t*>(&c);
#pragma unroll
  for (int i = 0; i < 8; ++i) f[i] = h2f(h[i]);
}

// codes of 8 fp16 values packed into two 32-bit words
__device__ __forceinline__ uint2 quant8(const float f[8], float inv) {
  uint32_t lo = 0, hi = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) lo |= (uint32_t)(q8_code(f[i], inv) & 0xFF) << (8 * i);
#pragma unroll
  for (int i = 0; i < 4; ++i) hi |= (uint32_t)(q8_code(f[4 + i], inv) & 0xFF) << (8 * i);
  return make_uint2(lo, hi);
}

// amax -> (scale, reciprocal); amax == 0 -> (0, 0) so every code is 0
__device__ __forceinline__ void q8_scale(float amax, float& s, float& inv) {
  if (amax > 0.0f) {
    s = amax / 127.0f;      // IEEE fp32 division (correctly rounded)
    inv = 127.0f / amax;
  } else {
    s = 0.0f;
    inv = 0.0f;
  }
}

template <int NV>
__global__ __launch_bounds__(256) void row_quant_kernel(const uint16_t* __restrict__ x, int64_t ldx, int M,
                                                        int K, int8_t* __restrict__ q, int64_t ldq,
                                                        float* __restrict__ scale) {
  const int lane = threadIdx.x & 63;
  const int m = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (m >= M) return;
  RowRegs<NV> r;
  load_row<NV>(r, x + (int64_t)m * ldx, K, lane);
  float amax = 0.0f;
#pragma unroll
  for (int j = 0; j < NV; ++j) {
    float f[8];
    unpack8(r.c[j], f);
#pragma unroll
    for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(f[i]));
  }
  amax = wave_max(amax);
  float s, inv;
  q8_scale(amax, s, inv);
  int8_t* qrow = q + (int64_t)m * ldq;
#pragma unroll
  for (int j = 0; j < NV; ++j) {
    int e = (lane + WAVE * j) * 8;
    if (e < K) {
      float f[8];
      unpack8(r.c[j], f);
      *reinterpret_cast<uint2*>(qrow + e) = quant8(f, inv);
    }
  }
  if (lane == 0) scale[m] = s;
}

// LayerNorm of one row held in registers; result rounded to fp16 in place
template <int NV>
__device__ __forceinline__ void layer_norm_regs(RowRegs<NV>& r, int H, int lane, const float* __restrict__ g,
                                                const float* __restrict__ b, float eps) {
  float sum = 0.0f;
#pragma unroll
  for (int j = 0; j < NV; ++j) {
    float f[8];
    unpack8(r.c[j], f);
#pragma unroll
    for (int i = 0; i < 8; ++i) sum += f[i];
  }
  const float mean = wave_sum(sum) / (float)H;
  float sq = 0.0f;
#pragma unroll
  for (int j = 0; j < NV; ++j) {
    int e = (lane + WAVE * j) * 8;
    if (e < H) {
      float f[8];
      unpack8(r.c[j], f);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        float d = f[i] - mean;
        sq += d * d;
      }
    }
  }
  const float var = wave_sum(sq) / (float)H;
  const float rstd = 1.0f / sqrtf(var + eps);
#pragma unroll
  for (int j = 0; j < NV; ++j) {
    int e = (lane + WAVE * j) * 8;
    if (e < H) {
      float f[8];
      unpack8(r.c[j], f);
      const float4 g0 = *reinterpret_cast<const float4*>(g + e);
      const float4 g1 = *reinterpret_cast<const float4*>(g + e + 4);
      const float4 b0 = *reinterpret_cast<const float4*>(b + e);
      const float4 b1 = *reinterpret_cast<const float4*>(b + e + 4);
      const float gg[8] = {g0.x, g0.y, g0.z, g0.w, g1.x, g1.y, g1.z, g1.w};
      const float bb[8] = {b0.x, b0.y, b0.z, b0.w, b1.x, b1.y, b1.z, b1.w};
      uint16_t* h = reinterpret_cast<uint16_t*>(&r.c[j]);
#pragma unroll
      for (int i = 0; i < 8; ++i) h[i] = f2h((f[i] - mean) * rstd * gg[i] + bb[i]);
    }
  }
}

template <int NV>
__global__ __launch_bounds__(256) void ln_quant_kernel(const uint16_t* __restrict__ x, int64_t ldx, int M, int H,
                                                       const float* __restrict__ g, const float* __restrict__ b,
                                                       float eps, uint16_t* __restrict__ u_out,
                                                       int8_t* __restrict__ q, float* __restrict__ scale) {
  const int lane = threadIdx.x & 63;
  const int m = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (m >= M) return;
  RowRegs<NV> r;
  load_row<NV>(r, x + (int64_t)m * ldx, H, lane);
  layer_norm_regs<NV>(r, H, lane, g, b, eps);
  float amax = 0.0f;
#pragma unroll
  for (int j = 0; j < NV; ++j) {
    float f[8];
    unpack8(r.c[j], f);  // padding chunks are zero
#pragma unroll
    for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(f[i]));
  }
  amax = wave_max(amax);
  float s, inv;
  q8_scale(amax, s, inv);
  int8_t* qrow = q + (int64_t)m * H;
  uint16_t* urow = u_out ? u_out + (int64_t)m * H : nullptr;
#pragma unroll
  for (int j = 0; j < NV; ++j) {
    int e = (lane + WAVE * j) * 8;
    if (e < H) {
      float f[8];
      unpack8(r.c[j], f);
      *reinterpret_cast<uint2*>(qrow + e) = quant8(f, inv);
      if (urow) st16(urow + e, r.c[j]);
    }
  }
  if (lane == 0) scale[m] = s;
}

template <int NV>
__global__ __launch_bounds__(256) void ln_f16_kernel(const uint16_t* __restrict__ x, int64_t ldx, int M, int H,
                                                     const float* __restrict__ g, const float* __restrict__ b,
                                                     float eps, uint16_t* __restrict__ y, int64_t ldy) {
  const int lane = threadIdx.x & 63;
  const int m = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (m >= M) return;
  RowRegs<NV> r;
  load_row<NV>(r, x + (int64_t)m * ldx, H, lane);
  layer_norm_regs<NV>(r, H, lane, g, b, eps);
  uint16_t* yrow = y + (int64_t)m * ldy;
#pragma unroll
  for (int j = 0; j < NV; ++j) {
    int e = (lane + WAVE * j) * 8;
    if (e < H) st16(yrow + e, r.c[j]);
  }
}

// one thread per group of 32 weights
__global__ __launch_bounds__(256) void q4_pack_kernel(const uint16_t* __restrict__ w, int64_t n_groups,
                                                      uint8_t* __restrict__ packed, uint16_t* __restrict__ scales) {
  const int64_t gi = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (gi >= n_groups) return;
  const uint16_t* src = w + gi * 32;
  v4i c[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) c[j] = ld16(src + 8 * j);
  float f[32];
#pragma unroll
  for (int j = 0; j < 4; ++j) unpack8(c[j], f + 8 * j);
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(f[i]));
  const uint16_t s16 = f2h(amax / 7.0f);
  const float s = h2f(s16);
  uint32_t words[4];
#pragma unroll
  for (int wd = 0; wd < 4; ++wd) {
    uint32_t v = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      int code = 0;
      if (s > 0.0f) {
        float r = __builtin_rintf(f[wd * 8 + i] / s);
        code = (int)fminf(fmaxf(r, -7.0f), 7.0f);
      }
      v |= (uint32_t)(code & 0xF) << (4 * i);
    }
    words[wd] = v;
  }
  *reinterpret_cast<uint4*>(packed + gi * 16) = make_uint4(words[0], words[1], words[2], words[3]);
  scales[gi] = s16;
}

// ---------------------------------------------------------------- launchers

#define ALD_ROW_DISPATCH(KERNEL, K, M, ST, ...)                                                      \
  do {                                                                                               \
    dim3 grid((unsigned)(((M) + 3) / 4)), block(256);                                                \
    int nv = ((K) + 511) / 512;                                                                      \
    if (nv <= 1) hipLaunchKernelGGL(KERNEL<1>, grid, block, 0, ST, __VA_ARGS__);                     \
    else if (nv <= 2) hipLaunchKernelGGL(KERNEL<2>, grid, block, 0, ST, __VA_ARGS__);                \
    else if (nv <= 4) hipLaunchKernelGGL(KERNEL<4>, grid, block, 0, ST, __VA_ARGS__);                \
    else if (nv <= 8) hipLaunchKernelGGL(KERNEL<8>, grid, block, 0, ST, __VA_ARGS__);                \
    else hipLaunchKernelGGL(KERNEL<16>, grid, block, 0, ST, __VA_ARGS__);                            \
  } while (0)

void launch_row_quant(const uint16_t* x, int64_t ldx, int M, int K, int8_t* q, int64_t ldq, float* scale,
                      hipStream_t st) {
  if (M <= 0) return;
  ALD_ROW_DISPATCH(row_quant_kernel, K, M, st, x, ldx, M, K, q, ldq, scale);
}

void launch_ln_quant(const uint16_t* x, int64_t ldx, int M, int H, const float* g, const float* b, float eps,
                     uint16_t* u_out, int8_t* q, float* scale, hipStream_t st) {
  if (M <= 0) return;
  ALD_ROW_DISPATCH(ln_quant_kernel, H, M, st, x, ldx, M, H, g, b, eps, u_out, q, scale);
}

void launch_ln_f16(const uint16_t* x, int64_t ldx, int M, int H, const float* g, const float* b, float eps,
                   uint16_t* y, int64_t ldy, hipStream_t st) {
  if (M <= 0) return;
  ALD_ROW_DISPATCH(ln_f16_kernel, H, M, st, x, ldx, M, H, g, b, eps, y, ldy);
}

void launch_q4_pack(const uint16_t* w, int N, int K, uint8_t* packed, uint16_t* scales, hipStream_t st) {
  int64_t groups = (int64_t)N * (K / 32);
  if (groups <= 0) return;
  hipLaunchKernelGGL(q4_pack_kernel, dim3((unsigned)((groups + 255) / 256)), dim3(256), 0, st, w, groups, packed,
                     scales);
}

}  // namespace ald
