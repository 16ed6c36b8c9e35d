// Bandwidth-bound row kernels: per-token int8 quantization, fused LayerNorm
// (+ quantization), 4-bit weight packing.
//
// One wave (64 lanes) owns one row at a time; the row is read once with
// 16-byte coalesced loads into registers, reduced with DPP lane moves, and
// written once.  Four waves per 256-thread workgroup; the grid is capped near
// what the chip keeps resident and each wave walks rows with the grid's
// stride, loading its next row before it reduces the current one, so the
// loads of one row overlap the reductions and stores of the previous.
#include <algorithm>

#include "common.h"
#include "kernels.h"

namespace ald {

template <int NV>
struct RowRegs {
  v4i c[NV];  // chunk j of this lane covers elements (lane + 64 j) * 8 .. +8
};

// Cache hints of the row kernels (CACHED: ordinary accesses where the next
// kernel reads the data again).  In the step, the int8 codes a quantizer
// writes are read at once by the next GEMM, and the residual stream that
// LayerNorm reads is read again by the next projection's residual epilogue.
// While a launch's data (2 B read and 1 B written per element) fits the
// 256 MB last-level cache, ordinary accesses leave it there for that reader:
// the serving step (8192 rows) ran 2.4 % faster with ordinary code stores and
// 1.1 % faster with ordinary LayerNorm loads (MI355X, same-box A/B).  Beyond
// the cache they only cost bandwidth (262144 x 1536 LayerNorm + quantize
// 75 -> 71 % of HBM, 65536 x 6144 quantize 79 -> 69 %), so larger launches
// keep the non-temporal hints.  Activations read once keep non-temporal
// loads.  The choice is a template parameter: as a run-time condition the
// compiler merged the two accesses and dropped the non-temporal hint.
inline bool fits_llc(int64_t M, int64_t K) { return 3 * M * K <= (int64_t(256) << 20); }

// NT: non-temporal loads
template <int NV, bool NT = true>
__device__ __forceinline__ void load_row(RowRegs<NV>& r, const uint16_t* row, int K, int lane) {
#pragma unroll
  for (int j = 0; j < NV; ++j) {
    int e = (lane + WAVE * j) * 8;
    if (e < K) r.c[j] = NT ? ld16_nt(row + e) : ld16(row + e);
    else r.c[j] = v4i{0, 0, 0, 0};
  }
}

__device__ __forceinline__ void unpack8(v4i c, float f[8]) {
  const uint16_t* h = reinterpret_cast<const uint16_t*>(&c);
#pragma unroll
  for (int i = 0; i < 8; ++i) f[i] = h2f(h[i]);
}

// Codes are packed 8 to two 32-bit words.  Each code is the round-half-even
// of the rounded fp32 product u * inv; adding 1.5 * 2^23 performs that
// rounding and leaves the code, in two's complement, in the low byte of the
// sum's bits.  No clamp is needed: every u of the row has |u| <= amax and
// inv = fp32(127 / amax), so |fp32(u * inv)| <= 127 (1 + 2^-24)^2 < 127.5 and
// the code stays within [-127, 127].  The product and the add are kept apart
// (the product is rounded first).
__device__ __forceinline__ uint32_t pack4_codes(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
  const uint32_t lo = __builtin_amdgcn_perm(b, a, 0x0C0C0400u);  // a.byte0, b.byte0, 0, 0
  const uint32_t hi = __builtin_amdgcn_perm(d, c, 0x0C0C0400u);
  return lo | (hi << 16);
}
// codes of 8 fp16 values: each product u * inv is formed straight from the
// fp16 operand (a mixed-precision fused multiply-add with a zero addend,
// v_fma_mix_f32: the exact product rounded once to fp32, the same value as
// converting u first and multiplying), then the add
__device__ __forceinline__ v2i quant8_h(v4i c, float inv) {
  const uint16_t* h = reinterpret_cast<const uint16_t*>(&c);
  uint32_t q[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float p = __builtin_fmaf(h2f(h[i]), inv, 0.0f);
    q[i] = __builtin_bit_cast(uint32_t, p + 12582912.0f);
  }
  return v2i{(int)pack4_codes(q[0], q[1], q[2], q[3]), (int)pack4_codes(q[4], q[5], q[6], q[7])};
}

// max |u| over 8 packed fp16 values, folded into a pair of 16-bit maxima:
// for finite fp16 the magnitude bits order like the magnitudes, so the max
// of (bits & 0x7FFF) is the bit pattern of the largest |u|, exactly
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ u16x2 absmax8_h(u16x2 acc, v4i c) {
  const uint32_t* w = reinterpret_cast<const uint32_t*>(&c);
#pragma unroll
  for (int k = 0; k < 4; ++k) acc = __builtin_elementwise_max(acc, __builtin_bit_cast(u16x2, w[k] & 0x7FFF7FFFu));
  return acc;
}

// max of a non-negative integer over the wave (the DPP pattern of wave_sum)
template <int CTRL, int ROWS>
__device__ __forceinline__ uint32_t dpp_mov_u(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, ROWS, 0xF, false);
}
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = max(v, dpp_mov_u<0xB1, 0xF>(v));
  v = max(v, dpp_mov_u<0x4E, 0xF>(v));
  v = max(v, dpp_mov_u<0x141, 0xF>(v));
  v = max(v, dpp_mov_u<0x140, 0xF>(v));
  v = max(v, dpp_mov_u<0x142, 0xA>(v));
  v = max(v, dpp_mov_u<0x143, 0x8>(v));
  return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}

// amax of a row from its lanes' 16-bit maxima, as fp32
__device__ __forceinline__ float row_absmax(u16x2 acc) {
  return h2f((uint16_t)wave_max_u32(max((uint32_t)acc.x, (uint32_t)acc.y)));
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

// codes and scale of one row held in registers (no conversion of the row to
// fp32: the amax from the fp16 bits, the products from fp16 operands)
template <int NV, bool FULL, bool CACHED>
__device__ __forceinline__ void quant_row_regs(const RowRegs<NV>& r, int K, int lane, int8_t* __restrict__ qrow,
                                               float* __restrict__ scale_m) {
  u16x2 acc = {0, 0};
#pragma unroll
  for (int j = 0; j < NV; ++j) acc = absmax8_h(acc, r.c[j]);  // padding chunks are zero
  float s, inv;
  q8_scale(row_absmax(acc), s, inv);
#pragma unroll
  for (int j = 0; j < NV; ++j) {
    const int e = (lane + WAVE * j) * 8;
    if (FULL || e < K) {
      if constexpr (CACHED) st8(qrow + e, quant8_h(r.c[j], inv));  // read next by the GEMM
      else st8_nt(qrow + e, quant8_h(r.c[j], inv));
    }
  }
  if (lane == 0) *scale_m = s;
}

// rows of up to 6 x 512 values prefetch the next row; longer rows already
// keep NV 16-byte loads per lane in flight and need the registers
template <int NV, bool FULL, bool CACHED>
__global__ __launch_bounds__(256) void row_quant_kernel(const uint16_t* __restrict__ x, int64_t ldx, int M,
                                                        int K, int8_t* __restrict__ q, int64_t ldq,
                                                        float* __restrict__ scale) {
  constexpr bool PREFETCH = NV <= 6;
  const int lane = threadIdx.x & 63;
  const int stride = gridDim.x * 4;
  int m = blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform per wave
  if (m >= M) return;
  RowRegs<NV> r;
  load_row<NV>(r, x + (int64_t)m * ldx, K, lane);
  for (;;) {
    const int mn = m + stride;
    RowRegs<NV> nx;
    if (PREFETCH && mn < M) load_row<NV>(nx, x + (int64_t)mn * ldx, K, lane);
    quant_row_regs<NV, FULL, CACHED>(r, K, lane, q + (int64_t)m * ldq, scale + m);
    if (mn >= M) break;
    if (PREFETCH) r = nx;
    else load_row<NV>(r, x + (int64_t)mn * ldx, K, lane);
    m = mn;
  }
}

// LayerNorm of one row held in registers (FULL: every chunk lies inside the
// row): statistics in fp32 (the sum as pairwise sums of the fp16 values, the
// square sums in two chains per chunk, so no long dependent chain sits
// between the row's loads and its reductions), output rounded to fp16 into
// `out` (which may be `r` itself: r is read only before the first write).
template <int NV, bool FULL>
__device__ __forceinline__ void layer_norm_row(const RowRegs<NV>& r, int H, int lane, const float* __restrict__ g,
                                               const float* __restrict__ b, float eps, RowRegs<NV>& out) {
  float sum = 0.0f;
#pragma unroll
  for (int j = 0; j < NV; ++j) {  // padding chunks are zero
    const uint32_t* w = reinterpret_cast<const uint32_t*>(&r.c[j]);
    float p[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) p[k] = h2f((uint16_t)(w[k] & 0xFFFFu)) + h2f((uint16_t)(w[k] >> 16));
    sum += (p[0] + p[1]) + (p[2] + p[3]);
  }
  const float inv_h = 1.0f / (float)H;  // loop-invariant: hoisted out of the row loop
  const float mean = wave_sum(sum) * inv_h;
  float d[NV][8];
  float sq = 0.0f;
#pragma unroll
  for (int j = 0; j < NV; ++j) {
    const int e = (lane + WAVE * j) * 8;
    if (FULL || e < H) {
      const uint16_t* h = reinterpret_cast<const uint16_t*>(&r.c[j]);
      float s0 = 0.0f, s1 = 0.0f;
#pragma unroll
      for (int i = 0; i < 8; i += 2) {
        d[j][i] = h2f(h[i]) - mean;
        d[j][i + 1] = h2f(h[i + 1]) - mean;
        s0 = fmaf(d[j][i], d[j][i], s0);
        s1 = fmaf(d[j][i + 1], d[j][i + 1], s1);
      }
      sq += s0 + s1;
    }
  }
  const float var = wave_sum(sq) * inv_h;
  const float rstd = __builtin_amdgcn_rsqf(var + eps);  // hardware 1/sqrt (1 ulp)
#pragma unroll
  for (int j = 0; j < NV; ++j) {
    const int e = (lane + WAVE * j) * 8;
    if (FULL || e < H) {
      const float4 g0 = *reinterpret_cast<const float4*>(g + e);
      const float4 g1 = *reinterpret_cast<const float4*>(g + e + 4);
      const float4 b0 = *reinterpret_cast<const float4*>(b + e);
      const float4 b1 = *reinterpret_cast<const float4*>(b + e + 4);
      const float gg[8] = {g0.x, g0.y, g0.z, g0.w, g1.x, g1.y, g1.z, g1.w};
      const float bb[8] = {b0.x, b0.y, b0.z, b0.w, b1.x, b1.y, b1.z, b1.w};
      uint16_t* h = reinterpret_cast<uint16_t*>(&out.c[j]);
#pragma unroll
      for (int i = 0; i < 8; ++i) h[i] = f2h(fmaf(d[j][i] * rstd, gg[i], bb[i]));
    }
  }
}

template <int NV, bool FULL, bool CACHED>
__global__ __launch_bounds__(256) void ln_quant_kernel(const uint16_t* __restrict__ x, int64_t ldx, int M, int H,
                                                       const float* __restrict__ g, const float* __restrict__ b,
                                                       float eps, uint16_t* __restrict__ u_out,
                                                       int8_t* __restrict__ q, float* __restrict__ scale) {
  constexpr bool PREFETCH = NV <= 6;
  const int lane = threadIdx.x & 63;
  const int stride = gridDim.x * 4;
  int m = blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform per wave
  if (m >= M) return;
  RowRegs<NV> r;
  load_row<NV, !CACHED>(r, x + (int64_t)m * ldx, H, lane);
  for (;;) {
    const int mn = m + stride;
    RowRegs<NV> nx;
    if (PREFETCH && mn < M) load_row<NV, !CACHED>(nx, x + (int64_t)mn * ldx, H, lane);
    RowRegs<NV>& y = r;  // the normalized row replaces the input row
    layer_norm_row<NV, FULL>(r, H, lane, g, b, eps, y);
    // the quantizer reads the fp16 LayerNorm output
    u16x2 acc = {0, 0};
#pragma unroll
    for (int j = 0; j < NV; ++j) {
      const int e = (lane + WAVE * j) * 8;
      if (FULL || e < H) acc = absmax8_h(acc, y.c[j]);
    }
    float s, inv;
    q8_scale(row_absmax(acc), s, inv);
    int8_t* qrow = q + (int64_t)m * H;
    uint16_t* urow = u_out ? u_out + (int64_t)m * H : nullptr;
#pragma unroll
    for (int j = 0; j < NV; ++j) {
      const int e = (lane + WAVE * j) * 8;
      if (FULL || e < H) {
        if constexpr (CACHED) st8(qrow + e, quant8_h(y.c[j], inv));  // read next by the GEMM
        else st8_nt(qrow + e, quant8_h(y.c[j], inv));
        if (urow) st16_nt(urow + e, y.c[j]);
      }
    }
    if (lane == 0) scale[m] = s;
    if (mn >= M) break;
    if (PREFETCH) r = nx;
    else load_row<NV, !CACHED>(r, x + (int64_t)mn * ldx, H, lane);
    m = mn;
  }
}

template <int NV, bool FULL, bool CACHED>
__global__ __launch_bounds__(256) void ln_f16_kernel(const uint16_t* __restrict__ x, int64_t ldx, int M, int H,
                                                     const float* __restrict__ g, const float* __restrict__ b,
                                                     float eps, uint16_t* __restrict__ y, int64_t ldy) {
  constexpr bool PREFETCH = NV <= 6;
  const int lane = threadIdx.x & 63;
  const int stride = gridDim.x * 4;
  int m = blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform per wave
  if (m >= M) return;
  RowRegs<NV> r;
  load_row<NV, !CACHED>(r, x + (int64_t)m * ldx, H, lane);
  for (;;) {
    const int mn = m + stride;
    RowRegs<NV> nx;
    if (PREFETCH && mn < M) load_row<NV, !CACHED>(nx, x + (int64_t)mn * ldx, H, lane);
    RowRegs<NV>& o = r;  // the normalized row replaces the input row
    layer_norm_row<NV, FULL>(r, H, lane, g, b, eps, o);
    uint16_t* yrow = y + (int64_t)m * ldy;
#pragma unroll
    for (int j = 0; j < NV; ++j) {
      const int e = (lane + WAVE * j) * 8;
      if (FULL || e < H) st16_nt(yrow + e, o.c[j]);
    }
    if (mn >= M) break;
    if (PREFETCH) r = nx;
    else load_row<NV, !CACHED>(r, x + (int64_t)mn * ldx, H, lane);
    m = mn;
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

// at most this many 4-row workgroups (each wave then walks 4 or more rows on
// the large shapes, with the next row's loads in flight): on 262144 rows of
// 1536 and 65536 rows of 6144 this measured faster than 2048 or 8192 (the
// activation quantization 73 -> 78 % of HBM bandwidth) and than one row per
// wave (LayerNorm + quantization 63 -> 53 %)
constexpr int64_t ROW_GRID_CAP = 16384;

// workgroups of a row kernel over M rows: one row per wave up to the cap, or,
// with `two_rows` (LayerNorm + quantization, whose reductions leave the load
// path idle longer), two rows per wave once one per wave would take more
// than 1024 workgroups: 8192 rows of 1536 take 9.1 us instead of 10.1 us, 8192
// rows of 2048 11.5 us instead of 12.7 (MI355X)
inline unsigned row_grid(int64_t M, bool two_rows) {
  const int64_t one = (M + 3) / 4;
  if (!two_rows || one <= 1024) return (unsigned)std::min(one, ROW_GRID_CAP);
  return (unsigned)std::min(std::max<int64_t>((M + 7) / 8, 1024), ROW_GRID_CAP);
}

#define ALD_ROW_LAUNCH(KERNEL, C, NV, K, GRID, ST, ...)                                              \
  do {                                                                                               \
    if ((K) == (NV) * 512) hipLaunchKernelGGL((KERNEL<NV, true, C>), GRID, dim3(256), 0, ST, __VA_ARGS__); \
    else hipLaunchKernelGGL((KERNEL<NV, false, C>), GRID, dim3(256), 0, ST, __VA_ARGS__);            \
  } while (0)

// one wave per row: NV 16-byte chunks per lane cover K values (NV * 512 >= K)
#define ALD_ROW_DISPATCH(KERNEL, C, K, M, TWO, ST, ...)                                              \
  do {                                                                                               \
    dim3 grid_(row_grid((M), (TWO)));                                                                \
    const int nv_ = ((K) + 511) / 512;                                                               \
    if (nv_ <= 1) ALD_ROW_LAUNCH(KERNEL, C, 1, K, grid_, ST, __VA_ARGS__);                           \
    else if (nv_ <= 2) ALD_ROW_LAUNCH(KERNEL, C, 2, K, grid_, ST, __VA_ARGS__);                      \
    else if (nv_ <= 3) ALD_ROW_LAUNCH(KERNEL, C, 3, K, grid_, ST, __VA_ARGS__);                      \
    else if (nv_ <= 4) ALD_ROW_LAUNCH(KERNEL, C, 4, K, grid_, ST, __VA_ARGS__);                      \
    else if (nv_ <= 6) ALD_ROW_LAUNCH(KERNEL, C, 6, K, grid_, ST, __VA_ARGS__);                      \
    else if (nv_ <= 8) ALD_ROW_LAUNCH(KERNEL, C, 8, K, grid_, ST, __VA_ARGS__);                      \
    else if (nv_ <= 12) ALD_ROW_LAUNCH(KERNEL, C, 12, K, grid_, ST, __VA_ARGS__);                    \
    else ALD_ROW_LAUNCH(KERNEL, C, 16, K, grid_, ST, __VA_ARGS__);                                   \
  } while (0)

void launch_row_quant(const uint16_t* x, int64_t ldx, int M, int K, int8_t* q, int64_t ldq, float* scale,
                      hipStream_t st) {
  if (M <= 0) return;
  if (fits_llc(M, K)) ALD_ROW_DISPATCH(row_quant_kernel, true, K, M, false, st, x, ldx, M, K, q, ldq, scale);
  else ALD_ROW_DISPATCH(row_quant_kernel, false, K, M, false, st, x, ldx, M, K, q, ldq, scale);
}

void launch_ln_quant(const uint16_t* x, int64_t ldx, int M, int H, const float* g, const float* b, float eps,
                     uint16_t* u_out, int8_t* q, float* scale, hipStream_t st) {
  if (M <= 0) return;
  if (fits_llc(M, H))
    ALD_ROW_DISPATCH(ln_quant_kernel, true, H, M, true, st, x, ldx, M, H, g, b, eps, u_out, q, scale);
  else
    ALD_ROW_DISPATCH(ln_quant_kernel, false, H, M, true, st, x, ldx, M, H, g, b, eps, u_out, q, scale);
}

void launch_ln_f16(const uint16_t* x, int64_t ldx, int M, int H, const float* g, const float* b, float eps,
                   uint16_t* y, int64_t ldy, hipStream_t st) {
  if (M <= 0) return;
  if (fits_llc(M, H)) ALD_ROW_DISPATCH(ln_f16_kernel, true, H, M, false, st, x, ldx, M, H, g, b, eps, y, ldy);
  else ALD_ROW_DISPATCH(ln_f16_kernel, false, H, M, false, st, x, ldx, M, H, g, b, eps, y, ldy);
}

void launch_q4_pack(const uint16_t* w, int N, int K, uint8_t* packed, uint16_t* scales, hipStream_t st) {
  int64_t groups = (int64_t)N * (K / 32);
  if (groups <= 0) return;
  hipLaunchKernelGGL(q4_pack_kernel, dim3((unsigned)((groups + 255) / 256)), dim3(256), 0, st, w, groups, packed,
                     scales);
}

}  // namespace ald
