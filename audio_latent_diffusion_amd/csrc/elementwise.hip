// Bandwidth-bound elementwise kernels: steering (residual, text and latent
// sites), CFG merge, sampler updates (flow-matching Euler and DDIM, with their
// warm-start re-noise), their fusions used inside the step,
// per-row L2 norms (steering calibration) and the CFG-pair sequence offsets.
//
// Latent kernels: one thread per vector of 4 consecutive latent values,
// streamed with nontemporal loads and stores (data touched once); measured on
// MI355X, more vectors per thread or grid-stride loops only lowered the
// achieved bandwidth.  Index arithmetic is 32-bit (the C ABI bounds the vector
// count).  Steering: one wave per row, the direction held in registers, rows
// walked with the grid's stride.
#include <algorithm>

#include "common.h"
#include "kernels.h"

namespace ald {

__device__ __forceinline__ int req_of(const RowMap& m, uint32_t row) {
  const uint32_t i = m.n_tok_mod ? row % (uint32_t)m.n_tok_mod : row;
  return m.row_req ? m.row_req[i] : (int)((i / (uint32_t)m.rows_per_req) % (uint32_t)m.R);
}

__device__ __forceinline__ void load4h_nt(const uint16_t* p, float f[4]) {
  const v2i r = ld8_nt(p);
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    f[2 * i] = h2f((uint16_t)((uint32_t)r[i] & 0xFFFFu));
    f[2 * i + 1] = h2f((uint16_t)((uint32_t)r[i] >> 16));
  }
}
__device__ __forceinline__ v4f ld4f_nt(const float* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const v4f*>(p));
}
__device__ __forceinline__ void st4f_nt(float* p, v4f v) { __builtin_nontemporal_store(v, reinterpret_cast<v4f*>(p)); }

// Steering of the rows m < M_steer whose request strength a = alpha[r] is
// nonzero (fp16 rows of H values, fp32 arithmetic, one rounding):
//   add      : dst[m, :] = src[m, :] + (a * resid_norm) * dir
//   project  : dst[m, :] = src[m, :] + (a * (src[m, :] . dir)) * dir
// In place (OOP false, src == dst) rows with a == 0 are not touched at all;
// out of place they and the rows m >= M_steer are copied unchanged.
template <int NV, bool PROJ, bool OOP>
__global__ __launch_bounds__(256) void steer_kernel(const uint16_t* src, int64_t lds, uint16_t* dst, int64_t ldd,
                                                    int M, int M_steer, int H, RowMap map,
                                                    const float* __restrict__ alpha, float resid_norm,
                                                    const float* __restrict__ dir) {
  const int lane = threadIdx.x & 63;
  const int stride = gridDim.x * 4;
  int m = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (m >= M) return;
  float dv[NV][8];
#pragma unroll
  for (int j = 0; j < NV; ++j) {
    const int e = (lane + WAVE * j) * 8;
    if (e < H) {
      const float4 d0 = *reinterpret_cast<const float4*>(dir + e);
      const float4 d1 = *reinterpret_cast<const float4*>(dir + e + 4);
      dv[j][0] = d0.x; dv[j][1] = d0.y; dv[j][2] = d0.z; dv[j][3] = d0.w;
      dv[j][4] = d1.x; dv[j][5] = d1.y; dv[j][6] = d1.z; dv[j][7] = d1.w;
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) dv[j][i] = 0.0f;
    }
  }
  for (; m < M; m += stride) {
    const float a = m < M_steer ? alpha[req_of(map, (uint32_t)m)] : 0.0f;
    const uint16_t* srow = src + (int64_t)m * lds;
    uint16_t* drow = dst + (int64_t)m * ldd;
    if (a == 0.0f) {  // exact no-op (uniform over the wave)
      if constexpr (OOP) {
#pragma unroll
        for (int j = 0; j < NV; ++j) {
          const int e = (lane + WAVE * j) * 8;
          if (e < H) st16_nt(drow + e, ld16_nt(srow + e));
        }
      }
      continue;
    }
    v4i raw[NV];
#pragma unroll
    for (int j = 0; j < NV; ++j) {
      const int e = (lane + WAVE * j) * 8;
      raw[j] = e < H ? ld16_nt(srow + e) : v4i{0, 0, 0, 0};
    }
    float coef = a * resid_norm;
    if constexpr (PROJ) {
      float dot = 0.0f;
#pragma unroll
      for (int j = 0; j < NV; ++j) {
        const uint16_t* hv = reinterpret_cast<const uint16_t*>(&raw[j]);
#pragma unroll
        for (int i = 0; i < 8; ++i) dot = fmaf(h2f(hv[i]), dv[j][i], dot);
      }
      coef = a * wave_sum(dot);
    }
#pragma unroll
    for (int j = 0; j < NV; ++j) {
      const int e = (lane + WAVE * j) * 8;
      if (e < H) {
        uint16_t* hv = reinterpret_cast<uint16_t*>(&raw[j]);
#pragma unroll
        for (int i = 0; i < 8; ++i) hv[i] = f2h(h2f(hv[i]) + coef * dv[j][i]);
        st16_nt(drow + e, raw[j]);
      }
    }
  }
}

// Steering of the fp32 latent fed to the model (the latent site), when C / 4
// divides 64: one thread per vector of 4 channels, the G = C / 4 lanes of a
// token consecutive and aligned inside a wave, the projection's dot product
// summed over them with lane exchanges (every lane takes part, also past the
// end); formulas as below.
template <bool PROJ>
__global__ __launch_bounds__(256) void steer_latent_vec_kernel(const float* __restrict__ x, float* __restrict__ xs,
                                                               uint32_t n_tok, int C, RowMap map,
                                                               const float* __restrict__ alpha, float resid_norm,
                                                               const float* __restrict__ dir) {
  const int G = C >> 2;
  const uint32_t i = blockIdx.x * 256u + threadIdx.x;
  const uint32_t tok = i / (uint32_t)G;
  const int c = (int)(i % (uint32_t)G) * 4;
  const bool valid = tok < n_tok;
  const int64_t o = (int64_t)tok * C + c;
  v4f v = valid ? ld4f_nt(x + o) : v4f{0.0f, 0.0f, 0.0f, 0.0f};
  const v4f d = *reinterpret_cast<const v4f*>(dir + c);
  const float a = valid ? alpha[req_of(map, tok)] : 0.0f;
  float coef = a * resid_norm;
  if constexpr (PROJ) {
    float dot = 0.0f;
#pragma unroll
    for (int k = 0; k < 4; ++k) dot = fmaf(v[k], d[k], dot);
    for (int m = 1; m < G; m <<= 1) dot += __shfl_xor(dot, m);
    coef = a * dot;
  }
  if (!valid) return;
  if (a != 0.0f) {
#pragma unroll
    for (int k = 0; k < 4; ++k) v[k] = fmaf(coef, d[k], v[k]);
  }
  st4f_nt(xs + o, v);
}

// The general form (C up to 512): one wave per token, a lane holds 4
// consecutive channels per 256-channel slice;
//   add     : xs[t, :] = x[t, :] + (a * resid_norm) * dir
//   project : xs[t, :] = x[t, :] + (a * (x[t, :] . dir)) * dir
// as one fp32 FMA per value; tokens with a == 0 are copied unchanged.
template <int NV, bool PROJ>
__global__ __launch_bounds__(256) void steer_latent_kernel(const float* __restrict__ x, float* __restrict__ xs,
                                                           uint32_t n_tok, int C, RowMap map,
                                                           const float* __restrict__ alpha, float resid_norm,
                                                           const float* __restrict__ dir) {
  const int lane = threadIdx.x & 63;
  const uint32_t stride = gridDim.x * 4u;
  uint32_t t = blockIdx.x * 4u + (threadIdx.x >> 6);
  if (t >= n_tok) return;
  v4f dv[NV];
#pragma unroll
  for (int j = 0; j < NV; ++j) {
    const int e = (lane + WAVE * j) * 4;
    dv[j] = e < C ? *reinterpret_cast<const v4f*>(dir + e) : v4f{0.0f, 0.0f, 0.0f, 0.0f};
  }
  for (; t < n_tok; t += stride) {
    const float a = alpha[req_of(map, t)];
    const float* row = x + (int64_t)t * C;
    float* orow = xs + (int64_t)t * C;
    v4f v[NV];
#pragma unroll
    for (int j = 0; j < NV; ++j) {
      const int e = (lane + WAVE * j) * 4;
      v[j] = e < C ? ld4f_nt(row + e) : v4f{0.0f, 0.0f, 0.0f, 0.0f};
    }
    if (a != 0.0f) {  // uniform over the wave
      float coef = a * resid_norm;
      if constexpr (PROJ) {
        float dot = 0.0f;
#pragma unroll
        for (int j = 0; j < NV; ++j)
#pragma unroll
          for (int i = 0; i < 4; ++i) dot = fmaf(v[j][i], dv[j][i], dot);
        coef = a * wave_sum(dot);
      }
#pragma unroll
      for (int j = 0; j < NV; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i) v[j][i] = fmaf(coef, dv[j][i], v[j][i]);
    }
#pragma unroll
    for (int j = 0; j < NV; ++j) {
      const int e = (lane + WAVE * j) * 4;
      if (e < C) st4f_nt(orow + e, v[j]);
    }
  }
}


// this thread's vector: token and column (false past the end)
__device__ __forceinline__ bool lat_vec(uint32_t n_tok, int C, uint32_t& tok, int& c) {
  const uint32_t cq = (uint32_t)C >> 2;
  const uint32_t i = blockIdx.x * 256u + threadIdx.x;
  tok = i / cq;
  c = (int)(i - tok * cq) * 4;
  return tok < n_tok;
}

// v_hat = w * cond + (1 - w) * uncond, fp32
__global__ __launch_bounds__(256) void cfg_merge_kernel(const uint16_t* __restrict__ v, uint32_t n_tok, int C,
                                                        RowMap map, const float* __restrict__ w,
                                                        float* __restrict__ v_hat) {
  uint32_t tok;
  int c;
  if (!lat_vec(n_tok, C, tok, c)) return;
  float fc[4], fu[4];
  load4h_nt(v + (int64_t)tok * C + c, fc);
  load4h_nt(v + ((int64_t)n_tok + tok) * C + c, fu);
  const float wr = w[req_of(map, tok)];
  const float wu = 1.0f - wr;
  v4f o;
#pragma unroll
  for (int i = 0; i < 4; ++i) o[i] = wr * fc[i] + wu * fu[i];
  st4f_nt(v_hat + (int64_t)tok * C + c, o);
}

__global__ __launch_bounds__(256) void euler_kernel(float* __restrict__ x, const float* __restrict__ v_hat,
                                                    uint32_t n_tok, int C, RowMap map,
                                                    const float* __restrict__ t_cur, const float* __restrict__ t_next,
                                                    const uint8_t* __restrict__ active) {
  uint32_t tok;
  int c;
  if (!lat_vec(n_tok, C, tok, c)) return;
  const int64_t o = (int64_t)tok * C + c;
  v4f xv = ld4f_nt(x + o);
  const v4f vv = ld4f_nt(v_hat + o);
  const int r = req_of(map, tok);
  if (active && !active[r]) return;
  const float dt = t_next[r] - t_cur[r];
#pragma unroll
  for (int i = 0; i < 4; ++i) xv[i] += dt * vv[i];
  st4f_nt(x + o, xv);
}

__global__ __launch_bounds__(256) void renoise_kernel(float* __restrict__ x, const float* __restrict__ x0,
                                                      const float* __restrict__ eps, uint32_t n_tok, int C, RowMap map,
                                                      const float* __restrict__ t_cur,
                                                      const uint8_t* __restrict__ active) {
  uint32_t tok;
  int c;
  if (!lat_vec(n_tok, C, tok, c)) return;
  const int64_t o = (int64_t)tok * C + c;
  const v4f av = ld4f_nt(x0 + o);
  const v4f ev = ld4f_nt(eps + o);
  const int r = req_of(map, tok);
  if (active && !active[r]) return;
  const float t = t_cur[r];
  const float s = 1.0f - t;
  v4f out;
#pragma unroll
  for (int i = 0; i < 4; ++i) out[i] = s * av[i] + t * ev[i];
  st4f_nt(x + o, out);
}

// fused CFG merge + Euler for the step: v_hat never touches memory
__global__ __launch_bounds__(256) void cfg_euler_kernel(const uint16_t* __restrict__ v, float* __restrict__ x,
                                                        uint32_t n_tok, int C, RowMap map, const float* __restrict__ w,
                                                        const float* __restrict__ t_cur,
                                                        const float* __restrict__ t_next,
                                                        const uint8_t* __restrict__ active) {
  uint32_t tok;
  int c;
  if (!lat_vec(n_tok, C, tok, c)) return;
  const int64_t o = (int64_t)tok * C + c;
  float fc[4], fu[4];
  load4h_nt(v + o, fc);
  load4h_nt(v + (int64_t)n_tok * C + o, fu);
  v4f xv = ld4f_nt(x + o);
  const int r = req_of(map, tok);
  if (active && !active[r]) return;
  const float wr = w[r];
  const float wu = 1.0f - wr;
  const float dt = t_next[r] - t_cur[r];
#pragma unroll
  for (int i = 0; i < 4; ++i) xv[i] += dt * (wr * fc[i] + wu * fu[i]);
  st4f_nt(x + o, xv);
}

// DDIM (eta = 0) on an epsilon prediction, in the method's two steps:
// x0 = (x - sqrt(1 - a) e) / sqrt(a), x' = sqrt(a') x0 + sqrt(1 - a') e
struct DdimCoef {
  float sb, inv_sa, san, sbn;
};
__device__ __forceinline__ DdimCoef ddim_coef(float a, float an) {
  return {sqrtf(1.0f - a), 1.0f / sqrtf(a), sqrtf(an), sqrtf(1.0f - an)};
}
__device__ __forceinline__ float ddim_apply(const DdimCoef& k, float x, float e) {
  const float x0 = (x - k.sb * e) * k.inv_sa;
  return k.san * x0 + k.sbn * e;
}

__global__ __launch_bounds__(256) void ddim_kernel(float* __restrict__ x, const float* __restrict__ e_hat,
                                                   uint32_t n_tok, int C, RowMap map, const float* __restrict__ ab,
                                                   const float* __restrict__ ab_next,
                                                   const uint8_t* __restrict__ active) {
  uint32_t tok;
  int c;
  if (!lat_vec(n_tok, C, tok, c)) return;
  const int64_t o = (int64_t)tok * C + c;
  v4f xv = ld4f_nt(x + o);
  const v4f ev = ld4f_nt(e_hat + o);
  const int r = req_of(map, tok);
  if (active && !active[r]) return;
  const DdimCoef k = ddim_coef(ab[r], ab_next[r]);
#pragma unroll
  for (int i = 0; i < 4; ++i) xv[i] = ddim_apply(k, xv[i], ev[i]);
  st4f_nt(x + o, xv);
}

// warm start under DDIM: x = sqrt(a) x0 + sqrt(1 - a) eps at the skip point
__global__ __launch_bounds__(256) void renoise_vp_kernel(float* __restrict__ x, const float* __restrict__ x0,
                                                         const float* __restrict__ eps, uint32_t n_tok, int C,
                                                         RowMap map, const float* __restrict__ ab,
                                                         const uint8_t* __restrict__ active) {
  uint32_t tok;
  int c;
  if (!lat_vec(n_tok, C, tok, c)) return;
  const int64_t o = (int64_t)tok * C + c;
  const v4f av = ld4f_nt(x0 + o);
  const v4f ev = ld4f_nt(eps + o);
  const int r = req_of(map, tok);
  if (active && !active[r]) return;
  const float sa = sqrtf(ab[r]), sb = sqrtf(1.0f - ab[r]);
  v4f out;
#pragma unroll
  for (int i = 0; i < 4; ++i) out[i] = sa * av[i] + sb * ev[i];
  st4f_nt(x + o, out);
}

// fused CFG merge + DDIM for the step: the guided prediction never touches memory
__global__ __launch_bounds__(256) void cfg_ddim_kernel(const uint16_t* __restrict__ v, float* __restrict__ x,
                                                       uint32_t n_tok, int C, RowMap map, const float* __restrict__ w,
                                                       const float* __restrict__ ab, const float* __restrict__ ab_next,
                                                       const uint8_t* __restrict__ active) {
  uint32_t tok;
  int c;
  if (!lat_vec(n_tok, C, tok, c)) return;
  const int64_t o = (int64_t)tok * C + c;
  float fc[4], fu[4];
  load4h_nt(v + o, fc);
  load4h_nt(v + (int64_t)n_tok * C + o, fu);
  v4f xv = ld4f_nt(x + o);
  const int r = req_of(map, tok);
  if (active && !active[r]) return;
  const float wr = w[r];
  const float wu = 1.0f - wr;
  const DdimCoef k = ddim_coef(ab[r], ab_next[r]);
#pragma unroll
  for (int i = 0; i < 4; ++i) xv[i] = ddim_apply(k, xv[i], wr * fc[i] + wu * fu[i]);
  st4f_nt(x + o, xv);
}

// per-row L2 norm (fp32), one wave per row
__global__ __launch_bounds__(256) void row_norms_kernel(const uint16_t* __restrict__ h, int64_t ldh, int M, int H,
                                                        float* __restrict__ out) {
  const int lane = threadIdx.x & 63;
  const int m = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (m >= M) return;
  const uint16_t* row = h + (int64_t)m * ldh;
  float s = 0.0f;
  for (int e = lane * 8; e < H; e += 512) {
    v4i raw = ld16(row + e);
    const uint16_t* hv = reinterpret_cast<const uint16_t*>(&raw);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      float f = h2f(hv[i]);
      s += f * f;
    }
  }
  s = wave_sum(s);
  if (lane == 0) out[m] = sqrtf(s);
}

// offsets of the 2R CFG sequences: cond rows of every request, then uncond
__global__ void cu_pairs_kernel(const int32_t* __restrict__ cu, int R, int64_t n_tok, int32_t* __restrict__ cu2) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b > 2 * R) return;
  cu2[b] = b <= R ? cu[b] : (int32_t)(n_tok + cu[b - R]);
}

// Input projection of the fp32 latent with the sinusoidal time embedding:
//   h[m, n] = fp16( sum_k fp16(x[m % n_tok, k]) w_in[n, k] + b_in[n] + temb(t_r, n) )
// for both CFG rows of every token (row m reads latent token m % n_tok, request
// r of that token), on the matrix cores: v_mfma_f32_32x32x16_f16 forms the
// fp16 products exactly and accumulates them in fp32.  Each wave computes a
// 64 x 64 block (2 x 2 MFMA blocks of 32 x 32) over K (the latent width, a
// multiple of 8) in steps of 16, zero-padded.  The operands go straight from
// global memory into registers in the MFMA layout (lane l: row of its block
// l % 32, the 8 values at K offset 8 (l / 32) of the step), converted to fp16
// on the way; with K this small nothing is worth sharing through LDS.  The
// weight fragment is the first operand, so accumulator register r of lane l
// holds row l % 32 and column 8 (r / 4) + 4 (l / 32) + r % 4 of its block:
// four consecutive columns per register quad, written as one 8-byte store.
//   temb(t, n) = sin(1000 t w_j) for n < H/2, cos(1000 t w_j) after,
//   w_j = exp(-ln(1e4) j / (H/2)), j = n mod H/2.
// 1000 w_j / (2 pi) (turns per unit of t) is computed once per workgroup and
// column into LDS; per output the argument is t times it (plus a quarter turn
// for the cosine half), reduced to a fraction of a turn and fed to the
// hardware sine (input in turns).  The argument reaches 1000 rad and the fp32
// value carries ~1e-4 rad of rounding error.
// CK > 0: the latent width is the compile-time CK (the K loop unrolls and all
// of a tile's operand loads are in flight at once); CK = 0: any multiple of 8.
// B: 32 x 32 blocks per wave along each side (B = 2: 64 x 64 per wave; B = 1:
// 32 x 32, four times the waves over the same tile, for short launches).
// Each output takes the same products in the same K order either way.
template <int WGN, int WGM, int CK, int B = 2>
__global__ __launch_bounds__(64 * WGN * WGM) void inproj_kernel(const float* __restrict__ x, int64_t n_tok, int M,
                                                                int C_rt, const uint16_t* __restrict__ w, int H,
                                                                const float* __restrict__ bias,
                                                                const float* __restrict__ t_cur, RowMap map,
                                                                uint16_t* __restrict__ h) {
  constexpr int TN = 32 * B * WGN, TM = 32 * B * WGM;
  const int C = CK > 0 ? CK : C_rt;
  __shared__ float turns_per_t[TN];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n0 = blockIdx.x * TN;
  for (int i = tid; i < TN; i += 64 * WGN * WGM) {
    const int half = H >> 1, col = n0 + i;
    const int j = col < half ? col : col - half;
    turns_per_t[i] = 1000.0f * __expf(-9.210340371976184f * (float)j / (float)half) * 0.15915494309189535f;
  }
  __syncthreads();
  const int li = lane & 31, hi = lane >> 5;
  const int cw = (wave % WGN) * 32 * B;  // this wave's columns within the tile
  int64_t wrow[B];
#pragma unroll
  for (int bj = 0; bj < B; ++bj) wrow[bj] = (int64_t)min(n0 + cw + 32 * bj + li, H - 1) * C;
  // row tiles beyond the grid's y extent (65535) are walked with its stride
  for (int m0 = blockIdx.y * TM; m0 < M; m0 += gridDim.y * TM) {
    const int mw = m0 + (wave / WGN) * 32 * B;
    int64_t xrow[B];
#pragma unroll
    for (int bi = 0; bi < B; ++bi) xrow[bi] = (int64_t)(min(mw + 32 * bi + li, M - 1) % n_tok) * C;
    v16f acc[B][B];
#pragma unroll
    for (int bi = 0; bi < B; ++bi)
#pragma unroll
      for (int bj = 0; bj < B; ++bj)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[bi][bj][r] = 0.0f;
#pragma unroll
    for (int k0 = 0; k0 < C; k0 += 16) {
      const int kk = k0 + 8 * hi;
      v8h xf[B], wf[B];
#pragma unroll
      for (int bi = 0; bi < B; ++bi) {
        if (kk < C) {
          const float4 a = *reinterpret_cast<const float4*>(x + xrow[bi] + kk);
          const float4 b = *reinterpret_cast<const float4*>(x + xrow[bi] + kk + 4);
          xf[bi] = v8h{(_Float16)a.x, (_Float16)a.y, (_Float16)a.z, (_Float16)a.w,
                       (_Float16)b.x, (_Float16)b.y, (_Float16)b.z, (_Float16)b.w};
        } else {
          xf[bi] = v8h{0, 0, 0, 0, 0, 0, 0, 0};
        }
      }
#pragma unroll
      for (int bj = 0; bj < B; ++bj)
        wf[bj] = kk < C ? __builtin_bit_cast(v8h, ld16(w + wrow[bj] + kk)) : v8h{0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
      for (int bi = 0; bi < B; ++bi)
#pragma unroll
        for (int bj = 0; bj < B; ++bj)
          acc[bi][bj] = __builtin_amdgcn_mfma_f32_32x32x16_f16(wf[bj], xf[bi], acc[bi][bj], 0, 0, 0);
    }
#pragma unroll
    for (int bi = 0; bi < B; ++bi) {
      const int m = mw + 32 * bi + li;
      if (m >= M) continue;
      const float t = t_cur[req_of(map, (uint32_t)m)];
      uint16_t* hrow = h + (int64_t)m * H;
#pragma unroll
      for (int bj = 0; bj < B; ++bj)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int cl = cw + 32 * bj + 8 * q + 4 * hi;  // column within the tile
          const int col = n0 + cl;
          if (col >= H) continue;  // H % 16 == 0: a quad is inside or outside as a whole
          uint32_t o[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            float turns = t * turns_per_t[cl + r];
            if (col + r >= (H >> 1)) turns += 0.25f;  // cos x = sin(x + pi/2)
            turns -= floorf(turns);
            o[r] = f2h(acc[bi][bj][4 * q + r] + bias[col + r] + __builtin_amdgcn_sinf(turns));
          }
          *reinterpret_cast<uint2*>(hrow + col) = make_uint2(o[0] | (o[1] << 16), o[2] | (o[3] << 16));
        }
    }
  }
}

void launch_inproj(const float* x, int64_t n_tok, int M, int C, const uint16_t* w, int H, const float* bias,
                   const float* t_cur, RowMap map, uint16_t* h, hipStream_t st) {
  if (M <= 0 || H <= 0) return;
  // 128 x 128 tiles of four waves (64 x 64 each), or 64 x 64 tiles of four
  // waves (32 x 32 each) when the large ones would not give every CU a
  // workgroup (the 512-row step)
  // (the latent width 64 of every model here takes the unrolled kernels)
  const int64_t big = (int64_t)((H + 127) / 128) * ((M + 127) / 128);
  if (big >= 256) {
    dim3 grid((unsigned)((H + 127) / 128), (unsigned)std::min<int64_t>((M + 127) / 128, 65535));
    if (C == 64)
      hipLaunchKernelGGL((inproj_kernel<2, 2, 64>), grid, dim3(256), 0, st, x, n_tok, M, C, w, H, bias, t_cur, map, h);
    else
      hipLaunchKernelGGL((inproj_kernel<2, 2, 0>), grid, dim3(256), 0, st, x, n_tok, M, C, w, H, bias, t_cur, map, h);
  } else {
    // 64 x 64 tiles as four waves of 32 x 32 (the 512-row step: 512 waves
    // instead of 128 single-wave tiles; its loop 908 -> 913 steps/s, MI355X)
    dim3 grid((unsigned)((H + 63) / 64), (unsigned)std::min<int64_t>((M + 63) / 64, 65535));
    if (C == 64)
      hipLaunchKernelGGL((inproj_kernel<2, 2, 64, 1>), grid, dim3(256), 0, st, x, n_tok, M, C, w, H, bias, t_cur, map, h);
    else
      hipLaunchKernelGGL((inproj_kernel<2, 2, 0, 1>), grid, dim3(256), 0, st, x, n_tok, M, C, w, H, bias, t_cur, map, h);
  }
}

static inline dim3 grid_for(int64_t n) { return dim3((unsigned)((n + 255) / 256)); }
static inline dim3 grid_lat(int64_t n_tok, int C) { return grid_for(n_tok * (C / 4)); }

template <bool PROJ, bool OOP>
static void launch_steer_mode(const uint16_t* src, int64_t lds, uint16_t* dst, int64_t ldd, int M, int M_steer,
                              int H, RowMap map, const float* alpha, float resid_norm, const float* dir,
                              hipStream_t st) {
  // grid caps measured on 262144 rows of 1536: the add (a stream) prefers
  // more workgroups, the projection (a row reduction before the store) fewer
  // (add 71 -> 73 %, projection 69 -> 73 % of HBM bandwidth against a cap of
  // 2048 for both)
  dim3 grid((unsigned)std::min<int64_t>((M + 3) / 4, PROJ ? 1024 : 4096)), block(256);
  const int nv = (H + 511) / 512;
#define ALD_STEER(NV)                                                                                          \
  hipLaunchKernelGGL((steer_kernel<NV, PROJ, OOP>), grid, block, 0, st, src, lds, dst, ldd, M, M_steer, H, map, \
                     alpha, resid_norm, dir)
  if (nv <= 1) ALD_STEER(1);
  else if (nv <= 2) ALD_STEER(2);
  else if (nv <= 3) ALD_STEER(3);
  else if (nv <= 4) ALD_STEER(4);
  else if (nv <= 8) ALD_STEER(8);
  else ALD_STEER(16);
#undef ALD_STEER
}

void launch_steer(uint16_t* h, int64_t ldh, int M, int H, RowMap map, const float* alpha, float resid_norm,
                  const float* dir, int project, hipStream_t st) {
  if (M <= 0 || H <= 0) return;
  if (project) launch_steer_mode<true, false>(h, ldh, h, ldh, M, M, H, map, alpha, resid_norm, dir, st);
  else launch_steer_mode<false, false>(h, ldh, h, ldh, M, M, H, map, alpha, resid_norm, dir, st);
}

void launch_steer_copy(const uint16_t* src, int64_t lds, uint16_t* dst, int64_t ldd, int M, int M_steer, int H,
                       RowMap map, const float* alpha, float resid_norm, const float* dir, int project,
                       hipStream_t st) {
  if (M <= 0 || H <= 0) return;
  if (project) launch_steer_mode<true, true>(src, lds, dst, ldd, M, M_steer, H, map, alpha, resid_norm, dir, st);
  else launch_steer_mode<false, true>(src, lds, dst, ldd, M, M_steer, H, map, alpha, resid_norm, dir, st);
}

void launch_steer_latent(const float* x, float* xs, int64_t n_tok, int C, RowMap map, const float* alpha,
                         float resid_norm, const float* dir, int project, hipStream_t st) {
  if (n_tok <= 0 || C <= 0) return;
  if (C % 4 == 0 && 64 % (C / 4) == 0) {
    if (project)
      hipLaunchKernelGGL((steer_latent_vec_kernel<true>), grid_lat(n_tok, C), dim3(256), 0, st, x, xs,
                         (uint32_t)n_tok, C, map, alpha, resid_norm, dir);
    else
      hipLaunchKernelGGL((steer_latent_vec_kernel<false>), grid_lat(n_tok, C), dim3(256), 0, st, x, xs,
                         (uint32_t)n_tok, C, map, alpha, resid_norm, dir);
    return;
  }
  dim3 grid((unsigned)std::min<int64_t>((n_tok + 3) / 4, 2048)), block(256);
  const bool two = C > 256;
#define ALD_STEER_LAT(NV, P)                                                                                   \
  hipLaunchKernelGGL((steer_latent_kernel<NV, P>), grid, block, 0, st, x, xs, (uint32_t)n_tok, C, map, alpha,   \
                     resid_norm, dir)
  if (project) {
    if (two) ALD_STEER_LAT(2, true);
    else ALD_STEER_LAT(1, true);
  } else {
    if (two) ALD_STEER_LAT(2, false);
    else ALD_STEER_LAT(1, false);
  }
#undef ALD_STEER_LAT
}

void launch_cfg_merge(const uint16_t* v, int64_t n_tok, int C, RowMap map, const float* w, float* v_hat,
                      hipStream_t st) {
  if (n_tok <= 0) return;
  hipLaunchKernelGGL(cfg_merge_kernel, grid_lat(n_tok, C), dim3(256), 0, st, v, (uint32_t)n_tok, C, map, w, v_hat);
}

void launch_euler(float* x, const float* v_hat, int64_t n_tok, int C, RowMap map, const float* t_cur,
                  const float* t_next, const uint8_t* active, hipStream_t st) {
  if (n_tok <= 0) return;
  hipLaunchKernelGGL(euler_kernel, grid_lat(n_tok, C), dim3(256), 0, st, x, v_hat, (uint32_t)n_tok, C, map, t_cur,
                     t_next, active);
}

void launch_renoise(float* x, const float* x0, const float* eps, int64_t n_tok, int C, RowMap map,
                    const float* t_cur, const uint8_t* active, hipStream_t st) {
  if (n_tok <= 0) return;
  hipLaunchKernelGGL(renoise_kernel, grid_lat(n_tok, C), dim3(256), 0, st, x, x0, eps, (uint32_t)n_tok, C, map,
                     t_cur, active);
}

void launch_cfg_euler(const uint16_t* v, float* x, int64_t n_tok, int C, RowMap map, const float* w,
                      const float* t_cur, const float* t_next, const uint8_t* active, hipStream_t st) {
  if (n_tok <= 0) return;
  hipLaunchKernelGGL(cfg_euler_kernel, grid_lat(n_tok, C), dim3(256), 0, st, v, x, (uint32_t)n_tok, C, map, w,
                     t_cur, t_next, active);
}

void launch_ddim(float* x, const float* e_hat, int64_t n_tok, int C, RowMap map, const float* ab,
                 const float* ab_next, const uint8_t* active, hipStream_t st) {
  if (n_tok <= 0) return;
  hipLaunchKernelGGL(ddim_kernel, grid_lat(n_tok, C), dim3(256), 0, st, x, e_hat, (uint32_t)n_tok, C, map, ab,
                     ab_next, active);
}

void launch_renoise_vp(float* x, const float* x0, const float* eps, int64_t n_tok, int C, RowMap map,
                       const float* ab, const uint8_t* active, hipStream_t st) {
  if (n_tok <= 0) return;
  hipLaunchKernelGGL(renoise_vp_kernel, grid_lat(n_tok, C), dim3(256), 0, st, x, x0, eps, (uint32_t)n_tok, C, map,
                     ab, active);
}

void launch_cfg_ddim(const uint16_t* v, float* x, int64_t n_tok, int C, RowMap map, const float* w,
                     const float* ab, const float* ab_next, const uint8_t* active, hipStream_t st) {
  if (n_tok <= 0) return;
  hipLaunchKernelGGL(cfg_ddim_kernel, grid_lat(n_tok, C), dim3(256), 0, st, v, x, (uint32_t)n_tok, C, map, w, ab,
                     ab_next, active);
}

void launch_row_norms(const uint16_t* h, int64_t ldh, int M, int H, float* out, hipStream_t st) {
  if (M <= 0) return;
  hipLaunchKernelGGL(row_norms_kernel, dim3((unsigned)((M + 3) / 4)), dim3(256), 0, st, h, ldh, M, H, out);
}

void launch_cu_pairs(const int32_t* cu, int R, int64_t n_tok, int32_t* cu2, hipStream_t st) {
  hipLaunchKernelGGL(cu_pairs_kernel, grid_for(2 * R + 1), dim3(256), 0, st, cu, R, n_tok, cu2);
}

}  // namespace ald
