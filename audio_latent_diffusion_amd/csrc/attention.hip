// Flash-style non-causal attention, head_dim 64, fp16 in/out, fp32 online
// softmax, on v_mfma_f32_16x16x32_f16.  Dense and packed varlen sequences.
//
// Workgroup = 4 waves; wave w owns 16 * QW queries of one (sequence, head).
// Keys/values stream through LDS in tiles of 64 (two stages: tile t+1 is
// fetched from HBM while tile t is consumed).
//
// Scores are computed transposed, S^T = K Q^T: the K fragment is the MFMA row
// operand (lane l: key l % 16, 8 dims at 8 (l / 16)), Q stays in registers as
// the column operand.  The accumulator of lane l then holds query l % 16 and
// keys 4 (l / 16) + r, which is exactly the column-operand layout the second
// product O^T = V^T P^T needs (the pairing of k-positions between the two
// operands is free as long as both use the same one), so P never leaves the
// registers.  V is stored transposed in LDS with the matching key order, so
// each V^T fragment is one 16-byte LDS read.  Row statistics reduce over the
// 4 lanes that share a query (xor 16, xor 32).
#include "common.h"
#include "kernels.h"

namespace ald {

constexpr int KT = 64;          // keys per tile
constexpr int HD = 64;          // head dim
constexpr int SROW = 72;        // LDS row stride in halves (144 bytes)

// position of key kv (within a 64-key tile) in the transposed V row
__device__ __forceinline__ int vperm(int kv) {
  int kc = kv >> 5, kl = kv & 31;
  int hh = kl >> 4, g = (kl & 15) >> 2, r = kl & 3;
  return kc * 32 + g * 8 + hh * 4 + r;
}

template <int QW>
__global__ __launch_bounds__(256) void attn_kernel(AttnArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t sK[2][KT * SROW];
  __shared__ __attribute__((aligned(16))) uint16_t sV[2][HD * SROW];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int b = blockIdx.z, h = blockIdx.y;
  const int q_begin = a.cu_q ? a.cu_q[b] : b * a.Sq;
  const int q_len = a.cu_q ? a.cu_q[b + 1] - q_begin : a.Sq;
  const int k_begin = a.cu_k ? a.cu_k[b] : b * a.Sk;
  const int k_len = a.cu_k ? a.cu_k[b + 1] - k_begin : a.Sk;
  const int QT = 64 * QW;
  const int tq0 = blockIdx.x * QT;
  if (tq0 >= q_len) return;  // whole workgroup exits together

  const int ql = lane & 15, g = lane >> 4;
  const int wq0 = tq0 + wave * 16 * QW;

  if (k_len <= 0) {  // no keys: zeros
#pragma unroll
    for (int qb = 0; qb < QW; ++qb) {
      int qi = wq0 + qb * 16 + ql;
      if (qi < q_len) {
        uint16_t* o = a.out + (int64_t)(q_begin + qi) * a.o_stride + h * HD + g * 16;
        st16(o, v4i{0, 0, 0, 0});
        st16(o + 8, v4i{0, 0, 0, 0});
      }
    }
    return;
  }

  // Q fragments (column operand): query ql, dims 32 c + 8 g .. + 8
  v8h qf[QW][2];
#pragma unroll
  for (int qb = 0; qb < QW; ++qb) {
    int qi = wq0 + qb * 16 + ql;
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      if (qi < q_len)
        qf[qb][c] = __builtin_bit_cast(v8h, ld16(a.q + (int64_t)(q_begin + qi) * a.q_stride + h * HD + 32 * c + 8 * g));
      else
        qf[qb][c] = __builtin_bit_cast(v8h, v4i{0, 0, 0, 0});
    }
  }

  v4f oacc[QW][4];
  float m_run[QW], l_run[QW];
#pragma unroll
  for (int qb = 0; qb < QW; ++qb) {
    m_run[qb] = -INFINITY;
    l_run[qb] = 0.0f;
#pragma unroll
    for (int d = 0; d < 4; ++d) oacc[qb][d] = v4f{0, 0, 0, 0};
  }

  // staging registers: K as 2 x 16 B chunks, V as 4 keys x 4 dims
  v4i kreg[2];
  uint64_t vreg[4];
  const int n_tiles = (k_len + KT - 1) / KT;

  auto load_tile = [&](int t) {
    const int kbase = t * KT;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      int c = tid + 256 * i, row = c >> 3, col = (c & 7) * 8;
      int kv = kbase + row;
      kreg[i] = kv < k_len ? ld16(a.k + (int64_t)(k_begin + kv) * a.kv_stride + h * HD + col) : v4i{0, 0, 0, 0};
    }
    const int kvg = tid >> 4, dg = tid & 15;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      int kv = kbase + kvg * 4 + r;
      vreg[r] = kv < k_len ? *reinterpret_cast<const uint64_t*>(a.v + (int64_t)(k_begin + kv) * a.kv_stride + h * HD + dg * 4)
                           : 0ull;
    }
  };
  auto store_tile = [&](int s) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      int c = tid + 256 * i, row = c >> 3, col = (c & 7) * 8;
      *reinterpret_cast<v4i*>(&sK[s][row * SROW + col]) = kreg[i];
    }
    const int kvg = tid >> 4, dg = tid & 15;
    const int p0 = vperm(kvg * 4);
#pragma unroll
    for (int dd = 0; dd < 4; ++dd) {
      // gather dim dd of the 4 keys into one 8-byte word
      uint64_t w = 0;
#pragma unroll
      for (int r = 0; r < 4; ++r) w |= ((vreg[r] >> (16 * dd)) & 0xFFFFull) << (16 * r);
      *reinterpret_cast<uint64_t*>(&sV[s][(dg * 4 + dd) * SROW + p0]) = w;
    }
  };

  load_tile(0);
  store_tile(0);
  __syncthreads();

  int s = 0;
  for (int t = 0; t < n_tiles; ++t) {
    if (t + 1 < n_tiles) load_tile(t + 1);
    const int kbase = t * KT;
    // K fragments (row operand): key kb * 16 + ql, dims 32 c + 8 g
    v8h kf[4][2];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int c = 0; c < 2; ++c)
        kf[kb][c] = *reinterpret_cast<const v8h*>(&sK[s][(kb * 16 + ql) * SROW + 32 * c + 8 * g]);
    // V^T fragments (row operand): dim db * 16 + ql, permuted keys 32 kc + 8 g
    v8h vf[4][2];
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int kc = 0; kc < 2; ++kc)
        vf[db][kc] = *reinterpret_cast<const v8h*>(&sV[s][(db * 16 + ql) * SROW + 32 * kc + 8 * g]);

    // scores of a full tile need no key mask; only the last tile can be partial
    const bool full = kbase + KT <= k_len;
#pragma unroll
    for (int qb = 0; qb < QW; ++qb) {
      v4f sc[4];
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        v4f z = {0, 0, 0, 0};
        z = __builtin_amdgcn_mfma_f32_16x16x32_f16(kf[kb][0], qf[qb][0], z, 0, 0, 0);
        z = __builtin_amdgcn_mfma_f32_16x16x32_f16(kf[kb][1], qf[qb][1], z, 0, 0, 0);
        sc[kb] = z;
      }
      if (!full) {
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if (kbase + kb * 16 + g * 4 + r >= k_len) sc[kb][r] = -INFINITY;
      }
      // running maximum of the raw scores (the softmax scale c > 0 commutes
      // with max), then p = 2^(c s - c m) with one fused multiply-add
      float mx = sc[0][0];
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int r = 0; r < 4; ++r) mx = fmaxf(mx, sc[kb][r]);
      mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
      const float m_old = m_run[qb];
      const float m_new = fmaxf(m_old, mx);
      m_run[qb] = m_new;
      const float c = a.scale_log2;
      const float cm = -c * m_new;
      float psum = 0.0f;
      v8h pf[2];
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float p = __builtin_amdgcn_exp2f(fmaf(sc[kb][r], c, cm));
          psum += p;
          pf[kb >> 1][(kb & 1) * 4 + r] = (_Float16)p;
        }
      // the output and the row sum are rescaled only when some row's maximum
      // moved (a factor of exactly 1 otherwise, so skipping is exact)
      if (__any(m_new != m_old)) {
        const float corr = __builtin_amdgcn_exp2f(c * (m_old - m_new));
        l_run[qb] = l_run[qb] * corr + psum;
#pragma unroll
        for (int db = 0; db < 4; ++db) oacc[qb][db] *= corr;
      } else {
        l_run[qb] += psum;
      }
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        v4f o = oacc[qb][db];
        o = __builtin_amdgcn_mfma_f32_16x16x32_f16(vf[db][0], pf[0], o, 0, 0, 0);
        o = __builtin_amdgcn_mfma_f32_16x16x32_f16(vf[db][1], pf[1], o, 0, 0, 0);
        oacc[qb][db] = o;
      }
    }
    if (t + 1 < n_tiles) store_tile(s ^ 1);
    __syncthreads();
    s ^= 1;
  }

  // normalise and store: lane holds query ql, dims 16 db + 4 g + r
#pragma unroll
  for (int qb = 0; qb < QW; ++qb) {
    float l = l_run[qb];
    l += __shfl_xor(l, 16, 64);
    l += __shfl_xor(l, 32, 64);
    const float inv = 1.0f / l;
    const int qi = wq0 + qb * 16 + ql;
    if (qi >= q_len) continue;
    uint16_t* o = a.out + (int64_t)(q_begin + qi) * a.o_stride + h * HD;
#pragma unroll
    for (int db = 0; db < 4; ++db) {
      uint16_t hv[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) hv[r] = f2h(oacc[qb][db][r] * inv);
      *reinterpret_cast<uint64_t*>(o + db * 16 + g * 4) = *reinterpret_cast<uint64_t*>(hv);
    }
  }
}

void launch_attn(const AttnArgs& a, int batch, int max_sq, hipStream_t st) {
  if (batch <= 0 || max_sq <= 0) return;
  // two query blocks per wave when there is enough parallelism, else one
  const int64_t wgs2 = (int64_t)((max_sq + 127) / 128) * a.n_heads * batch;
  if (wgs2 >= 512) {
    dim3 grid((unsigned)((max_sq + 127) / 128), (unsigned)a.n_heads, (unsigned)batch);
    hipLaunchKernelGGL(attn_kernel<2>, grid, dim3(256), 0, st, a);
  } else {
    dim3 grid((unsigned)((max_sq + 63) / 64), (unsigned)a.n_heads, (unsigned)batch);
    hipLaunchKernelGGL(attn_kernel<1>, grid, dim3(256), 0, st, a);
  }
}

}  // namespace ald
