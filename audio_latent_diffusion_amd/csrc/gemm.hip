// MFMA GEMMs for the DiT linears: y[M, N] = epilogue(A[M, K] . B[N, K]^T).
//
//  * W8A8   : int8 x int8 -> int32 with v_mfma_i32_16x16x64_i8; epilogue
//             acc * x_scale[m] * w_scale[n] (+ bias, GELU, residual) -> fp16,
//             optional raw int32 accumulator dump.
//  * fp16   : fp16 x fp16 -> fp32 with v_mfma_f32_16x16x32_f16.
//  * q4     : 4-bit weights + fp16 group scales dequantized to fp16(q * s)
//             while staging B into LDS, then the fp16 MFMA.
//
// Both operands are K-contiguous, so every lane of an MFMA fragment reads
// one 16-byte run of a row: the A (B) fragment of lane l is row (l % 16) of
// the 16-row block, bytes [16 (l / 16), 16 (l / 16) + 16) of a 64-byte
// k-slice; the 16x16 accumulator of lane l holds rows 4 (l / 16) + r,
// column l % 16.  LDS rows are padded to 144 bytes (128 + 16), which puts
// the 16 lanes of each fragment read on 16 disjoint 4-bank groups.
// Two LDS stages: the global loads of stage k+1 are in flight while stage k
// feeds the MFMAs.
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace ald {

constexpr int ROWB = 128;        // bytes of K per stage and row
constexpr int LDS_STRIDE = 144;  // padded LDS row (bytes)

template <int AK, int BK, int BM, int BN>
struct GemmTile {
  static constexpr int THREADS = 256;
  static constexpr int WM = BM / 2;  // wave tile rows (2 x 2 waves)
  static constexpr int WN = BN / 2;
  static constexpr int MI = WM / 16;
  static constexpr int NJ = WN / 16;
  static constexpr int A_CHUNKS = BM * (ROWB / 16) / THREADS;  // 16-byte LDS chunks per thread
  static constexpr int B_CHUNKS = BN * (ROWB / 16) / THREADS;
  static constexpr int LDS_A = BM * LDS_STRIDE;
  static constexpr int LDS_B = BN * LDS_STRIDE;
  static constexpr int LDS_BYTES = 2 * (LDS_A + LDS_B);
  static constexpr bool INT = (AK == A_I8);
  static constexpr int KSTAGE = INT ? 128 : 64;  // K elements per stage
};

// ----------------------------------------------------------------- staging

// A operand: int8 or fp16 rows, 16-byte chunks
template <int AK, int BM>
struct AStage;

template <int BM>
struct AStage<A_I8, BM> {
  static constexpr int N = BM * 8 / 256;
  v4i r[N];
  __device__ void load(const GemmArgs& g, int m0, int k0, int tid) {
    const int8_t* A = static_cast<const int8_t*>(g.A);
#pragma unroll
    for (int i = 0; i < N; ++i) {
      int c = tid + 256 * i, row = c >> 3, col = (c & 7) * 16;
      int m = m0 + row, k = k0 + col;
      r[i] = (m < g.M && k < g.K) ? ld16(A + (int64_t)m * g.lda + k) : v4i{0, 0, 0, 0};
    }
  }
  __device__ void store(uint8_t* lds, int tid) {
#pragma unroll
    for (int i = 0; i < N; ++i) {
      int c = tid + 256 * i, row = c >> 3, col = (c & 7) * 16;
      *reinterpret_cast<v4i*>(lds + row * LDS_STRIDE + col) = r[i];
    }
  }
};

template <int BM>
struct AStage<A_F16, BM> {
  static constexpr int N = BM * 8 / 256;
  v4i r[N];
  __device__ void load(const GemmArgs& g, int m0, int k0, int tid) {
    const uint16_t* A = static_cast<const uint16_t*>(g.A);
#pragma unroll
    for (int i = 0; i < N; ++i) {
      int c = tid + 256 * i, row = c >> 3, col = (c & 7) * 8;
      int m = m0 + row, k = k0 + col;
      r[i] = (m < g.M && k < g.K) ? ld16(A + (int64_t)m * g.lda + k) : v4i{0, 0, 0, 0};
    }
  }
  __device__ void store(uint8_t* lds, int tid) {
#pragma unroll
    for (int i = 0; i < N; ++i) {
      int c = tid + 256 * i, row = c >> 3, col = (c & 7) * 16;
      *reinterpret_cast<v4i*>(lds + row * LDS_STRIDE + col) = r[i];
    }
  }
};

template <int BK, int BN>
struct BStage;

template <int BN>
struct BStage<B_I8, BN> {
  static constexpr int N = BN * 8 / 256;
  v4i r[N];
  __device__ void load(const GemmArgs& g, int n0, int k0, int tid) {
    const int8_t* B = static_cast<const int8_t*>(g.B);
#pragma unroll
    for (int i = 0; i < N; ++i) {
      int c = tid + 256 * i, row = c >> 3, col = (c & 7) * 16;
      int n = n0 + row, k = k0 + col;
      r[i] = (n < g.N && k < g.K) ? ld16(B + (int64_t)n * g.K + k) : v4i{0, 0, 0, 0};
    }
  }
  __device__ void store(uint8_t* lds, int tid) {
#pragma unroll
    for (int i = 0; i < N; ++i) {
      int c = tid + 256 * i, row = c >> 3, col = (c & 7) * 16;
      *reinterpret_cast<v4i*>(lds + row * LDS_STRIDE + col) = r[i];
    }
  }
};

template <int BN>
struct BStage<B_F16, BN> {
  static constexpr int N = BN * 8 / 256;
  v4i r[N];
  __device__ void load(const GemmArgs& g, int n0, int k0, int tid) {
    const uint16_t* B = static_cast<const uint16_t*>(g.B);
#pragma unroll
    for (int i = 0; i < N; ++i) {
      int c = tid + 256 * i, row = c >> 3, col = (c & 7) * 8;
      int n = n0 + row, k = k0 + col;
      r[i] = (n < g.N && k < g.K) ? ld16(B + (int64_t)n * g.K + k) : v4i{0, 0, 0, 0};
    }
  }
  __device__ void store(uint8_t* lds, int tid) {
#pragma unroll
    for (int i = 0; i < N; ++i) {
      int c = tid + 256 * i, row = c >> 3, col = (c & 7) * 16;
      *reinterpret_cast<v4i*>(lds + row * LDS_STRIDE + col) = r[i];
    }
  }
};

// 4-bit weights: a stage covers 64 k = two groups of 32 per row.  Item
// (row, group) = 16 packed bytes + one fp16 scale -> 32 fp16 = 64 LDS bytes.
template <int BN>
struct BStage<B_Q4, BN> {
  static constexpr int N = (BN * 2 + 255) / 256;
  v4i r[N];
  uint16_t s[N];
  __device__ void load(const GemmArgs& g, int n0, int k0, int tid) {
    const uint8_t* B = static_cast<const uint8_t*>(g.B);
    const int kg = g.K / 32;
#pragma unroll
    for (int i = 0; i < N; ++i) {
      int it = tid + 256 * i;
      int row = it >> 1, grp = it & 1;
      int n = n0 + row, k = k0 + grp * 32;
      if (it < BN * 2 && n < g.N && k < g.K) {
        r[i] = ld16(B + (int64_t)n * (g.K / 2) + k / 2);
        s[i] = g.b_scale[(int64_t)n * kg + k / 32];
      } else {
        r[i] = v4i{0, 0, 0, 0};
        s[i] = 0;
      }
    }
  }
  __device__ void store(uint8_t* lds, int tid) {
#pragma unroll
    for (int i = 0; i < N; ++i) {
      int it = tid + 256 * i;
      if (it >= BN * 2) continue;
      int row = it >> 1, grp = it & 1;
      const _Float16 sc = __builtin_bit_cast(_Float16, s[i]);
      const uint32_t* wds = reinterpret_cast<const uint32_t*>(&r[i]);
      uint8_t* dst = lds + row * LDS_STRIDE + grp * 64;
#pragma unroll
      for (int wd = 0; wd < 4; ++wd) {
        uint32_t v = wds[wd];
        _Float16 h[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          int code = (int)((v >> (4 * e)) & 0xF);
          code = (code ^ 8) - 8;  // sign-extend the nibble
          h[e] = (_Float16)code * sc;  // exact product rounded once to fp16
        }
        *reinterpret_cast<v4i*>(dst + wd * 16) = *reinterpret_cast<v4i*>(h);
      }
    }
  }
};

// ----------------------------------------------------------------- kernel

template <int AK, int BK, int BM, int BN>
__global__ __launch_bounds__(256) void gemm_kernel(GemmArgs g) {
  using T = GemmTile<AK, BK, BM, BN>;
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  // stage s: A at smem + s * LDS_A, B at smem + 2 LDS_A + s * LDS_B
  uint8_t* const sA0 = smem;
  uint8_t* const sB0 = smem + 2 * T::LDS_A;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int m0 = blockIdx.y * BM, n0 = blockIdx.x * BN;

  typedef typename std::conditional<T::INT, v4i, v4f>::type Acc;
  Acc acc[T::MI][T::NJ];
#pragma unroll
  for (int i = 0; i < T::MI; ++i)
#pragma unroll
    for (int j = 0; j < T::NJ; ++j) acc[i][j] = Acc{0, 0, 0, 0};

  AStage<AK, BM> as;
  BStage<BK, BN> bs;
  const int nk = (g.K + T::KSTAGE - 1) / T::KSTAGE;
  as.load(g, m0, 0, tid);
  bs.load(g, n0, 0, tid);
  as.store(sA0, tid);
  bs.store(sB0, tid);
  __syncthreads();

  const int frow = lane & 15;         // fragment row within a 16-row block
  const int fcol = (lane >> 4) * 16;  // fragment byte offset within a 64-byte k-slice
  int buf = 0;
  for (int kt = 0; kt < nk; ++kt) {
    if (kt + 1 < nk) {
      as.load(g, m0, (kt + 1) * T::KSTAGE, tid);
      bs.load(g, n0, (kt + 1) * T::KSTAGE, tid);
    }
    const uint8_t* pa = sA0 + buf * T::LDS_A + (wm * T::WM + frow) * LDS_STRIDE + fcol;
    const uint8_t* pb = sB0 + buf * T::LDS_B + (wn * T::WN + frow) * LDS_STRIDE + fcol;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      v4i fa[T::MI], fb[T::NJ];
#pragma unroll
      for (int i = 0; i < T::MI; ++i) fa[i] = *reinterpret_cast<const v4i*>(pa + i * 16 * LDS_STRIDE + ks * 64);
#pragma unroll
      for (int j = 0; j < T::NJ; ++j) fb[j] = *reinterpret_cast<const v4i*>(pb + j * 16 * LDS_STRIDE + ks * 64);
#pragma unroll
      for (int i = 0; i < T::MI; ++i)
#pragma unroll
        for (int j = 0; j < T::NJ; ++j) {
          if constexpr (T::INT) {
            acc[i][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(fa[i], fb[j], acc[i][j], 0, 0, 0);
          } else {
            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(v8h, fa[i]),
                                                               __builtin_bit_cast(v8h, fb[j]), acc[i][j], 0, 0, 0);
          }
        }
    }
    if (kt + 1 < nk) {
      as.store(sA0 + (buf ^ 1) * T::LDS_A, tid);
      bs.store(sB0 + (buf ^ 1) * T::LDS_B, tid);
    }
    __syncthreads();
    buf ^= 1;
  }

  // epilogue: lane holds rows 4 (lane / 16) + r, column lane % 16 of each block
  const EpiArgs& e = g.epi;
#pragma unroll
  for (int j = 0; j < T::NJ; ++j) {
    const int col = n0 + wn * T::WN + j * 16 + (lane & 15);
    if (col >= g.N) continue;
    const float ws = (T::INT && e.w_scale) ? e.w_scale[col] : 1.0f;
    const float bias = e.bias ? e.bias[col] : 0.0f;
#pragma unroll
    for (int i = 0; i < T::MI; ++i) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = m0 + wm * T::WM + i * 16 + (lane >> 4) * 4 + r;
        if (row >= g.M) continue;
        float v;
        if constexpr (T::INT) {
          const int a = acc[i][j][r];
          if (e.acc) e.acc[(int64_t)row * g.N + col] = a;
          v = (float)a * e.x_scale[row] * ws;
        } else {
          v = acc[i][j][r];
        }
        if (!e.y) continue;
        v += bias;
        if (e.act == 1) v = gelu_erf(v);
        if (e.residual) v += h2f(e.residual[(int64_t)row * e.ldr + col]);
        e.y[(int64_t)row * e.ldy + col] = f2h(v);
      }
    }
  }
}

template <int AK, int BK, int BM, int BN>
static void launch_tile(const GemmArgs& g, hipStream_t st) {
  using T = GemmTile<AK, BK, BM, BN>;
  dim3 grid((unsigned)((g.N + BN - 1) / BN), (unsigned)((g.M + BM - 1) / BM));
  hipLaunchKernelGGL((gemm_kernel<AK, BK, BM, BN>), grid, dim3(256), T::LDS_BYTES, st, g);
}

template <int AK, int BK, int BM, int BN>
static void set_lds() {
  using T = GemmTile<AK, BK, BM, BN>;
  (void)hipFuncSetAttribute(reinterpret_cast<const void*>(&gemm_kernel<AK, BK, BM, BN>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, T::LDS_BYTES);
}

void gemm_prepare() {
  gemm_dma_prepare();
  set_lds<A_I8, B_I8, 128, 128>();
  set_lds<A_I8, B_I8, 128, 64>();
  set_lds<A_F16, B_F16, 128, 128>();
  set_lds<A_F16, B_F16, 128, 64>();
  set_lds<A_F16, B_Q4, 128, 128>();
  set_lds<A_F16, B_Q4, 128, 64>();
}

bool gemm_supported(int akind, int bkind, const GemmArgs& g) {
  if (g.M <= 0 || g.N <= 0) return true;  // nothing to compute
  if (gemm_dma_applicable(akind, bkind, g)) return true;
  // the register-staged kernel covers int8 x int8, fp16 x fp16 and fp16 x 4-bit;
  // fp16 x int8 (8-bit weight-only) exists only in the direct-to-LDS kernel
  return (akind == A_I8 && bkind == B_I8) || (akind == A_F16 && (bkind == B_F16 || bkind == B_Q4));
}

bool launch_gemm(int akind, int bkind, const GemmArgs& g, hipStream_t st) {
  if (g.M <= 0 || g.N <= 0) return true;
  if (gemm_dma_applicable(akind, bkind, g)) {
    launch_gemm_dma(akind, bkind, g, st);
    return true;
  }
  const bool narrow = g.N <= 64;
  if (akind == A_I8 && bkind == B_I8) {
    if (narrow) launch_tile<A_I8, B_I8, 128, 64>(g, st);
    else launch_tile<A_I8, B_I8, 128, 128>(g, st);
  } else if (akind == A_F16 && bkind == B_F16) {
    if (narrow) launch_tile<A_F16, B_F16, 128, 64>(g, st);
    else launch_tile<A_F16, B_F16, 128, 128>(g, st);
  } else if (akind == A_F16 && bkind == B_Q4) {
    if (narrow) launch_tile<A_F16, B_Q4, 128, 64>(g, st);
    else launch_tile<A_F16, B_Q4, 128, 128>(g, st);
  } else {
    return false;  // no kernel for this operand pair and shape: nothing enqueued
  }
  return true;
}

}  // namespace ald
