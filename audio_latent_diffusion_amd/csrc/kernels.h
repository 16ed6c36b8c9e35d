// Internal launchers shared by the C ABI (abi.cpp) and the kernel files.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ald {

enum AKind { A_I8 = 0, A_F16 = 1 };
enum BKind { B_I8 = 0, B_F16 = 1, B_Q4 = 2 };

struct EpiArgs {
  const float* x_scale = nullptr;   // [M]    (int8 A)
  const float* w_scale = nullptr;   // [N]    (int8 B)
  const float* bias = nullptr;      // [N]
  const uint16_t* residual = nullptr;
  int64_t ldr = 0;
  uint16_t* y = nullptr;
  int64_t ldy = 0;
  int32_t* acc = nullptr;           // [M, N] raw accumulators (int8 path)
  int act = 0;
};

struct GemmArgs {
  const void* A = nullptr;
  int64_t lda = 0;
  const void* B = nullptr;          // [N, K] int8/fp16, or packed q4 [N, K/2]
  const uint16_t* b_scale = nullptr;// q4 group scales [N, K/32]
  int M = 0, N = 0, K = 0;
  EpiArgs epi;
};

struct AttnArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  uint16_t* out;
  int64_t q_stride, kv_stride, o_stride;
  int n_heads;
  int Sq, Sk;
  const int32_t* cu_q;
  const int32_t* cu_k;
  float scale_log2;  // softmax scale * log2(e)
};

struct RowMap {        // token / row -> request
  int64_t n_tok_mod;   // row -> token: row % n_tok_mod (0: row itself)
  int rows_per_req;    // token -> request: (token / rows_per_req) % R
  int R;
  const int32_t* row_req;  // or row_req[token]
};

void launch_row_quant(const uint16_t* x, int64_t ldx, int M, int K, int8_t* q, int64_t ldq, float* scale,
                      hipStream_t st);
void launch_ln_quant(const uint16_t* x, int64_t ldx, int M, int H, const float* g, const float* b, float eps,
                     uint16_t* u_out, int8_t* q, float* scale, hipStream_t st);
void launch_ln_f16(const uint16_t* x, int64_t ldx, int M, int H, const float* g, const float* b, float eps,
                   uint16_t* y, int64_t ldy, hipStream_t st);
void launch_q4_pack(const uint16_t* w, int N, int K, uint8_t* packed, uint16_t* scales, hipStream_t st);

// false (and nothing enqueued) when no kernel covers the operand pair and
// shape; gemm_supported answers the same question without launching
bool launch_gemm(int akind, int bkind, const GemmArgs& g, hipStream_t st);
bool gemm_supported(int akind, int bkind, const GemmArgs& g);
void gemm_prepare();  // one-time kernel attributes (large dynamic LDS)

// pipelined direct-to-LDS MFMA GEMM (gemm_dma.hip): int8 x int8, fp16 x fp16 or
// fp16 x 4-bit with K-contiguous operands whose X row bytes are a multiple of 128
bool gemm_dma_applicable(int akind, int bkind, const GemmArgs& g);
void launch_gemm_dma(int akind, int bkind, const GemmArgs& g, hipStream_t st);
void gemm_dma_prepare();

void launch_attn(const AttnArgs& a, int batch, int max_sq, hipStream_t st);

// project = 0: h += (alpha resid_norm) dir; project = 1: h += (alpha (h . dir)) dir
// out of place: rows m < M_steer steered into dst, the other rows copied
void launch_steer_copy(const uint16_t* src, int64_t lds, uint16_t* dst, int64_t ldd, int M, int M_steer, int H,
                       RowMap map, const float* alpha, float resid_norm, const float* dir, int project,
                       hipStream_t st);
// fp32 latent [n_tok, C] (C % 4 == 0, C <= 512) -> steered copy xs
void launch_steer_latent(const float* x, float* xs, int64_t n_tok, int C, RowMap map, const float* alpha,
                         float resid_norm, const float* dir, int project, hipStream_t st);
void launch_steer(uint16_t* h, int64_t ldh, int M, int H, RowMap map, const float* alpha, float resid_norm,
                  const float* dir, int project, hipStream_t st);
void launch_cfg_merge(const uint16_t* v, int64_t n_tok, int C, RowMap map, const float* w, float* v_hat,
                      hipStream_t st);
void launch_euler(float* x, const float* v_hat, int64_t n_tok, int C, RowMap map, const float* t_cur,
                  const float* t_next, const uint8_t* active, hipStream_t st);
void launch_renoise(float* x, const float* x0, const float* eps, int64_t n_tok, int C, RowMap map,
                    const float* t_cur, const uint8_t* active, hipStream_t st);
// DDIM on alpha_bar (ab: current grid point, ab_next: the next one), warm-start
// re-noise sqrt(ab) x0 + sqrt(1 - ab) eps, and the step's fused CFG + DDIM
void launch_ddim(float* x, const float* e_hat, int64_t n_tok, int C, RowMap map, const float* ab,
                 const float* ab_next, const uint8_t* active, hipStream_t st);
void launch_renoise_vp(float* x, const float* x0, const float* eps, int64_t n_tok, int C, RowMap map,
                       const float* ab, const uint8_t* active, hipStream_t st);
void launch_cfg_ddim(const uint16_t* v, float* x, int64_t n_tok, int C, RowMap map, const float* w,
                     const float* ab, const float* ab_next, const uint8_t* active, hipStream_t st);
void launch_cfg_euler(const uint16_t* v, float* x, int64_t n_tok, int C, RowMap map, const float* w,
                      const float* t_cur, const float* t_next, const uint8_t* active, hipStream_t st);
void launch_row_norms(const uint16_t* h, int64_t ldh, int M, int H, float* out, hipStream_t st);
void launch_cu_pairs(const int32_t* cu, int R, int64_t n_tok, int32_t* cu2, hipStream_t st);
void launch_inproj(const float* x, int64_t n_tok, int M, int C, const uint16_t* w, int H, const float* bias,
                   const float* t_cur, RowMap map, uint16_t* h, hipStream_t st);

}  // namespace ald
