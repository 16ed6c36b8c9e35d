// C ABI of the DiT denoise step: host-side validation, workspace carving,
// kernel enqueueing and graph capture.  No device allocation, no host sync.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <mutex>
#include <new>
#include <vector>

#include "../../include/ald.h"
#include "kernels.h"

using namespace ald;

namespace {

inline bool al16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
inline bool al8(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 7u) == 0; }

std::once_flag g_prep;
void prepare() { std::call_once(g_prep, [] { gemm_prepare(); }); }

inline int launched() {
  hipError_t e = hipGetLastError();
  return e == hipSuccess ? ALD_OK : ALD_E_LAUNCH;
}

#define CHECK(cond, code) \
  do {                    \
    if (!(cond)) return (code); \
  } while (0)

int check_epilogue(int M, int N, const uint16_t* residual, int64_t ldr, int act, const uint16_t* y, int64_t ldy) {
  CHECK(act == ALD_ACT_NONE || act == ALD_ACT_GELU, ALD_E_INVALID);
  if (y) CHECK(ldy >= N && M >= 0, ALD_E_INVALID);
  if (residual) CHECK(ldr >= N, ALD_E_INVALID);
  return ALD_OK;
}

size_t align256(size_t b) { return (b + 255) & ~size_t(255); }

struct Carve {
  uint8_t* base;
  size_t off = 0;
  size_t cap;
  template <class T>
  T* take(size_t n) {
    T* p = reinterpret_cast<T*>(base + off);
    off += align256(n * sizeof(T));
    return p;
  }
  bool ok() const { return off <= cap; }
};

struct StepBuffers {
  uint16_t* h;
  uint16_t* big;
  uint16_t* ao;
  uint16_t* u;
  int8_t* codes;
  float* xs;
  uint16_t* v;
  int32_t* cu2;
  float* x_lat;      // latent site: steered model input [n_tok, C]
  uint16_t* text_s;  // text site: steered text [2R*T, D_t]
  int8_t* tcodes;    // text site, W8A8: its int8 codes and row scales
  float* tscale;
  uint16_t* kv;      // text site: K/V of the steered text, [2R*T, n_blocks*2H] (one block's in its first 2H
                     // columns when the linears are not stacked)
};

bool steers(const dit_config* c, int site) { return c->steer_block >= 0 && c->steer_site == site; }

// same carve used by dit_workspace_size (with base = nullptr) and dit_step
size_t carve_step(const dit_config* c, int64_t n_tok, int R, uint8_t* base, size_t cap, StepBuffers* b) {
  const int64_t M = 2 * n_tok;
  const int64_t H = c->hidden, F = c->mlp, C = c->channels;
  const int64_t rows_t = 2 * (int64_t)R * c->text_tokens;
  const int64_t wide = std::max<int64_t>(3 * H, F);
  const int64_t codes = std::max<int64_t>(M * std::max<int64_t>(H, F), rows_t * c->text_dim);
  Carve cv{base, 0, cap};
  StepBuffers t{};
  t.h = cv.take<uint16_t>(M * H);
  t.big = cv.take<uint16_t>(M * wide);
  t.ao = cv.take<uint16_t>(M * H);
  t.u = cv.take<uint16_t>(M * H);
  t.codes = cv.take<int8_t>(codes);
  t.xs = cv.take<float>(std::max<int64_t>(M, rows_t));
  t.v = cv.take<uint16_t>(M * C);
  t.cu2 = cv.take<int32_t>(2 * (int64_t)R + 1);
  if (steers(c, ALD_SITE_LATENT)) t.x_lat = cv.take<float>(n_tok * C);
  if (steers(c, ALD_SITE_TEXT)) {
    t.text_s = cv.take<uint16_t>(rows_t * c->text_dim);
    if (c->wmode == ALD_W8A8) {
      t.tcodes = cv.take<int8_t>(rows_t * c->text_dim);
      t.tscale = cv.take<float>(rows_t);
    }
    t.kv = cv.take<uint16_t>(rows_t * 2 * H * std::max(1, c->n_blocks));  // every block's (stacked linears)
  }
  if (b) *b = t;
  return cv.off;
}

int check_config(const dit_config* c) {
  CHECK(c, ALD_E_INVALID);
  CHECK(c->n_blocks >= 0 && c->hidden > 0 && c->n_heads > 0 && c->mlp > 0 && c->channels > 0 &&
            c->text_tokens > 0 && c->text_dim > 0,
        ALD_E_INVALID);
  CHECK(c->wmode == ALD_W8A8 || c->wmode == ALD_F16 || c->wmode == ALD_Q4 || c->wmode == ALD_W8A16,
        ALD_E_INVALID);
  CHECK(c->head_dim == 64 && c->hidden == c->n_heads * 64, ALD_E_UNSUPPORTED);
  CHECK(c->hidden % 16 == 0 && c->mlp % 16 == 0 && c->text_dim % 16 == 0 && c->channels % 8 == 0,
        ALD_E_UNSUPPORTED);
  if (c->wmode == ALD_Q4)
    CHECK(c->hidden % 32 == 0 && c->mlp % 32 == 0 && c->text_dim % 32 == 0, ALD_E_UNSUPPORTED);
  // the 8-bit weight-only GEMM streams 64-element K slices and has no generic fallback
  if (c->wmode == ALD_W8A16)
    CHECK(c->hidden % 64 == 0 && c->mlp % 64 == 0 && c->text_dim % 64 == 0, ALD_E_UNSUPPORTED);
  CHECK(c->hidden <= 8192 && c->mlp <= 8192 && c->text_dim <= 8192, ALD_E_UNSUPPORTED);
  CHECK(c->hidden % 2 == 0, ALD_E_UNSUPPORTED);
  CHECK(c->steer_block >= -1 && c->steer_block < c->n_blocks, ALD_E_INVALID);
  CHECK(c->steer_mode == ALD_STEER_ADD || c->steer_mode == ALD_STEER_PROJECT, ALD_E_INVALID);
  CHECK(c->steer_site == ALD_SITE_RESIDUAL || c->steer_site == ALD_SITE_LATENT || c->steer_site == ALD_SITE_TEXT,
        ALD_E_INVALID);
  if (steers(c, ALD_SITE_LATENT)) CHECK(c->channels <= 512, ALD_E_UNSUPPORTED);
  CHECK(c->sampler == ALD_SAMPLER_FLOW || c->sampler == ALD_SAMPLER_DDIM, ALD_E_INVALID);
  CHECK(c->ln_eps >= 0.0f, ALD_E_INVALID);
  return ALD_OK;
}

int check_linear(const dit_linear& l, int wmode) {
  CHECK(l.w && al16(l.w), ALD_E_INVALID);
  if (wmode != ALD_F16) CHECK(l.scale != nullptr, ALD_E_INVALID);
  return ALD_OK;
}

int check_weights(const dit_config* c, const dit_weights* w) {
  CHECK(w, ALD_E_INVALID);
  CHECK(c->n_blocks == 0 || w->blocks, ALD_E_INVALID);
  CHECK(w->w_in && w->b_in && w->lnf_g && w->lnf_b && w->w_out && w->b_out, ALD_E_INVALID);
  CHECK(al16(w->w_in) && al16(w->w_out) && al16(w->lnf_g) && al16(w->lnf_b), ALD_E_INVALID);
  for (int l = 0; l < c->n_blocks; ++l) {
    const dit_block_weights& b = w->blocks[l];
    CHECK(b.ln1_g && b.ln1_b && b.ln2_g && b.ln2_b && b.ln3_g && b.ln3_b, ALD_E_INVALID);
    CHECK(al16(b.ln1_g) && al16(b.ln1_b) && al16(b.ln2_g) && al16(b.ln2_b) && al16(b.ln3_g) && al16(b.ln3_b),
          ALD_E_INVALID);
    const dit_linear* ls[7] = {&b.qkv, &b.o, &b.q, &b.kv, &b.ox, &b.up, &b.down};
    for (auto* p : ls) {
      int e = check_linear(*p, c->wmode);
      if (e) return e;
    }
  }
  if (w->kv_all.w) {
    int e = check_linear(w->kv_all, c->wmode);
    if (e) return e;
  }
  return ALD_OK;
}

int akind_of(int wmode) { return wmode == ALD_W8A8 ? A_I8 : A_F16; }
int bkind_of(int wmode) { return wmode == ALD_Q4 ? B_Q4 : (wmode == ALD_F16 ? B_F16 : B_I8); }

// the GEMM of one block linear: A is int8 codes (W8A8, with per-row scales
// xs) or fp16 (F16 / Q4 / W8A16)
GemmArgs linear_args(const dit_linear& L, int wmode, const void* A, int64_t lda, const float* xs, int M, int K,
                     int N, const uint16_t* residual, int64_t ldr, int act, uint16_t* y, int64_t ldy) {
  GemmArgs g;
  g.A = A;
  g.lda = lda;
  g.B = L.w;
  g.M = M;
  g.N = N;
  g.K = K;
  g.epi.bias = L.bias;
  g.epi.residual = residual;
  g.epi.ldr = ldr;
  g.epi.y = y;
  g.epi.ldy = ldy;
  g.epi.act = act;
  if (wmode == ALD_W8A8) {
    g.epi.x_scale = xs;
    g.epi.w_scale = static_cast<const float*>(L.scale);
  } else if (wmode == ALD_Q4) {
    g.b_scale = static_cast<const uint16_t*>(L.scale);
  } else if (wmode == ALD_W8A16) {
    g.epi.w_scale = static_cast<const float*>(L.scale);
  }
  return g;
}

// y[M, N] = epilogue(A . W^T); false (nothing enqueued) when no kernel covers it
bool run_linear(const dit_linear& L, int wmode, const void* A, int64_t lda, const float* xs, int M, int K, int N,
                const uint16_t* residual, int64_t ldr, int act, uint16_t* y, int64_t ldy, hipStream_t st) {
  return launch_gemm(akind_of(wmode), bkind_of(wmode),
                     linear_args(L, wmode, A, lda, xs, M, K, N, residual, ldr, act, y, ldy), st);
}

bool linear_ok(const dit_linear& L, int wmode, const void* A, int M, int K, int N) {
  return gemm_supported(akind_of(wmode), bkind_of(wmode),
                        linear_args(L, wmode, A, K, nullptr, M, K, N, nullptr, 0, 0, nullptr, 0));
}

// activation input of a linear: W8A8 quantizes per token, else fp16 as is
struct ActIn {
  const void* A;
  int64_t lda;
  const float* xs;
};

ActIn quantize_in(int wmode, const uint16_t* x, int64_t ldx, int M, int K, const StepBuffers& b, hipStream_t st) {
  if (wmode == ALD_W8A8) {
    launch_row_quant(x, ldx, M, K, b.codes, K, b.xs, st);
    return {b.codes, K, b.xs};
  }
  return {x, ldx, nullptr};
}

ActIn layernorm_in(int wmode, const uint16_t* x, int M, int H, const float* g, const float* be, float eps,
                   const StepBuffers& b, hipStream_t st) {
  if (wmode == ALD_W8A8) {
    launch_ln_quant(x, H, M, H, g, be, eps, nullptr, b.codes, b.xs, st);
    return {b.codes, H, b.xs};
  }
  launch_ln_f16(x, H, M, H, g, be, eps, b.u, H, st);
  return {b.u, H, nullptr};
}

// Every GEMM the step will launch has a kernel for its operands and shape
// (the 8-bit weight-only operand pair exists only in the direct-to-LDS
// kernel, which addresses operands with 32-bit byte offsets); checked before
// any launch so that an unsupported step enqueues nothing.
int check_step_gemms(const dit_config* c, const dit_weights* w, int M, int rows_t, const StepBuffers& b) {
  const int wm = c->wmode, H = c->hidden, F = c->mlp, Dt = c->text_dim;
  const bool q = wm == ALD_W8A8;
  const void* ln_in = q ? static_cast<const void*>(b.codes) : b.u;    // after a LayerNorm
  const void* ao_in = q ? static_cast<const void*>(b.codes) : b.ao;   // after an attention
  const void* mlp_in = q ? static_cast<const void*>(b.codes) : b.big; // after the GELU
  bool ok = true;
  for (int l = 0; l < c->n_blocks; ++l) {
    const dit_block_weights& bw = w->blocks[l];
    ok = ok && linear_ok(bw.qkv, wm, ln_in, M, H, 3 * H) && linear_ok(bw.o, wm, ao_in, M, H, H) &&
         linear_ok(bw.q, wm, ln_in, M, H, H) && linear_ok(bw.ox, wm, ao_in, M, H, H) &&
         linear_ok(bw.up, wm, ln_in, M, H, F) && linear_ok(bw.down, wm, mlp_in, M, F, H);
  }
  if (steers(c, ALD_SITE_TEXT) && c->n_blocks > 0) {
    const void* tin = q ? static_cast<const void*>(b.tcodes) : b.text_s;
    if (w->kv_all.w) ok = ok && linear_ok(w->kv_all, wm, tin, rows_t, Dt, 2 * H * c->n_blocks);
    else
      for (int l = 0; l < c->n_blocks; ++l) ok = ok && linear_ok(w->blocks[l].kv, wm, tin, rows_t, Dt, 2 * H);
  }
  GemmArgs out;  // output projection: fp16 x fp16
  out.A = b.u;
  out.lda = H;
  out.B = w->w_out;
  out.M = M;
  out.N = c->channels;
  out.K = H;
  ok = ok && gemm_supported(A_F16, B_F16, out);
  return ok ? ALD_OK : ALD_E_UNSUPPORTED;
}

int enqueue_step(const dit_config* c, const dit_weights* w, const dit_step_args* a, void* ws, size_t ws_bytes,
                 hipStream_t st) {
  int e = check_config(c);
  if (e) return e;
  e = check_weights(c, w);
  if (e) return e;
  CHECK(a, ALD_E_INVALID);
  CHECK(a->R > 0 && a->n_tok > 0, ALD_E_INVALID);
  CHECK(a->x && al16(a->x), ALD_E_INVALID);
  // the text site recomputes the K/V from the steered text: text_kv unused
  if (!steers(c, ALD_SITE_TEXT)) CHECK(a->text_kv && al16(a->text_kv), ALD_E_INVALID);
  CHECK(a->t_cur && a->t_next && a->guidance, ALD_E_INVALID);
  const bool ddim = c->sampler == ALD_SAMPLER_DDIM;
  if (ddim) CHECK(a->abar_cur && a->abar_next, ALD_E_INVALID);
  const bool varlen = a->cu_seqlens != nullptr;
  if (varlen) {
    CHECK(a->row_req && a->max_seq > 0, ALD_E_INVALID);
  } else {
    CHECK(a->seq > 0 && (int64_t)a->seq * a->R == a->n_tok, ALD_E_INVALID);
  }
  if (c->steer_block >= 0) CHECK(a->alpha && a->direction && al16(a->direction), ALD_E_INVALID);
  if (steers(c, ALD_SITE_TEXT)) CHECK(a->text && al16(a->text), ALD_E_INVALID);
  if (a->renoise) CHECK(a->x0 && a->eps && al16(a->x0) && al16(a->eps), ALD_E_INVALID);
  if (a->v_out) CHECK(al16(a->v_out), ALD_E_INVALID);
  CHECK(2 * a->n_tok <= INT32_MAX, ALD_E_UNSUPPORTED);
  // the latent kernels index vectors of 4 values with 32-bit arithmetic
  CHECK(a->n_tok * (c->channels / 4) < ((int64_t)1 << 31), ALD_E_UNSUPPORTED);
  CHECK(ws && al16(ws), ALD_E_INVALID);
  StepBuffers b;
  size_t need = carve_step(c, a->n_tok, a->R, static_cast<uint8_t*>(ws), ws_bytes, &b);
  CHECK(need <= ws_bytes, ALD_E_WORKSPACE);
  e = check_step_gemms(c, w, (int)(2 * a->n_tok), 2 * a->R * c->text_tokens, b);
  if (e) return e;
  prepare();

  const int H = c->hidden, F = c->mlp, C = c->channels, T = c->text_tokens, nh = c->n_heads;
  const int64_t n_tok = a->n_tok;
  const int M = (int)(2 * n_tok);
  const int R = a->R;
  const int wm = c->wmode;
  RowMap map{n_tok, varlen ? 1 : a->seq, R, varlen ? a->row_req : nullptr};
  const int max_sq = varlen ? a->max_seq : a->seq;
  const int32_t* cu2 = nullptr;
  if (varlen) {
    launch_cu_pairs(a->cu_seqlens, R, n_tok, b.cu2, st);
    cu2 = b.cu2;
  }
  if (a->renoise) {
    if (ddim) launch_renoise_vp(a->x, a->x0, a->eps, n_tok, C, map, a->abar_cur, a->renoise, st);
    else launch_renoise(a->x, a->x0, a->eps, n_tok, C, map, a->t_cur, a->renoise, st);
  }

  const bool project = c->steer_mode == ALD_STEER_PROJECT;
  // latent site: the model reads a steered copy of the latent, the state stays
  const float* x_in = a->x;
  if (steers(c, ALD_SITE_LATENT)) {
    launch_steer_latent(a->x, b.x_lat, n_tok, C, map, a->alpha, a->resid_norm, a->direction, project, st);
    x_in = b.x_lat;
  }
  // input projection of the fp32 latent (both CFG rows read the same latent) + time embedding
  launch_inproj(x_in, n_tok, M, C, w->w_in, H, w->b_in, a->t_cur, map, b.h, st);

  // text site: steer the cond text rows (request r owns rows [r T, (r+1) T)),
  // copy the null-prompt rows, and take its activation operand once
  const bool text_site = steers(c, ALD_SITE_TEXT);
  const int rows_t = 2 * R * T;
  ActIn tin{nullptr, 0, nullptr};
  if (text_site) {
    const int Dt = c->text_dim;
    launch_steer_copy(a->text, Dt, b.text_s, Dt, rows_t, R * T, Dt, RowMap{0, T, R, nullptr}, a->alpha,
                      a->resid_norm, a->direction, project, st);
    if (wm == ALD_W8A8) {
      launch_row_quant(b.text_s, Dt, rows_t, Dt, b.tcodes, Dt, b.tscale, st);
      tin = {b.tcodes, Dt, b.tscale};
    } else {
      tin = {b.text_s, Dt, nullptr};
    }
  }

  // text site with the blocks' K/V linears stacked: the steered text's K/V of
  // every block in one launch, block l's in columns [l 2H, (l + 1) 2H)
  const bool kv_stacked = text_site && w->kv_all.w && c->n_blocks > 0;
  const int64_t kv_ld = kv_stacked ? 2 * (int64_t)H * c->n_blocks : 2 * H;
  if (kv_stacked)
    CHECK(run_linear(w->kv_all, wm, tin.A, tin.lda, tin.xs, rows_t, c->text_dim, (int)kv_ld, nullptr, 0, 0, b.kv,
                     kv_ld, st),
          ALD_E_UNSUPPORTED);

  const float sl2 = 0.125f * 1.4426950408889634f;  // 1/sqrt(64) * log2(e)
  for (int l = 0; l < c->n_blocks; ++l) {
    const dit_block_weights& bw = w->blocks[l];
    const uint16_t* kv = text_site ? (kv_stacked ? b.kv + (int64_t)l * 2 * H : b.kv)
                                   : a->text_kv + (int64_t)l * (2 * (int64_t)R * T) * (2 * H);
    if (text_site && !kv_stacked)  // the same linear dit_text_kv applies, on the steered text
      CHECK(run_linear(bw.kv, wm, tin.A, tin.lda, tin.xs, rows_t, c->text_dim, 2 * H, nullptr, 0, 0, b.kv, 2 * H, st),
            ALD_E_UNSUPPORTED);
    // self-attention
    ActIn in = layernorm_in(wm, b.h, M, H, bw.ln1_g, bw.ln1_b, c->ln_eps, b, st);
    CHECK(run_linear(bw.qkv, wm, in.A, in.lda, in.xs, M, H, 3 * H, nullptr, 0, 0, b.big, 3 * H, st), ALD_E_UNSUPPORTED);
    AttnArgs at{b.big, b.big + H, b.big + 2 * H, b.ao, 3 * H, 3 * H, H, nh, a->seq, a->seq, cu2, cu2, sl2};
    launch_attn(at, 2 * R, max_sq, st);
    in = quantize_in(wm, b.ao, H, M, H, b, st);
    CHECK(run_linear(bw.o, wm, in.A, in.lda, in.xs, M, H, H, b.h, H, 0, b.h, H, st), ALD_E_UNSUPPORTED);
    // cross-attention to the text
    in = layernorm_in(wm, b.h, M, H, bw.ln2_g, bw.ln2_b, c->ln_eps, b, st);
    CHECK(run_linear(bw.q, wm, in.A, in.lda, in.xs, M, H, H, nullptr, 0, 0, b.big, H, st), ALD_E_UNSUPPORTED);
    AttnArgs ax{b.big, kv, kv + H, b.ao, H, text_site ? kv_ld : 2 * H, H, nh, a->seq, T, cu2, nullptr, sl2};
    launch_attn(ax, 2 * R, max_sq, st);
    in = quantize_in(wm, b.ao, H, M, H, b, st);
    CHECK(run_linear(bw.ox, wm, in.A, in.lda, in.xs, M, H, H, b.h, H, 0, b.h, H, st), ALD_E_UNSUPPORTED);
    // GELU MLP
    in = layernorm_in(wm, b.h, M, H, bw.ln3_g, bw.ln3_b, c->ln_eps, b, st);
    CHECK(run_linear(bw.up, wm, in.A, in.lda, in.xs, M, H, F, nullptr, 0, ALD_ACT_GELU, b.big, F, st), ALD_E_UNSUPPORTED);
    in = quantize_in(wm, b.big, F, M, F, b, st);
    CHECK(run_linear(bw.down, wm, in.A, in.lda, in.xs, M, F, H, b.h, H, 0, b.h, H, st), ALD_E_UNSUPPORTED);
    if (steers(c, ALD_SITE_RESIDUAL) && l == c->steer_block) {
      if (a->block_norms) launch_row_norms(b.h, H, M, H, a->block_norms, st);
      launch_steer(b.h, H, M, H, map, a->alpha, a->resid_norm, a->direction, project, st);
    }
  }

  // final LayerNorm + output projection -> velocity of both CFG rows
  launch_ln_f16(b.h, H, M, H, w->lnf_g, w->lnf_b, c->ln_eps, b.u, H, st);
  uint16_t* v = a->v_out ? a->v_out : b.v;
  {
    GemmArgs g;
    g.A = b.u;
    g.lda = H;
    g.B = w->w_out;
    g.M = M;
    g.N = C;
    g.K = H;
    g.epi.bias = w->b_out;
    g.epi.y = v;
    g.epi.ldy = C;
    CHECK(launch_gemm(A_F16, B_F16, g, st), ALD_E_UNSUPPORTED);
  }
  if (ddim) launch_cfg_ddim(v, a->x, n_tok, C, map, a->guidance, a->abar_cur, a->abar_next, a->active, st);
  else launch_cfg_euler(v, a->x, n_tok, C, map, a->guidance, a->t_cur, a->t_next, a->active, st);
  return launched();
}

struct GraphHandle {
  hipGraph_t graph;
  hipGraphExec_t exec;
};

// Scratch of dit_step_static: a file-scope device array, one copy per device,
// held until the process ends.  On the host, `scratch` names a host-side
// stand-in, not device memory: its device address comes from
// hipGetSymbolAddress, taken once per device with that device current and
// kept in g_scratch; only that address is ever handed to a kernel.
__device__ __align__(256) uint8_t scratch[ALD_STATIC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch[kMaxDevices] = {};

int device_scratch(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return ALD_E_LAUNCH;
  CHECK(dev >= 0 && dev < kMaxDevices, ALD_E_UNSUPPORTED);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return ALD_E_LAUNCH;
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return ALD_OK;
}

}  // namespace

extern "C" {

const char* ald_strerror(int code) {
  switch (code) {
    case ALD_OK: return "ok";
    case ALD_E_INVALID: return "invalid argument (null, misaligned, negative size or bad enum)";
    case ALD_E_UNSUPPORTED: return "unsupported shape or mode";
    case ALD_E_WORKSPACE: return "workspace too small";
    case ALD_E_LAUNCH: return "HIP launch error";
    default: return "unknown error";
  }
}

int ald_version(void) { return ALD_VERSION; }

int quantize_rows_q8(const uint16_t* x, int64_t ldx, int M, int K, int8_t* q, int64_t ldq, float* scale,
                     hipStream_t stream) {
  CHECK(M >= 0 && K >= 0, ALD_E_INVALID);
  if (M == 0) return ALD_OK;
  CHECK(x && q && scale, ALD_E_INVALID);
  CHECK(K % 8 == 0 && ldx >= K && ldq >= K && ldx % 8 == 0 && ldq % 8 == 0 && al16(x) && al8(q), ALD_E_INVALID);
  CHECK(K <= 8192, ALD_E_UNSUPPORTED);
  launch_row_quant(x, ldx, M, K, q, ldq, scale, stream);
  return launched();
}

int quantize_q4(const uint16_t* w, int N, int K, uint8_t* packed, uint16_t* scales, hipStream_t stream) {
  CHECK(N >= 0 && K >= 0, ALD_E_INVALID);
  if (N == 0 || K == 0) return ALD_OK;
  CHECK(w && packed && scales && al16(w) && al16(packed), ALD_E_INVALID);
  CHECK(K % 32 == 0, ALD_E_UNSUPPORTED);
  launch_q4_pack(w, N, K, packed, scales, stream);
  return launched();
}

int ln_quant(const uint16_t* x, int64_t ldx, int M, int H, const float* gamma, const float* beta, float eps,
             uint16_t* u_out, int8_t* q, float* scale, hipStream_t stream) {
  CHECK(M >= 0 && H > 0, ALD_E_INVALID);
  if (M == 0) return ALD_OK;
  CHECK(x && gamma && beta && q && scale, ALD_E_INVALID);
  CHECK(H % 8 == 0 && ldx >= H && ldx % 8 == 0 && al16(x) && al16(gamma) && al16(beta) && al8(q), ALD_E_INVALID);
  if (u_out) CHECK(al16(u_out), ALD_E_INVALID);
  CHECK(H <= 8192, ALD_E_UNSUPPORTED);
  launch_ln_quant(x, ldx, M, H, gamma, beta, eps, u_out, q, scale, stream);
  return launched();
}

int ln_f16(const uint16_t* x, int64_t ldx, int M, int H, const float* gamma, const float* beta, float eps,
           uint16_t* y, int64_t ldy, hipStream_t stream) {
  CHECK(M >= 0 && H > 0, ALD_E_INVALID);
  if (M == 0) return ALD_OK;
  CHECK(x && gamma && beta && y, ALD_E_INVALID);
  CHECK(H % 8 == 0 && ldx >= H && ldy >= H && ldx % 8 == 0 && ldy % 8 == 0 && al16(x) && al16(y) && al16(gamma) &&
            al16(beta),
        ALD_E_INVALID);
  CHECK(H <= 8192, ALD_E_UNSUPPORTED);
  launch_ln_f16(x, ldx, M, H, gamma, beta, eps, y, ldy, stream);
  return launched();
}

int w8a8_linear(const uint16_t* x, int64_t ldx, int M, int K, const int8_t* wq, const float* w_scale, int N,
                const float* bias, const uint16_t* residual, int64_t ldr, int act, uint16_t* y, int64_t ldy,
                int8_t* xq, float* x_scale, int32_t* acc, unsigned flags, hipStream_t stream) {
  CHECK(M >= 0 && N >= 0 && K > 0, ALD_E_INVALID);
  CHECK((flags & ~ALD_PREQUANT) == 0, ALD_E_INVALID);
  int e = check_epilogue(M, N, residual, ldr, act, y, ldy);
  if (e) return e;
  if (M == 0 || N == 0) return ALD_OK;
  CHECK(wq && w_scale && xq && x_scale && (y || acc), ALD_E_INVALID);
  CHECK(K % 16 == 0 && al16(wq) && al16(xq), ALD_E_INVALID);
  CHECK(K <= 8192, ALD_E_UNSUPPORTED);
  if (!(flags & ALD_PREQUANT)) {
    CHECK(x && al16(x) && ldx >= K && ldx % 8 == 0, ALD_E_INVALID);
  }
  GemmArgs g;
  g.A = xq;
  g.lda = K;
  g.B = wq;
  g.M = M;
  g.N = N;
  g.K = K;
  g.epi.x_scale = x_scale;
  g.epi.w_scale = w_scale;
  g.epi.bias = bias;
  g.epi.residual = residual;
  g.epi.ldr = ldr;
  g.epi.y = y;
  g.epi.ldy = ldy;
  g.epi.acc = acc;
  g.epi.act = act;
  CHECK(gemm_supported(A_I8, B_I8, g), ALD_E_UNSUPPORTED);
  prepare();
  if (!(flags & ALD_PREQUANT)) launch_row_quant(x, ldx, M, K, xq, K, x_scale, stream);
  CHECK(launch_gemm(A_I8, B_I8, g, stream), ALD_E_UNSUPPORTED);
  return launched();
}

int q8w_linear(const uint16_t* x, int64_t ldx, int M, int K, const int8_t* wq, const float* w_scale, int N,
               const float* bias, const uint16_t* residual, int64_t ldr, int act, uint16_t* y, int64_t ldy,
               hipStream_t stream) {
  CHECK(M >= 0 && N >= 0 && K > 0, ALD_E_INVALID);
  int e = check_epilogue(M, N, residual, ldr, act, y, ldy);
  if (e) return e;
  if (M == 0 || N == 0) return ALD_OK;
  CHECK(x && wq && w_scale && y, ALD_E_INVALID);
  CHECK(al16(x) && al16(wq) && ldx >= K && ldx % 8 == 0, ALD_E_INVALID);
  CHECK(K % 64 == 0, ALD_E_UNSUPPORTED);
  GemmArgs g;
  g.A = x;
  g.lda = ldx;
  g.B = wq;
  g.M = M;
  g.N = N;
  g.K = K;
  g.epi.w_scale = w_scale;
  g.epi.bias = bias;
  g.epi.residual = residual;
  g.epi.ldr = ldr;
  g.epi.y = y;
  g.epi.ldy = ldy;
  g.epi.act = act;
  // only the direct-to-LDS GEMM implements this operand pair
  CHECK(gemm_supported(A_F16, B_I8, g), ALD_E_UNSUPPORTED);
  prepare();
  CHECK(launch_gemm(A_F16, B_I8, g, stream), ALD_E_UNSUPPORTED);
  return launched();
}

int q4_linear(const uint16_t* x, int64_t ldx, int M, int K, const uint8_t* wq4, const uint16_t* w_scale, int N,
              const float* bias, const uint16_t* residual, int64_t ldr, int act, uint16_t* y, int64_t ldy,
              hipStream_t stream) {
  CHECK(M >= 0 && N >= 0 && K > 0, ALD_E_INVALID);
  int e = check_epilogue(M, N, residual, ldr, act, y, ldy);
  if (e) return e;
  if (M == 0 || N == 0) return ALD_OK;
  CHECK(x && wq4 && w_scale && y, ALD_E_INVALID);
  CHECK(al16(x) && al16(wq4) && ldx >= K && ldx % 8 == 0, ALD_E_INVALID);
  CHECK(K % 32 == 0, ALD_E_UNSUPPORTED);
  prepare();
  GemmArgs g;
  g.A = x;
  g.lda = ldx;
  g.B = wq4;
  g.b_scale = w_scale;
  g.M = M;
  g.N = N;
  g.K = K;
  g.epi.bias = bias;
  g.epi.residual = residual;
  g.epi.ldr = ldr;
  g.epi.y = y;
  g.epi.ldy = ldy;
  g.epi.act = act;
  CHECK(gemm_supported(A_F16, B_Q4, g), ALD_E_UNSUPPORTED);
  CHECK(launch_gemm(A_F16, B_Q4, g, stream), ALD_E_UNSUPPORTED);
  return launched();
}

int f16_linear(const uint16_t* x, int64_t ldx, int M, int K, const uint16_t* w, int N, const float* bias,
               const uint16_t* residual, int64_t ldr, int act, uint16_t* y, int64_t ldy, hipStream_t stream) {
  CHECK(M >= 0 && N >= 0 && K > 0, ALD_E_INVALID);
  int e = check_epilogue(M, N, residual, ldr, act, y, ldy);
  if (e) return e;
  if (M == 0 || N == 0) return ALD_OK;
  CHECK(x && w && y, ALD_E_INVALID);
  CHECK(K % 8 == 0 && al16(x) && al16(w) && ldx >= K && ldx % 8 == 0, ALD_E_INVALID);
  prepare();
  GemmArgs g;
  g.A = x;
  g.lda = ldx;
  g.B = w;
  g.M = M;
  g.N = N;
  g.K = K;
  g.epi.bias = bias;
  g.epi.residual = residual;
  g.epi.ldr = ldr;
  g.epi.y = y;
  g.epi.ldy = ldy;
  g.epi.act = act;
  CHECK(gemm_supported(A_F16, B_F16, g), ALD_E_UNSUPPORTED);
  CHECK(launch_gemm(A_F16, B_F16, g, stream), ALD_E_UNSUPPORTED);
  return launched();
}

int attn_fwd(const uint16_t* q, const uint16_t* k, const uint16_t* v, int64_t q_stride, int64_t kv_stride,
             int n_heads, int head_dim, int batch, int Sq, int Sk, const int32_t* cu_seqlens_q,
             const int32_t* cu_seqlens_k, int max_sq, int max_sk, float scale, uint16_t* out, int64_t o_stride,
             hipStream_t stream) {
  CHECK(n_heads > 0 && batch >= 0, ALD_E_INVALID);
  CHECK(head_dim == 64, ALD_E_UNSUPPORTED);
  // the softmax keeps a running reference maximum in units of the scaled
  // score, which assumes a finite positive scale
  CHECK(std::isfinite(scale) && scale > 0.0f, ALD_E_INVALID);
  if (batch == 0) return ALD_OK;
  CHECK(q && k && v && out && al16(q) && al16(k) && al16(v) && al16(out), ALD_E_INVALID);
  const int64_t width = (int64_t)n_heads * 64;
  CHECK(q_stride >= width && kv_stride >= width && o_stride >= width, ALD_E_INVALID);
  CHECK(q_stride % 8 == 0 && kv_stride % 8 == 0 && o_stride % 8 == 0, ALD_E_INVALID);
  if (cu_seqlens_q) CHECK(max_sq >= 0, ALD_E_INVALID);
  else CHECK(Sq >= 0, ALD_E_INVALID);
  if (cu_seqlens_k) CHECK(max_sk >= 0, ALD_E_INVALID);
  else CHECK(Sk >= 0, ALD_E_INVALID);
  const int msq = cu_seqlens_q ? max_sq : Sq;
  if (msq == 0) return ALD_OK;
  AttnArgs a{q, k, v, out, q_stride, kv_stride, o_stride, n_heads, Sq, Sk, cu_seqlens_q, cu_seqlens_k,
             scale * 1.4426950408889634f};
  launch_attn(a, batch, msq, stream);
  return launched();
}

int steer_add(uint16_t* h, int64_t ldh, int M, int H, int rows_per_req, int R, const int32_t* row_req,
              const float* alpha, float resid_norm, const float* dir, int mode, hipStream_t stream) {
  CHECK(M >= 0 && H > 0, ALD_E_INVALID);
  CHECK(mode == ALD_STEER_ADD || mode == ALD_STEER_PROJECT, ALD_E_INVALID);
  if (M == 0) return ALD_OK;
  CHECK(h && alpha && dir && al16(h) && al16(dir), ALD_E_INVALID);
  CHECK(H % 8 == 0 && ldh >= H && ldh % 8 == 0, ALD_E_INVALID);
  CHECK(H <= 8192, ALD_E_UNSUPPORTED);
  if (!row_req) CHECK(rows_per_req > 0 && R > 0, ALD_E_INVALID);
  RowMap map{0, row_req ? 1 : rows_per_req, row_req ? 1 : R, row_req};
  launch_steer(h, ldh, M, H, map, alpha, resid_norm, dir, mode == ALD_STEER_PROJECT, stream);
  return launched();
}

int steer_latent(const float* x, float* x_out, int64_t n_tok, int C, int rows_per_req, int R,
                 const int32_t* row_req, const float* alpha, float resid_norm, const float* dir, int mode,
                 hipStream_t stream) {
  CHECK(n_tok >= 0 && C > 0, ALD_E_INVALID);
  CHECK(mode == ALD_STEER_ADD || mode == ALD_STEER_PROJECT, ALD_E_INVALID);
  if (n_tok == 0) return ALD_OK;
  CHECK(x && x_out && alpha && dir && x != x_out, ALD_E_INVALID);
  CHECK(al16(x) && al16(x_out) && al16(dir) && C % 4 == 0, ALD_E_INVALID);
  CHECK(C <= 512 && n_tok * (C / 4) < ((int64_t)1 << 31), ALD_E_UNSUPPORTED);
  if (!row_req) CHECK(rows_per_req > 0 && R > 0, ALD_E_INVALID);
  RowMap map{0, row_req ? 1 : rows_per_req, row_req ? 1 : R, row_req};
  launch_steer_latent(x, x_out, n_tok, C, map, alpha, resid_norm, dir, mode == ALD_STEER_PROJECT, stream);
  return launched();
}

int cfg_merge(const uint16_t* v, int64_t n_tok, int C, int rows_per_req, const int32_t* row_req, const float* w,
              float* v_hat, hipStream_t stream) {
  CHECK(n_tok >= 0 && C > 0, ALD_E_INVALID);
  if (n_tok == 0) return ALD_OK;
  CHECK(v && w && v_hat && al16(v) && al16(v_hat), ALD_E_INVALID);
  CHECK(C % 8 == 0, ALD_E_INVALID);
  CHECK(n_tok * (C / 4) < ((int64_t)1 << 31), ALD_E_UNSUPPORTED);
  if (!row_req) CHECK(rows_per_req > 0, ALD_E_INVALID);
  RowMap map{0, row_req ? 1 : rows_per_req, INT32_MAX, row_req};
  launch_cfg_merge(v, n_tok, C, map, w, v_hat, stream);
  return launched();
}

int sampler_update(int op, float* x, const float* v_hat, const float* x0, const float* eps, int64_t n_tok, int C,
                   int rows_per_req, const int32_t* row_req, const float* t_cur, const float* t_next,
                   const uint8_t* active, hipStream_t stream) {
  CHECK(op == ALD_EULER || op == ALD_RENOISE || op == ALD_DDIM || op == ALD_RENOISE_VP, ALD_E_INVALID);
  CHECK(n_tok >= 0 && C > 0, ALD_E_INVALID);
  if (n_tok == 0) return ALD_OK;
  CHECK(x && t_cur && al16(x) && C % 4 == 0, ALD_E_INVALID);
  CHECK(n_tok * (C / 4) < ((int64_t)1 << 31), ALD_E_UNSUPPORTED);
  if (!row_req) CHECK(rows_per_req > 0, ALD_E_INVALID);
  RowMap map{0, row_req ? 1 : rows_per_req, INT32_MAX, row_req};
  if (op == ALD_EULER || op == ALD_DDIM) {
    CHECK(v_hat && t_next && al16(v_hat), ALD_E_INVALID);
    if (op == ALD_EULER) launch_euler(x, v_hat, n_tok, C, map, t_cur, t_next, active, stream);
    else launch_ddim(x, v_hat, n_tok, C, map, t_cur, t_next, active, stream);
  } else {
    CHECK(x0 && eps && al16(x0) && al16(eps), ALD_E_INVALID);
    if (op == ALD_RENOISE) launch_renoise(x, x0, eps, n_tok, C, map, t_cur, active, stream);
    else launch_renoise_vp(x, x0, eps, n_tok, C, map, t_cur, active, stream);
  }
  return launched();
}

int ddim_alpha_bar(int T, double beta_1, double beta_T, const int32_t* timesteps, int n, float* abar_out) {
  CHECK(T >= 2 && n >= 0 && abar_out && (n == 0 || timesteps), ALD_E_INVALID);
  CHECK(beta_1 > 0.0 && beta_T > 0.0 && beta_1 < 1.0 && beta_T < 1.0, ALD_E_INVALID);
  for (int i = 0; i < n; ++i) CHECK(timesteps[i] >= 0 && timesteps[i] < T, ALD_E_INVALID);
  // the running product, one factor per training step, read at each grid timestep
  std::vector<double> ab(T);
  double prod = 1.0;
  for (int t = 0; t < T; ++t) {
    const double beta = beta_1 + (beta_T - beta_1) * t / (T - 1);
    prod *= 1.0 - beta;
    ab[t] = prod;
  }
  for (int i = 0; i < n; ++i) abar_out[i] = (float)ab[timesteps[i]];
  abar_out[n] = 1.0f;
  return ALD_OK;
}

size_t dit_workspace_size(const dit_config* cfg, int64_t max_tokens, int R) {
  if (check_config(cfg) != ALD_OK || max_tokens < 0 || R < 0) return 0;
  return carve_step(cfg, max_tokens, R, nullptr, SIZE_MAX, nullptr);
}

int dit_text_kv(const dit_config* c, const dit_weights* w, const uint16_t* text, int rows, uint16_t* kv_out,
                void* ws, size_t ws_bytes, hipStream_t stream) {
  int e = check_config(c);
  if (e) return e;
  e = check_weights(c, w);
  if (e) return e;
  CHECK(rows >= 0, ALD_E_INVALID);
  if (rows == 0 || c->n_blocks == 0) return ALD_OK;
  CHECK(text && kv_out && ws && al16(text) && al16(kv_out) && al16(ws), ALD_E_INVALID);
  const int Dt = c->text_dim, H = c->hidden;
  size_t need = align256((size_t)rows * Dt) + align256((size_t)rows * 4);
  CHECK(need <= ws_bytes, ALD_E_WORKSPACE);
  int8_t* codes = static_cast<int8_t*>(ws);
  float* xs = reinterpret_cast<float*>(static_cast<uint8_t*>(ws) + align256((size_t)rows * Dt));
  const void* A = c->wmode == ALD_W8A8 ? static_cast<const void*>(codes) : text;
  for (int l = 0; l < c->n_blocks; ++l) CHECK(linear_ok(w->blocks[l].kv, c->wmode, A, rows, Dt, 2 * H), ALD_E_UNSUPPORTED);
  prepare();
  if (c->wmode == ALD_W8A8) launch_row_quant(text, Dt, rows, Dt, codes, Dt, xs, stream);
  for (int l = 0; l < c->n_blocks; ++l)
    CHECK(run_linear(w->blocks[l].kv, c->wmode, A, Dt, xs, rows, Dt, 2 * H, nullptr, 0, 0,
                     kv_out + (int64_t)l * rows * 2 * H, 2 * H, stream),
          ALD_E_UNSUPPORTED);
  return launched();
}

int dit_step(const dit_config* cfg, const dit_weights* w, const dit_step_args* args, void* ws, size_t ws_bytes,
             hipStream_t stream) {
  return enqueue_step(cfg, w, args, ws, ws_bytes, stream);
}

int dit_step_static(const dit_config* cfg, const dit_weights* w, const dit_step_args* args, hipStream_t stream) {
  int e = check_config(cfg);
  if (e) return e;
  CHECK(args && args->R > 0 && args->n_tok > 0, ALD_E_INVALID);
  // the same carve dit_step takes from a caller workspace, here from the
  // device's scratch array; too large a step is refused before any launch
  const size_t need = carve_step(cfg, args->n_tok, args->R, nullptr, SIZE_MAX, nullptr);
  CHECK(need <= ALD_STATIC_SCRATCH_BYTES, ALD_E_WORKSPACE);
  void* ws = nullptr;
  e = device_scratch(&ws);
  if (e) return e;
  return enqueue_step(cfg, w, args, ws, ALD_STATIC_SCRATCH_BYTES, stream);
}

int dit_graph_capture(const dit_config* cfg, const dit_weights* w, const dit_step_args* args, int n_steps, void* ws,
                      size_t ws_bytes, hipStream_t stream, void** graph_out) {
  CHECK(args && graph_out && n_steps > 0, ALD_E_INVALID);
  CHECK(stream != nullptr, ALD_E_INVALID);  // the legacy null stream cannot be captured
  *graph_out = nullptr;
  // validate every step before opening the capture
  int e = check_config(cfg);
  if (e) return e;
  e = check_weights(cfg, w);
  if (e) return e;
  prepare();
  if (hipStreamBeginCapture(stream, hipStreamCaptureModeRelaxed) != hipSuccess) return ALD_E_LAUNCH;
  int rc = ALD_OK;
  for (int i = 0; i < n_steps && rc == ALD_OK; ++i) rc = enqueue_step(cfg, w, &args[i], ws, ws_bytes, stream);
  hipGraph_t graph = nullptr;
  hipError_t ce = hipStreamEndCapture(stream, &graph);
  if (rc != ALD_OK || ce != hipSuccess) {
    if (graph) (void)hipGraphDestroy(graph);
    return rc != ALD_OK ? rc : ALD_E_LAUNCH;
  }
  hipGraphExec_t exec = nullptr;
  if (hipGraphInstantiate(&exec, graph, nullptr, nullptr, 0) != hipSuccess) {
    (void)hipGraphDestroy(graph);
    return ALD_E_LAUNCH;
  }
  GraphHandle* gh = new (std::nothrow) GraphHandle{graph, exec};
  if (!gh) {
    (void)hipGraphExecDestroy(exec);
    (void)hipGraphDestroy(graph);
    return ALD_E_LAUNCH;
  }
  *graph_out = gh;
  return ALD_OK;
}

int dit_graph_launch(void* graph, hipStream_t stream) {
  CHECK(graph, ALD_E_INVALID);
  GraphHandle* gh = static_cast<GraphHandle*>(graph);
  return hipGraphLaunch(gh->exec, stream) == hipSuccess ? ALD_OK : ALD_E_LAUNCH;
}

int dit_graph_nodes(void* graph, size_t* n_nodes) {
  CHECK(graph && n_nodes, ALD_E_INVALID);
  GraphHandle* gh = static_cast<GraphHandle*>(graph);
  size_t n = 0;
  if (hipGraphGetNodes(gh->graph, nullptr, &n) != hipSuccess) return ALD_E_LAUNCH;
  *n_nodes = n;
  return ALD_OK;
}

int dit_graph_destroy(void* graph) {
  CHECK(graph, ALD_E_INVALID);
  GraphHandle* gh = static_cast<GraphHandle*>(graph);
  (void)hipGraphExecDestroy(gh->exec);
  (void)hipGraphDestroy(gh->graph);
  delete gh;
  return ALD_OK;
}

}  // extern "C"
