/*
 * ald.h -- C ABI of the MI355X (gfx950) audio-latent DiT denoise step.
 *
 * One denoising step of a text-conditioned audio-latent diffusion transformer
 * as described by "A Quantized Native Runtime for On-Device Semantic Audio
 * Generation" (aria): a DiT denoiser over the audio latent that cross-attends
 * to the text (Section II, reference model), run with 8-bit weights and
 * 8-bit arithmetic (W8A8), 8-bit weights alone, 4-bit weights or half
 * precision (Section III-A, runtime), with activation steering (the direction
 * added or projected onto, at a block's output, at the latent or at the text
 * conditioning) whose strength lives in device memory so that a captured step
 * loop never needs re-capture (Section III, steering; the Chinese summary of
 * the same paper gives the formula h <- h + alpha * ||h_bar|| * d_hat).
 * Classifier-free
 * guidance runs the cond row and its null-prompt companion in one batch and
 * merges them with w * cond + (1 - w) * uncond ("An Efficient vLLM-Based
 * Inference Pipeline for Unified Audio Understanding and Generation",
 * Section 2.4, Eq. (1)).  The sampler may warm-start from a cached clean
 * latent forward-noised to an intermediate step ("SoundWeaver: Semantic
 * Warm-Starting for Text-to-Audio Diffusion Serving", Section 2), under the
 * flow-matching Euler sampler or the DDIM sampler that page's backbones run.
 *
 * Conventions for every call:
 *   - Pointers are DEVICE pointers unless a parameter says "host".
 *   - The caller owns every buffer.  The library allocates no device memory
 *     and keeps no pointer between calls (the graph object of
 *     dit_graph_capture is the one exception: it records the pointers it was
 *     captured with, which must stay valid until it is destroyed).
 *   - fp16 tensors are IEEE binary16 bit patterns passed as uint16_t.
 *   - Matrices are row-major; leading dimensions (ld*) are in elements.
 *   - All work is enqueued on `stream`; calls never synchronise the host,
 *     never read device memory on the host, and can be captured into a
 *     hipGraph.
 *   - Arguments are validated on the host before any launch.  Return value:
 *     ALD_OK, or a negative ALD_E_* code; on error nothing was enqueued.
 *   - Vector accesses are 16 bytes wide: fp16/int8 row pointers and leading
 *     dimensions must give 16-byte aligned rows (ALD_E_INVALID otherwise).
 */
#ifndef ALD_H
#define ALD_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ALD_VERSION 202  /* 200: steering sites, W8A16, the DDIM sampler (new config and step fields);
                            201: dit_weights.kv_all (stacked text K/V linears);
                            202: dit_graph_nodes; attn_fwd rejects a non-positive scale; text_kv
                                 optional under text-site steering */

enum {
  ALD_OK = 0,
  ALD_E_INVALID = -1,      /* null pointer, misalignment, negative size, bad enum   */
  ALD_E_UNSUPPORTED = -2,  /* shape or operand pair the kernels do not cover
                              (e.g. head_dim != 64)                              */
  ALD_E_WORKSPACE = -3,    /* workspace smaller than dit_workspace_size()          */
  ALD_E_LAUNCH = -4        /* the HIP runtime reported an error after a launch      */
};

/* Weight precision of the block linears (aria, Section III-A: the precision
 * ladder fp16 / 8-bit / W8A8 / 4-bit; ALD_W8A16 is the 8-bit weight-only
 * rung). */
enum { ALD_W8A8 = 0, ALD_F16 = 1, ALD_Q4 = 2, ALD_W8A16 = 3 };

/* Epilogue activation. */
enum { ALD_ACT_NONE = 0, ALD_ACT_GELU = 1 };

/* w8a8_linear flags. */
#define ALD_PREQUANT 1u   /* xq / x_scale are inputs (already quantized); x unused */

/* sampler_update ops. */
enum { ALD_EULER = 0, ALD_RENOISE = 1, ALD_DDIM = 2, ALD_RENOISE_VP = 3 };

/* Samplers of the step: flow matching (velocity, Euler on t) or DDIM
 * (epsilon prediction, deterministic DDIM on alpha_bar). */
enum { ALD_SAMPLER_FLOW = 0, ALD_SAMPLER_DDIM = 1 };

/* steer_add modes (aria, Section III: add the direction, or project onto it). */
enum { ALD_STEER_ADD = 0, ALD_STEER_PROJECT = 1 };

/* Steering sites of the step (aria, Section III: the residual stream at a
 * block's output, the compact audio latent, the text conditioning). */
enum { ALD_SITE_RESIDUAL = 0, ALD_SITE_LATENT = 1, ALD_SITE_TEXT = 2 };

const char* ald_strerror(int code);
int ald_version(void);

/* ------------------------------------------------------------------------ *
 * Quantizers (aria, Section III-A: 8-bit weights, activations quantized   *
 * alongside weights for W8A8, 4-bit weights).                             *
 * ------------------------------------------------------------------------ */

/* Symmetric per-row int8 quantization of an fp16 [M, K] matrix (per-token
 * activation scales, or per-output-channel weight scales).
 *   amax = max |x| of the row; scale[m] = fp32(amax / 127);
 *   q = clamp(rint_half_even(fp32(x * fp32(127 / amax))), -127, 127);
 *   amax == 0 gives scale 0 and zero codes.
 * x [M, ldx] fp16; q [M, ldq] int8 out; scale [M] fp32 out.
 * K % 8 == 0 and K <= 8192 (one row is held in registers). */
int quantize_rows_q8(const uint16_t* x, int64_t ldx, int M, int K,
                     int8_t* q, int64_t ldq, float* scale, hipStream_t stream);

/* 4-bit weight packing, groups of 32 along K with fp16 scales:
 *   s = fp16(fp32(amax_g) / 7); q = clamp(rint(fp32(w) / fp32(s)), -7, 7)
 *   (s == 0 gives zero codes); two's-complement nibbles, byte j of a row holds
 *   k = 2j in the low nibble and k = 2j + 1 in the high nibble.
 * w [N, K] fp16 (dense); packed [N, K/2] out; scales [N, K/32] fp16 out.
 * K % 32 == 0. */
int quantize_q4(const uint16_t* w, int N, int K, uint8_t* packed,
                uint16_t* scales, hipStream_t stream);

/* LayerNorm over H (fp32 statistics, biased variance, affine gamma/beta),
 * rounded to fp16, then per-row int8 quantization of that fp16 row exactly
 * as quantize_rows_q8.  u_out [M, H] fp16 (optional, NULL to skip) receives
 * the fp16 LayerNorm output the codes were taken from; q [M, H] dense.
 * H % 8 == 0, H <= 8192. */
int ln_quant(const uint16_t* x, int64_t ldx, int M, int H, const float* gamma,
             const float* beta, float eps, uint16_t* u_out, int8_t* q,
             float* scale, hipStream_t stream);

/* LayerNorm to fp16 without quantization: y [M, ldy]. */
int ln_f16(const uint16_t* x, int64_t ldx, int M, int H, const float* gamma,
           const float* beta, float eps, uint16_t* y, int64_t ldy,
           hipStream_t stream);

/* ------------------------------------------------------------------------ *
 * Linear layers.  Weights are output-major: W [N, K], y = x W^T.           *
 * Epilogue (fp32, one rounding to fp16):                                   *
 *   y = act(acc * dequant + bias) + residual                               *
 * residual may alias y (in-place residual add: same ld required).          *
 * ------------------------------------------------------------------------ */

/* W8A8 linear (aria, Section III-A: 8-bit arithmetic on integer matrix
 * units, activations quantized with the weights).
 * Per-token dynamic quantization of x (as quantize_rows_q8) into xq/x_scale
 * (caller buffers, [M, K] and [M]) unless flags & ALD_PREQUANT, in which case
 * xq/x_scale are inputs and x may be NULL.  int8 x int8 -> int32 on MFMA;
 * dequant acc * x_scale[m] * w_scale[n].
 *   x [M, ldx] fp16; wq [N, K] int8 (dense); w_scale [N] fp32;
 *   bias [N] fp32 or NULL; residual [M, ldr] fp16 or NULL; act ALD_ACT_*;
 *   y [M, ldy] fp16 out (may be NULL when acc is given);
 *   acc [M, N] int32 out or NULL: the raw accumulators (bit-exact observable).
 * K % 16 == 0, K <= 8192. */
int w8a8_linear(const uint16_t* x, int64_t ldx, int M, int K,
                const int8_t* wq, const float* w_scale, int N,
                const float* bias, const uint16_t* residual, int64_t ldr,
                int act, uint16_t* y, int64_t ldy, int8_t* xq, float* x_scale,
                int32_t* acc, unsigned flags, hipStream_t stream);

/* 8-bit weight-only linear (aria, Section III-A: 8-bit weights, a rung of the
 * precision ladder distinct from W8A8): fp16 activations, int8 weights with
 * one fp32 scale per output channel (layout of quantize_rows_q8 applied to
 * the weights):
 *   y[m, n] = fp16( s[n] * sum_k x[m, k] q[n, k] + bias[n] (+GELU) (+res) )
 * The codes are widened to fp16 exactly inside the GEMM main loop, fp16 x
 * fp16 -> fp32 on MFMA, and the channel scale is applied in the epilogue
 * (equal in real arithmetic to x . (q s)).  wq [N, K] int8, w_scale [N] fp32.
 * K % 64 == 0, ldx % 8 == 0, x and wq 16-byte aligned (ALD_E_UNSUPPORTED /
 * ALD_E_INVALID otherwise). */
int q8w_linear(const uint16_t* x, int64_t ldx, int M, int K,
               const int8_t* wq, const float* w_scale, int N,
               const float* bias, const uint16_t* residual, int64_t ldr,
               int act, uint16_t* y, int64_t ldy, hipStream_t stream);

/* 4-bit weight-only linear (aria, Section III-A: the weights stored as 4-bit
 * integers, the rung of the precision ladder that fits the larger model on
 * small devices; the activations stay half precision): W = fp16(q * s)
 * dequantized inside the GEMM main loop, fp16 x fp16 -> fp32 on MFMA.
 * wq4 [N, K/2], w_scale [N, K/32] fp16 (layout of quantize_q4).  K % 32 == 0. */
int q4_linear(const uint16_t* x, int64_t ldx, int M, int K,
              const uint8_t* wq4, const uint16_t* w_scale, int N,
              const float* bias, const uint16_t* residual, int64_t ldr,
              int act, uint16_t* y, int64_t ldy, hipStream_t stream);

/* fp16-weight linear (aria, Section III-A: the GPU path's half-precision
 * tensor-core matrix multiplies), fp32 accumulation.  w [N, K] fp16 dense.
 * K % 8 == 0. */
int f16_linear(const uint16_t* x, int64_t ldx, int M, int K,
               const uint16_t* w, int N, const float* bias,
               const uint16_t* residual, int64_t ldr, int act, uint16_t* y,
               int64_t ldy, hipStream_t stream);

/* ------------------------------------------------------------------------ *
 * Attention (aria: half-precision attention on the GPU path; the DiT       *
 * self-attends over the latent and cross-attends to the text).             *
 * ------------------------------------------------------------------------ */

/* Non-causal softmax attention, fp16 in/out, fp32 softmax, head_dim 64.
 * Token-major layouts: q[(row) * q_stride + h * 64 + c]; k and v share
 * kv_stride; out[(row) * o_stride + h * 64 + c].
 * Sequence b (0 <= b < batch) uses query rows
 *   cu_seqlens_q ? [cu_q[b], cu_q[b+1]) : [b * Sq, (b+1) * Sq)
 * and key rows
 *   cu_seqlens_k ? [cu_k[b], cu_k[b+1]) : [b * Sk, (b+1) * Sk).
 * With cu_seqlens, max_sq / max_sk bound the lengths (host values); lengths
 * above them are a caller error (rows beyond are not computed).  A sequence
 * with no keys writes zeros.  scale multiplies q.k (e.g. 1/sqrt(64)); it must
 * be finite and > 0 (ALD_E_INVALID otherwise).
 * head_dim must be 64 (ALD_E_UNSUPPORTED otherwise); strides % 8 == 0. */
int attn_fwd(const uint16_t* q, const uint16_t* k, const uint16_t* v,
             int64_t q_stride, int64_t kv_stride, int n_heads, int head_dim,
             int batch, int Sq, int Sk, const int32_t* cu_seqlens_q,
             const int32_t* cu_seqlens_k, int max_sq, int max_sk, float scale,
             uint16_t* out, int64_t o_stride, hipStream_t stream);

/* ------------------------------------------------------------------------ *
 * Steering, CFG merge, sampler.                                           *
 * ------------------------------------------------------------------------ */

/* Residual-stream steering (aria, Section III: the direction is added, or
 * projected onto, at the chosen block's output; Chinese summary, activation
 * steering, for the additive formula): for every row m of h [M, ldh] fp16
 * with request r = row_req ? row_req[m] : (m / rows_per_req) % R and
 * strength a = alpha[r],
 *   ALD_STEER_ADD    : h[m, :] = fp16(h[m, :] + (a * resid_norm) * dir[:])
 *   ALD_STEER_PROJECT: h[m, :] = fp16(h[m, :] + (a * (h[m, :] . dir)) * dir[:])
 * (fp32 math; the projection strength carries no residual-norm unit and
 * resid_norm is ignored).  alpha [R] fp32 is read on the device at execution
 * time (a captured graph picks up new values without re-capture).  Rows with
 * a == 0 are not written at all, so the result is bit-identical to not
 * calling.  dir [H] fp32 unit direction.  H % 8 == 0, H <= 8192. */
int steer_add(uint16_t* h, int64_t ldh, int M, int H, int rows_per_req, int R,
              const int32_t* row_req, const float* alpha, float resid_norm,
              const float* dir, int mode, hipStream_t stream);

/* Latent-site steering (aria, Section III: the compact audio latent is an
 * injection site): x_out = x + (a * resid_norm) * dir (ALD_STEER_ADD) or
 * x + (a * (x . dir)) * dir (ALD_STEER_PROJECT) per token, one fp32 FMA per
 * value, with a = alpha[r] and r = row_req ? row_req[i] : (i / rows_per_req) % R.
 * Tokens with a == 0 are copied unchanged.  x, x_out fp32 [n_tok, C]
 * (distinct), dir [C] fp32; C % 4 == 0, C <= 512, n_tok * C / 4 below 2^31;
 * 16-byte aligned.  The step
 * feeds x_out to the model and keeps x as the sampler state. */
int steer_latent(const float* x, float* x_out, int64_t n_tok, int C, int rows_per_req, int R,
                 const int32_t* row_req, const float* alpha, float resid_norm,
                 const float* dir, int mode, hipStream_t stream);

/* CFG merge (vLLM audio pipeline page, Section 2.4, Eq. (1)) on the model
 * velocity: v [2 * n_tok, C] fp16 holds the cond rows [0, n_tok) then the
 * uncond rows [n_tok, 2 n_tok); token i belongs to request
 * r = row_req ? row_req[i] : i / rows_per_req, and
 *   v_hat[i, c] = w[r] * cond + (1 - w[r]) * uncond   (fp32)
 * w [R] fp32 device.  v_hat [n_tok, C] fp32 out.  C % 8 == 0; n_tok * C / 4
 * below 2^31 (else ALD_E_UNSUPPORTED). */
int cfg_merge(const uint16_t* v, int64_t n_tok, int C, int rows_per_req,
              const int32_t* row_req, const float* w, float* v_hat,
              hipStream_t stream);

/* Sampler update on the fp32 latent x [n_tok, C]; token i -> request r as in
 * cfg_merge; only requests with active[r] != 0 (or all, if active is NULL)
 * are written.
 *   ALD_EULER  : x += (t_next[r] - t_cur[r]) * v_hat       (flow-matching Euler)
 *   ALD_RENOISE: x  = (1 - t_cur[r]) * x0 + t_cur[r] * eps (warm start,
 *                SoundWeaver Section 2: forward-noise a cached clean latent
 *                to the skip time; eps is supplied by the caller).
 * For the DDIM ops (SoundWeaver, Section 3 setup: the backbones run the DDIM
 * sampler) t_cur / t_next hold alpha_bar at the current and the next grid
 * point instead of times, and v_hat is the guided epsilon prediction:
 *   ALD_DDIM      : x0 = (x - sqrt(1 - a) v_hat) / sqrt(a),
 *                   x  = sqrt(a') x0 + sqrt(1 - a') v_hat  (a = t_cur[r],
 *                   a' = t_next[r]; eta = 0; fp32; a' = 1 gives x0)
 *   ALD_RENOISE_VP: x = sqrt(a) x0 + sqrt(1 - a) eps      (warm start at the
 *                   skip point's alpha_bar a = t_cur[r])
 * Unused pointers (v_hat for the re-noise ops; x0, eps, t_next for the
 * updates) may be NULL.
 * C % 4 == 0; n_tok * C / 4 below 2^31 (else ALD_E_UNSUPPORTED). */
int sampler_update(int op, float* x, const float* v_hat, const float* x0,
                   const float* eps, int64_t n_tok, int C, int rows_per_req,
                   const int32_t* row_req, const float* t_cur,
                   const float* t_next, const uint8_t* active,
                   hipStream_t stream);

/* ------------------------------------------------------------------------ *
 * The whole step.                                                         *
 * ------------------------------------------------------------------------ */

typedef struct {
  int n_blocks;
  int hidden;        /* H                              */
  int n_heads;       /* H / 64                         */
  int head_dim;      /* must be 64                     */
  int mlp;           /* F                              */
  int channels;      /* latent channels C              */
  int text_tokens;   /* T                              */
  int text_dim;      /* D_t                            */
  int wmode;         /* ALD_W8A8 | ALD_F16 | ALD_Q4 | ALD_W8A16 */
  int steer_block;   /* block whose output is steered (residual site);
                        -1: no steering at any site */
  float ln_eps;
  int steer_mode;    /* ALD_STEER_ADD | ALD_STEER_PROJECT */
  int steer_site;    /* ALD_SITE_RESIDUAL | ALD_SITE_LATENT | ALD_SITE_TEXT */
  int sampler;       /* ALD_SAMPLER_FLOW | ALD_SAMPLER_DDIM */
} dit_config;

/* One linear layer's weights in the precision of dit_config.wmode:
 *   ALD_W8A8 and ALD_W8A16: w = int8 [N, K], scale = fp32 [N]
 *   ALD_F16 : w = fp16 [N, K], scale = NULL
 *   ALD_Q4  : w = uint8 [N, K/2], scale = fp16 [N, K/32]
 * bias fp32 [N]. */
typedef struct {
  const void* w;
  const void* scale;
  const float* bias;
} dit_linear;

/* Pre-LN residual block (reading of the pages' DiT): self-attention,
 * cross-attention to the text, GELU MLP, each h += f(LN(h)).
 * Shapes (N x K): qkv 3H x H, o H x H, q H x H, kv 2H x D_t, ox H x H,
 * up F x H, down H x F.  LayerNorm params fp32 [H]. */
typedef struct {
  const float *ln1_g, *ln1_b, *ln2_g, *ln2_b, *ln3_g, *ln3_b;
  dit_linear qkv, o, q, kv, ox, up, down;
} dit_block_weights;

typedef struct {
  const dit_block_weights* blocks; /* HOST array [n_blocks] of device pointers */
  const uint16_t* w_in;  /* fp16 [H, C]  input projection            */
  const float* b_in;     /* fp32 [H]                                  */
  const float* lnf_g;    /* fp32 [H]     final LayerNorm             */
  const float* lnf_b;
  const uint16_t* w_out; /* fp16 [C, H]  output projection           */
  const float* b_out;    /* fp32 [C]                                  */
  /* Optional (w == NULL: unused): the text K/V linears of every block stacked
   * along N, in the blocks' weight format: block l's output rows are
   * [l * 2H, (l + 1) * 2H) of w [n_blocks * 2H, D_t], with its scales and
   * biases in the same order.  With it, a step that steers the text site
   * projects the steered text for every block in one launch instead of one
   * per block; the results are bit-identical either way. */
  dit_linear kv_all;
} dit_weights;

/* Arguments of one step over R requests (2R CFG rows).
 * Latent rows are request-packed: request r owns tokens
 *   cu_seqlens ? [cu[r], cu[r+1]) : [r * seq, (r+1) * seq).
 * The hidden state holds the cond rows of all tokens, then the uncond rows.
 * All per-request arrays are device fp32 [R] read at execution time. */
typedef struct {
  float* x;                   /* fp32 [n_tok, C] latent state, updated in place */
  const uint16_t* text_kv;    /* fp16 [n_blocks][2R * T, 2H] from dit_text_kv;
                                 unused (may be NULL) with text-site steering    */
  int R;
  int seq;                    /* tokens per request when cu_seqlens == NULL     */
  const int32_t* cu_seqlens;  /* int32 [R + 1] or NULL                          */
  const int32_t* row_req;     /* int32 [n_tok] request of each token; required
                                 with cu_seqlens, ignored otherwise             */
  int64_t n_tok;              /* total latent tokens (host)                     */
  int max_seq;                /* longest request (host); = seq when dense       */
  const float* t_cur;
  const float* t_next;
  const float* guidance;      /* CFG weight w per request                       */
  const float* alpha;         /* steering strength per request for this step    */
  float resid_norm;           /* ||h_bar|| of the steered block (host)          */
  const float* direction;     /* fp32 unit steering direction: [H] residual site,
                                 [C] latent site, [D_t] text site               */
  const uint8_t* active;      /* uint8 [R]: requests whose latent is updated, or NULL (all) */
  const uint8_t* renoise;     /* uint8 [R]: requests re-noised at t_cur before the pass, or NULL */
  const float* x0;            /* fp32 [n_tok, C] cached clean latent (renoise)  */
  const float* eps;           /* fp32 [n_tok, C] re-noising draw (renoise)      */
  uint16_t* v_out;            /* optional fp16 [2 n_tok, C]: model velocity     */
  float* block_norms;         /* optional fp32 [2 n_tok]: per-row L2 norm of the
                                 steered block's output before steering         */
  const uint16_t* text;       /* fp16 [2R * T, D_t] text conditioning as given to
                                 dit_text_kv; read by the text site only         */
  const float* abar_cur;      /* DDIM: alpha_bar [R] at this step's grid point  */
  const float* abar_next;     /*       and at the next one (1 after the last)   */
} dit_step_args;

/* HOST helper for the DDIM sampler: alpha_bar of the noise schedule whose
 * betas run linearly from beta_1 to beta_T over T training steps,
 * alpha_bar[t] = prod_{s <= t} (1 - beta_s) (double precision), gathered at
 * the n grid timesteps (each in [0, T)) into abar_out[0..n-1], and
 * abar_out[n] = 1 (after the last step the clean estimate is returned).
 * abar_out holds n + 1 floats.  Host pointers; no device work. */
int ddim_alpha_bar(int T, double beta_1, double beta_T, const int32_t* timesteps, int n, float* abar_out);

/* Workspace bytes needed by dit_step / dit_text_kv for up to max_tokens
 * latent tokens (n_tok) and R requests. */
size_t dit_workspace_size(const dit_config* cfg, int64_t max_tokens, int R);

/* Step-invariant text keys/values: kv_out[l] = linear_kv_l(text) for every
 * block l, fp16 [n_blocks][rows, 2H].  text [rows, D_t] fp16 (the 2R CFG
 * rows x T tokens; the uncond rows are zeros, the null prompt). */
int dit_text_kv(const dit_config* cfg, const dit_weights* w,
                const uint16_t* text, int rows, uint16_t* kv_out, void* ws,
                size_t ws_bytes, hipStream_t stream);

/* One denoising step: input projection + time embedding, n_blocks DiT
 * blocks, final LayerNorm + output projection, CFG merge, sampler update
 * (with optional warm-start re-noise first).  ALD_SAMPLER_FLOW: the model
 * output is a velocity, Euler from t_cur to t_next, re-noise
 * (1 - t) x0 + t eps.  ALD_SAMPLER_DDIM: the model output is an epsilon
 * prediction, DDIM from abar_cur to abar_next, re-noise
 * sqrt(a) x0 + sqrt(1 - a) eps at abar_cur; t_cur feeds only the time
 * embedding (the grid timestep / T).  Steering (when steer_block >= 0), at
 * steer_site with operation steer_mode and strength alpha[r]:
 *   ALD_SITE_RESIDUAL: every row of request r after block steer_block;
 *   ALD_SITE_LATENT  : the latent fed to the input projection (steer_latent;
 *                      the sampler state x itself is not shifted); C <= 512;
 *   ALD_SITE_TEXT    : the cond text rows of request r (the null-prompt rows
 *                      are left alone), after which every block's text K/V is
 *                      recomputed from the steered text inside the step
 *                      (args->text required; args->text_kv is then unused).
 * Enqueues only; capturable. */
int dit_step(const dit_config* cfg, const dit_weights* w,
             const dit_step_args* args, void* ws, size_t ws_bytes,
             hipStream_t stream);

/* Largest workspace dit_step_static serves (bytes): dit_workspace_size() of
 * the call's config, tokens and requests must not exceed it (64 MiB covers
 * the mid-size model up to about 1800 latent tokens, or one request of the
 * serving model). */
#define ALD_STATIC_SCRATCH_BYTES (64u << 20)

/* dit_step without a caller workspace, for callers that cannot allocate
 * device memory (code under graph capture, tight serving loops, harnesses
 * that forbid allocation).  The step's scratch is a device array inside the
 * library, ALD_STATIC_SCRATCH_BYTES per device, held by every device the
 * library runs on until the process ends; the call itself allocates nothing.
 * Same arguments, arithmetic and results as dit_step.  Every call on one
 * device shares that device's array, and nothing in it needs to start
 * cleared (each region is written before it is read within a call): calls
 * (or replays of graphs that captured them) that overlap on one device race.
 * Returns ALD_E_WORKSPACE, before any launch, when the step needs more than
 * ALD_STATIC_SCRATCH_BYTES. */
int dit_step_static(const dit_config* cfg, const dit_weights* w,
                    const dit_step_args* args, hipStream_t stream);

/* Capture n_steps consecutive dit_step calls (args: HOST array [n_steps])
 * into one hipGraph on `stream` (aria: the per-step denoising loop is
 * captured once and replayed as a single GPU graph; per-step t, alpha and w
 * are read from device memory, so new values need no re-capture).
 * *graph_out receives an opaque handle. */
int dit_graph_capture(const dit_config* cfg, const dit_weights* w,
                      const dit_step_args* args, int n_steps, void* ws,
                      size_t ws_bytes, hipStream_t stream, void** graph_out);
int dit_graph_launch(void* graph, hipStream_t stream);
/* Number of nodes (kernel launches: the step records no copies or memsets)
 * in a captured graph, written to *n_nodes (host). */
int dit_graph_nodes(void* graph, size_t* n_nodes);
int dit_graph_destroy(void* graph);

#ifdef __cplusplus
}
#endif
#endif /* ALD_H */
