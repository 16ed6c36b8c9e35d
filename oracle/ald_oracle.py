"""CPU oracle for one denoising step of a text-conditioned audio-latent DiT.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute this module: only tests/, __graft_entry__.smoke() and the
cpu_baseline leg of bench.py do.  It shares no code with the HIP library;
the only module both sides use is ald_inputs (seeded shapes and draws).

Plain, slow and meant to be read against the pages:
  * "A Quantized Native Runtime for On-Device Semantic Audio Generation"
    (aria): the DiT denoiser with text cross-attention trained with flow
    matching (Section II, reference model); 8-bit weight storage, W8A8
    arithmetic that quantizes activations alongside weights, 4-bit storage,
    fp32 kept where fidelity is sensitive (Section III-A, runtime); the
    steering add at a chosen block's output, strength in units of the mean
    baseline residual norm, an exact no-op at zero strength and applied only
    inside a span of steps (Section III, steering).
  * The Chinese summary of the same paper (activation-steering prerequisite
    and method-step details): h <- h + alpha * ||h_bar|| * d_hat.
  * "An Efficient vLLM-Based Inference Pipeline for Unified Audio
    Understanding and Generation", Section 2.4, Eq. (1): the guided output
    w * cond + (1 - w) * uncond from a cond/uncond pair in one batch.
  * "SoundWeaver: Semantic Warm-Starting for Text-to-Audio Diffusion
    Serving", Section 2: warm start by forward-noising a cached clean latent
    to an intermediate step and running the reverse process from there.

Arithmetic is fp64 except where the contract fixes fp32: the quantizers
(codes must be bit-exact), the CFG merge and the sampler state.  Storage
precisions between operations follow the method: activations fp16, latent
state fp32.  A library matmul serves as a step only where its result is
exact (integer-valued operands, |sum| < 2**53) or where fp64 is the reference.

Parity pins for every function are in tests/test_oracle_*.py (closed forms,
brute force on tiny inputs, invariants, error bounds).  The whole-step
composition has no printed worked example on the pages: parity unpinned by
the pages, checked through its pinned parts and through invariants
(permutation equivariance, request independence, alpha = 0 identity,
guidance 1 = conditional branch).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Dict, List, Optional, Sequence

import numpy as np
from scipy.special import erf as _erf

F16 = np.float16
F32 = np.float32
F64 = np.float64


# --------------------------------------------------------------------------
# quantizers (aria, Section III-A: 8-bit weights and W8A8 activations; 4-bit)
# --------------------------------------------------------------------------

def quantize_rows_q8(u16: np.ndarray):
    """Symmetric per-row int8 quantization of an fp16 matrix.

    Used for per-token dynamic activation scales (W8A8) and for the
    per-output-channel weight scales (q8).  Reading of the pages, which leave
    the quantizer open: symmetric, codes in [-127, 127], amax = max |u| of the
    fp16-rounded row, scale s = fp32(amax / 127), codes
    clamp(rint(fp32(u * fp32(127 / amax))), -127, 127) with round-half-even;
    an all-zero row gives s = 0 and all-zero codes.
    Returns (codes int8 [M, K], scale fp32 [M]).
    """
    u = np.asarray(u16, dtype=F16).astype(F32)
    amax = np.max(np.abs(u), axis=1) if u.shape[1] else np.zeros(u.shape[0], F32)
    amax = amax.astype(F32)
    s = (amax / F32(127.0)).astype(F32)
    inv = np.zeros_like(amax)
    nz = amax > 0
    inv[nz] = F32(127.0) / amax[nz]
    prod = (u * inv[:, None]).astype(F32)
    q = np.clip(np.rint(prod), -127, 127).astype(np.int8)
    return q, s


def dequantize_rows_q8(q: np.ndarray, s: np.ndarray) -> np.ndarray:
    """fp64 value q * s of per-row int8 codes."""
    return q.astype(F64) * s.astype(F64)[:, None]


def quantize_q4(w16: np.ndarray, group: int = 32):
    """Symmetric 4-bit weight quantization with groups of `group` along K.

    Reading (aria lists 4-bit integer storage without the format; the group
    size 32 and fp16 scales come from the q4 workload): per group,
    s = fp16(fp32(amax) / 7) and codes clamp(rint(fp32(w) / fp32(s)), -7, 7);
    a zero scale gives zero codes.  Packing: two's-complement nibbles, byte j
    of a row holds k = 2j in its low nibble and k = 2j + 1 in its high nibble.
    Returns (packed uint8 [N, K/2], scales fp16 [N, K/group]).
    """
    w = np.asarray(w16, dtype=F16)
    N, K = w.shape
    assert K % group == 0 and K % 2 == 0
    g = w.astype(F32).reshape(N, K // group, group)
    amax = np.max(np.abs(g), axis=2).astype(F32)
    s16 = (amax / F32(7.0)).astype(F16)
    s32 = s16.astype(F32)
    q = np.zeros(g.shape, dtype=np.int64)
    nz = s32 > 0
    div = np.zeros(g.shape, dtype=F32)
    np.divide(g, s32[:, :, None], out=div, where=np.broadcast_to(nz[:, :, None], g.shape))
    q = np.clip(np.rint(div), -7, 7).astype(np.int64).reshape(N, K)
    nib = (q & 0xF).astype(np.uint8)
    packed = (nib[:, 0::2] | (nib[:, 1::2] << 4)).astype(np.uint8)
    return packed, s16


def unpack_q4(packed: np.ndarray) -> np.ndarray:
    """Signed codes int8 [N, K] from packed nibbles."""
    p = np.asarray(packed, dtype=np.uint8)
    lo = (p & 0xF).astype(np.int16)
    hi = (p >> 4).astype(np.int16)
    lo = np.where(lo >= 8, lo - 16, lo)
    hi = np.where(hi >= 8, hi - 16, hi)
    out = np.empty((p.shape[0], p.shape[1] * 2), dtype=np.int8)
    out[:, 0::2] = lo
    out[:, 1::2] = hi
    return out


def dequantize_q4(packed: np.ndarray, scales16: np.ndarray, group: int = 32) -> np.ndarray:
    """fp16 weights fp16(q * s): the product is exact in fp32, rounded once (RNE)."""
    q = unpack_q4(packed).astype(F32)
    N, K = q.shape
    s = np.repeat(np.asarray(scales16, dtype=F16).astype(F32), group, axis=1)
    return (q * s).astype(F16)


# --------------------------------------------------------------------------
# linear layers
# --------------------------------------------------------------------------

def int_gemm(qa: np.ndarray, qb: np.ndarray) -> np.ndarray:
    """acc[m, n] = sum_k qa[m, k] * qb[n, k], exact, as int64.

    The fp64 product of int8-valued matrices is exact while K * 127^2 < 2^53,
    so a library fp64 matmul serves as the (exact) integer sum.
    """
    K = qa.shape[1]
    assert qb.shape[1] == K
    assert K * 127 * 127 < 2 ** 53
    return (qa.astype(F64) @ qb.astype(F64).T).astype(np.int64)


def gelu(x: np.ndarray) -> np.ndarray:
    """Exact (erf) GELU, x * (1 + erf(x / sqrt 2)) / 2, in fp64."""
    x = np.asarray(x, dtype=F64)
    return 0.5 * x * (1.0 + _erf(x / math.sqrt(2.0)))


def _epilogue(y64, bias, residual, act):
    if bias is not None:
        y64 = y64 + np.asarray(bias, dtype=F64)[None, :]
    if act == 1:
        y64 = gelu(y64)
    if residual is not None:
        y64 = y64 + np.asarray(residual, dtype=F16).astype(F64)
    return y64.astype(F16)


@dataclass
class W8A8Result:
    y: np.ndarray        # fp16 [M, N]
    xq: np.ndarray       # int8 [M, K]
    x_scale: np.ndarray  # fp32 [M]
    acc: np.ndarray      # int64 [M, N]


def w8a8_linear(x16, wq, w_scale, bias=None, residual=None, act=0) -> W8A8Result:
    """W8A8 linear (aria, Section III-A: 8-bit arithmetic on integer tensor
    cores, activations quantized alongside the weights).

    Per-token dynamic activation quantization of the fp16 input, exact integer
    accumulation, then y = fp16(act(acc * s_x * s_w + bias) + residual) with
    the dequant/bias/residual done in fp64 and rounded once.
    """
    xq, sx = quantize_rows_q8(x16)
    acc = int_gemm(xq, wq)
    y64 = acc.astype(F64) * sx.astype(F64)[:, None] * np.asarray(w_scale, F32).astype(F64)[None, :]
    return W8A8Result(_epilogue(y64, bias, residual, act), xq, sx, acc)


def f16_linear(x16, w16, bias=None, residual=None, act=0) -> np.ndarray:
    """fp16-weight linear: fp16 operands, wide accumulation, fp16 output
    (aria: half-precision matrix multiplies on the GPU path)."""
    y64 = np.asarray(x16, F16).astype(F64) @ np.asarray(w16, F16).astype(F64).T
    return _epilogue(y64, bias, residual, act)


def q8w_linear(x16, wq, w_scale, bias=None, residual=None, act=0) -> np.ndarray:
    """8-bit weight-only linear (aria, Section III-A: 8-bit weight storage;
    the activations stay fp16).  The weight is its dequantized value
    W[n, k] = q[n, k] * s[n] in fp64; y = fp16(act(x . W^T + bias) + residual)."""
    w64 = np.asarray(wq, np.int8).astype(F64) * np.asarray(w_scale, F32).astype(F64)[:, None]
    y64 = np.asarray(x16, F16).astype(F64) @ w64.T
    return _epilogue(y64, bias, residual, act)


def q4_linear(x16, packed, scales16, bias=None, residual=None, act=0, group=32) -> np.ndarray:
    """4-bit weight-only linear: weights dequantized to fp16, then as f16_linear."""
    return f16_linear(x16, dequantize_q4(packed, scales16, group), bias, residual, act)


# --------------------------------------------------------------------------
# normalisation, attention, timestep embedding
# --------------------------------------------------------------------------

def layer_norm(x16, gamma, beta, eps=1e-5) -> np.ndarray:
    """LayerNorm over the last axis in fp64 (biased variance), output fp16."""
    x = np.asarray(x16, F16).astype(F64)
    mu = x.mean(axis=-1, keepdims=True)
    var = ((x - mu) ** 2).mean(axis=-1, keepdims=True)
    y = (x - mu) / np.sqrt(var + eps) * np.asarray(gamma, F64) + np.asarray(beta, F64)
    return y.astype(F16)


def attention(q16, k16, v16, scale) -> np.ndarray:
    """Non-causal softmax attention of one sequence and one head group.

    q [Sq, nh, d], k/v [Sk, nh, d] fp16 -> out [Sq, nh, d] fp16.  fp64 scores,
    max-subtracted softmax, fp64 weighted sum, one rounding to fp16.
    """
    q = np.asarray(q16, F16).astype(F64).transpose(1, 0, 2)
    k = np.asarray(k16, F16).astype(F64).transpose(1, 0, 2)
    v = np.asarray(v16, F16).astype(F64).transpose(1, 0, 2)
    s = (q @ k.transpose(0, 2, 1)) * float(scale)
    s = s - s.max(axis=-1, keepdims=True)
    p = np.exp(s)
    p = p / p.sum(axis=-1, keepdims=True)
    o = p @ v
    return o.transpose(1, 0, 2).astype(F16)


def attention_varlen(q16, k16, v16, cu_q, cu_k, n_heads, scale) -> np.ndarray:
    """Packed variable-length attention: sequence b uses query rows
    [cu_q[b], cu_q[b+1]) and key rows [cu_k[b], cu_k[b+1]).  q/k/v are
    [tokens, n_heads * d]; output [tokens_q, n_heads * d]."""
    q16 = np.asarray(q16, F16)
    Mq, Hd = q16.shape
    d = Hd // n_heads
    out = np.zeros((Mq, Hd), dtype=F16)
    for b in range(len(cu_q) - 1):
        q0, q1, k0, k1 = int(cu_q[b]), int(cu_q[b + 1]), int(cu_k[b]), int(cu_k[b + 1])
        if q1 == q0:
            continue
        if k1 == k0:
            continue  # no keys: output rows stay zero
        o = attention(q16[q0:q1].reshape(-1, n_heads, d),
                      np.asarray(k16[k0:k1], F16).reshape(-1, n_heads, d),
                      np.asarray(v16[k0:k1], F16).reshape(-1, n_heads, d), scale)
        out[q0:q1] = o.reshape(q1 - q0, Hd)
    return out


def timestep_embedding(t: np.ndarray, H: int) -> np.ndarray:
    """Sinusoidal embedding of the flow time (reading: the pages say only that
    the DiT is time-conditioned): omega_j = exp(-ln(1e4) * j / (H/2)),
    temb[j] = sin(1000 t omega_j) for j < H/2 and cos(1000 t omega_{j-H/2})
    after.  t [n] -> [n, H] fp64."""
    half = H // 2
    j = np.arange(half, dtype=F64)
    om = np.exp(-math.log(1e4) * j / half)
    a = 1000.0 * np.asarray(t, F64)[:, None] * om[None, :]
    return np.concatenate([np.sin(a), np.cos(a)], axis=1)


# --------------------------------------------------------------------------
# steering, CFG merge, sampler (the method's own operations)
# --------------------------------------------------------------------------

def steer_add(h16, row_alpha, resid_norm, direction) -> np.ndarray:
    """Residual-stream steering (aria, Section III; Chinese summary, activation
    steering): h <- h + alpha * ||h_bar|| * d_hat at the chosen block output.

    Rows whose strength is exactly 0 are returned untouched (bit-identical
    to the unsteered pass).  Other rows: fp64 sum rounded once to fp16.
    """
    h = np.array(h16, dtype=F16, copy=True)
    a = np.asarray(row_alpha, dtype=F32)
    rows = np.nonzero(a != 0)[0]
    if rows.size:
        c = a[rows].astype(F64) * float(resid_norm)
        h[rows] = (h[rows].astype(F64) + c[:, None] * np.asarray(direction, F32).astype(F64)[None, :]).astype(F16)
    return h


def steer_project(h16, row_beta, direction) -> np.ndarray:
    """Projection steering (aria, Section III: the direction is either added
    or projected onto; the steering ablation compares the additive strength
    alpha with a projection strength beta).  Reading: projection
    amplification, h <- h + beta * (h . d_hat) * d_hat, which scales the
    component of h along d_hat by (1 + beta) and leaves the orthogonal part
    alone; beta carries no residual-norm unit (the dot product already does).

    Rows whose strength is exactly 0 are returned untouched.  Other rows: the
    dot product and the sum in fp64, rounded once to fp16.
    """
    h = np.array(h16, dtype=F16, copy=True)
    b = np.asarray(row_beta, dtype=F32)
    rows = np.nonzero(b != 0)[0]
    if rows.size:
        d = np.asarray(direction, F32).astype(F64)
        hr = h[rows].astype(F64)
        c = b[rows].astype(F64) * (hr @ d)
        h[rows] = (hr + c[:, None] * d[None, :]).astype(F16)
    return h


def steer_latent(x32, row_alpha, resid_norm, direction, mode="add") -> np.ndarray:
    """Steering at the compact audio latent (aria, Section III: the latent is
    one of three injection sites, beside the residual stream and the text
    conditioning).  Reading: the shift applies to the denoiser's input at the
    steered step, not to the sampler state, as a hook on the model input would.

    x32: fp32 [N, C] latent state; returns the fp16 model input [N, C].  Rows
    whose strength is exactly 0 are fp16(x) (the unsteered input); others
    x + a * resid_norm * d (add) or x + a * (x . d) * d (project) in fp64,
    rounded once to fp16.
    """
    x = np.asarray(x32, F32)
    out = x.astype(F16)
    a = np.asarray(row_alpha, dtype=F32)
    rows = np.nonzero(a != 0)[0]
    if rows.size:
        d = np.asarray(direction, F32).astype(F64)
        xr = x[rows].astype(F64)
        if mode == "project":
            c = a[rows].astype(F64) * (xr @ d)
        elif mode == "add":
            c = a[rows].astype(F64) * float(resid_norm)
        else:
            raise ValueError(mode)
        out[rows] = (xr + c[:, None] * d[None, :]).astype(F16)
    return out


def steer_text(text16, R, T, alpha_req, resid_norm, direction, mode="add") -> np.ndarray:
    """Steering at the text conditioning (aria, Section III, third injection
    site).  text16: fp16 [2R*T, D_t], the cond rows of request r at
    [r*T, (r+1)*T), then the null-prompt rows.  Reading: only the cond rows
    carry text conditioning, so only they are steered (strength alpha_req[r]);
    the null prompt stays as it is.  Same arithmetic as the residual site."""
    t = np.asarray(text16, F16).reshape(2 * R * T, -1)
    row_alpha = np.zeros(2 * R * T, F32)
    row_alpha[:R * T] = np.repeat(np.asarray(alpha_req, F32), T)
    if mode == "project":
        return steer_project(t, row_alpha, direction)
    if mode == "add":
        return steer_add(t, row_alpha, resid_norm, direction)
    raise ValueError(mode)


def cfg_merge(v_cond16, v_uncond16, w) -> np.ndarray:
    """Classifier-free-guidance merge of the vLLM audio pipeline page,
    Section 2.4, Eq. (1), applied to the velocity: w * cond + (1 - w) * uncond,
    evaluated in that form in fp32 (so w = 1 returns the cond branch)."""
    c = np.asarray(v_cond16, F16).astype(F32)
    u = np.asarray(v_uncond16, F16).astype(F32)
    w = np.asarray(w, F32)
    return (w * c + (F32(1.0) - w) * u).astype(F32)


def euler_update(x, v_hat, t_cur, t_next) -> np.ndarray:
    """Flow-matching Euler step x <- x + (t_next - t_cur) * v_hat in fp32
    (rectified-flow reading of 'trained with flow matching', t from 1 to 0)."""
    x = np.asarray(x, F32)
    dt = (np.asarray(t_next, F32) - np.asarray(t_cur, F32)).astype(F32)
    return (x + dt * np.asarray(v_hat, F32)).astype(F32)


def renoise(x0, eps, t) -> np.ndarray:
    """Warm start (SoundWeaver, Section 2): a sample of the forward process
    q(x_t | x0_hat) at the skip time t, x_t = (1 - t) x0 + t eps under the
    rectified-flow convention, in fp32."""
    t = np.asarray(t, F32)
    return ((F32(1.0) - t) * np.asarray(x0, F32) + t * np.asarray(eps, F32)).astype(F32)


def ddpm_alpha_bar(T: int, beta_1: float, beta_T: float) -> np.ndarray:
    """Cumulative signal fraction of a diffusion noise schedule with betas
    linear from beta_1 to beta_T over T training steps (the schedule of the
    DDPM paper; the pages name the DDIM sampler but not its schedule):
    alpha_bar[t] = prod_{s <= t} (1 - beta_s), t = 0..T-1, fp64."""
    beta = np.linspace(beta_1, beta_T, T, dtype=F64)
    return np.cumprod(1.0 - beta)


def ddim_update(x, eps_hat, abar_cur, abar_next) -> np.ndarray:
    """Deterministic DDIM step (eta = 0) on an epsilon prediction: first the
    clean-latent estimate x0 = (x - sqrt(1 - a) eps) / sqrt(a), then the
    latent at the next grid point sqrt(a') x0 + sqrt(1 - a') eps.  fp64, the
    new state rounded once to fp32.  a' = 1 (the end of the grid) returns x0."""
    x = np.asarray(x, F32).astype(F64)
    e = np.asarray(eps_hat, F32).astype(F64)
    a = np.asarray(abar_cur, F32).astype(F64)
    an = np.asarray(abar_next, F32).astype(F64)
    x0 = (x - np.sqrt(1.0 - a) * e) / np.sqrt(a)
    return (np.sqrt(an) * x0 + np.sqrt(1.0 - an) * e).astype(F32)


def renoise_vp(x0, eps, abar) -> np.ndarray:
    """Warm start under the DDIM sampler (SoundWeaver, Section 2: a sample of
    the forward process q(x_t* | x0_hat)): sqrt(a) x0 + sqrt(1 - a) eps at the
    skip point's alpha_bar a, fp64 rounded to fp32."""
    a = np.asarray(abar, F32).astype(F64)
    return (np.sqrt(a) * np.asarray(x0, F32).astype(F64)
            + np.sqrt(1.0 - a) * np.asarray(eps, F32).astype(F64)).astype(F32)


def ddim_alpha_bars(cfg, timesteps) -> np.ndarray:
    """alpha_bar at each grid point of a DDIM run over the given descending
    training timesteps, with 1 after the last (so the last step returns the
    clean estimate), rounded to the fp32 the sampler state uses; [N + 1]."""
    ab = ddpm_alpha_bar(cfg.train_steps, cfg.beta_1, cfg.beta_T)
    return np.concatenate([ab[np.asarray(timesteps, np.int64)], [1.0]]).astype(F32)


def skip_start_step(p: float, n_steps: int) -> int:
    """Steps skipped for a skip fraction p: k = floor(p * N + 1/2)."""
    return int(math.floor(p * n_steps + 0.5))


# --------------------------------------------------------------------------
# the DiT model
# --------------------------------------------------------------------------

@dataclass
class PreparedLinear:
    mode: str
    w16: np.ndarray
    bias: np.ndarray
    wq: Optional[np.ndarray] = None
    ws: Optional[np.ndarray] = None
    q4: Optional[np.ndarray] = None
    q4s: Optional[np.ndarray] = None

    def __call__(self, x16, residual=None, act=0):
        if self.mode == "w8a8":
            return w8a8_linear(x16, self.wq, self.ws, self.bias, residual, act).y
        if self.mode == "q4":
            return q4_linear(x16, self.q4, self.q4s, self.bias, residual, act)
        if self.mode == "w8a16":
            return q8w_linear(x16, self.wq, self.ws, self.bias, residual, act)
        return f16_linear(x16, self.w16, self.bias, residual, act)


def prepare_linear(w16, bias, mode) -> PreparedLinear:
    p = PreparedLinear(mode, np.asarray(w16, F16), np.asarray(bias, F32))
    if mode in ("w8a8", "w8a16"):
        p.wq, p.ws = quantize_rows_q8(p.w16)
    elif mode == "q4":
        p.q4, p.q4s = quantize_q4(p.w16)
    elif mode != "f16":
        raise ValueError(mode)
    return p


@dataclass
class PreparedModel:
    cfg: object
    params: object
    lin: List[Dict[str, PreparedLinear]]


def prepare_model(cfg, params) -> PreparedModel:
    lin = []
    for blk in params.blocks:
        lin.append({name: prepare_linear(blk.w[name], blk.b[name], cfg.wmode) for name in blk.w})
    return PreparedModel(cfg, params, lin)


def text_kv(model: PreparedModel, text16: np.ndarray) -> List[np.ndarray]:
    """Per-block text keys/values, fp16 [2R*T, 2H]: the cross-attention
    projection of the text conditioning.  It does not depend on the step, so
    it is computed once per request (same arithmetic as inside the step)."""
    cfg = model.cfg
    t = np.asarray(text16, F16).reshape(-1, cfg.text_dim)
    return [lin["kv"](t) for lin in model.lin]


@dataclass
class StepTrace:
    v: Optional[np.ndarray] = None            # fp16 [2N, C] model velocity
    v_hat: Optional[np.ndarray] = None        # fp32 [N, C] guided velocity
    block_out: Dict[int, np.ndarray] = field(default_factory=dict)  # fp16 [2N, H]


def dit_forward(model: PreparedModel, x: np.ndarray, seqlens: Sequence[int], kv: List[np.ndarray],
                t_cur: np.ndarray, row_alpha_req: np.ndarray, resid_norm: float,
                direction: np.ndarray, keep_blocks: Sequence[int] = (),
                text16: Optional[np.ndarray] = None) -> (np.ndarray, StepTrace):
    """Model velocity v (fp16, [cond tokens | uncond tokens] x C) for the
    packed latent x (fp32 [N, C]) of R requests with per-request t and
    steering strength.  The steering site is cfg.steer_site: "residual" (the
    chosen block's output), "latent" (the model input) or "text" (the cond
    text conditioning, whose keys/values are then recomputed from the steered
    text; text16 is required for it).

    Block topology (reading; the pages say only that each block writes an
    additive update into a residual stream and that the denoiser
    cross-attends to the text): pre-LN residual block
      h += O(SelfAttn(W8A8 QKV(LN1 h)));  h += Ox(CrossAttn(Q(LN2 h), text K/V));
      h += Down(GELU(Up(LN3 h)));  steering add at the chosen block output.
    Input projection adds a sinusoidal time embedding; no positional encoding.
    """
    cfg = model.cfg
    P = model.params
    H, C, nh, T = cfg.hidden, cfg.channels, cfg.n_heads, cfg.text_tokens
    d = H // nh
    R = len(seqlens)
    cu = np.concatenate([[0], np.cumsum(seqlens)]).astype(np.int64)
    Ntot = int(cu[-1])
    req_of_tok = np.repeat(np.arange(R), np.asarray(seqlens, dtype=np.int64))
    # rows: [cond tokens (request-packed) | uncond tokens]; both rows of a
    # CFG pair see the same latent (the companion is kept in sync with the
    # main request, vLLM audio pipeline page, Section 2.4)
    site = getattr(cfg, "steer_site", "residual")
    steering = cfg.steer_block >= 0
    if steering and site == "latent":
        x_in = steer_latent(x, np.asarray(row_alpha_req, F32)[req_of_tok], resid_norm, direction, cfg.steer_mode)
    else:
        x_in = np.asarray(x, F32).astype(F16)
    if steering and site == "text":
        kv = text_kv(model, steer_text(text16, R, T, row_alpha_req, resid_norm, direction, cfg.steer_mode))
    x2 = np.concatenate([x_in, x_in], axis=0)
    req_of_row = np.concatenate([req_of_tok, req_of_tok])
    t_row = np.asarray(t_cur, F32)[req_of_row]
    temb = timestep_embedding(t_row, H)
    h64 = x2.astype(F64) @ P.w_in.astype(F64).T
    h = (h64 + P.b_in.astype(F64)[None, :] + temb).astype(F16)
    cu_q = np.concatenate([cu, Ntot + cu[1:]])       # 2R sequences
    cu_t = np.arange(2 * R + 1, dtype=np.int64) * T  # text rows per CFG row
    scale = 1.0 / math.sqrt(d)
    row_alpha = np.asarray(row_alpha_req, F32)[req_of_row]
    trace = StepTrace()
    for li, blk in enumerate(P.blocks):
        lin = model.lin[li]
        u = layer_norm(h, blk.ln1_g, blk.ln1_b, cfg.ln_eps)
        qkv = lin["qkv"](u)
        o = attention_varlen(qkv[:, :H], qkv[:, H:2 * H], qkv[:, 2 * H:], cu_q, cu_q, nh, scale)
        h = lin["o"](o, residual=h)
        u = layer_norm(h, blk.ln2_g, blk.ln2_b, cfg.ln_eps)
        qx = lin["q"](u)
        ox = attention_varlen(qx, kv[li][:, :H], kv[li][:, H:], cu_q, cu_t, nh, scale)
        h = lin["ox"](ox, residual=h)
        u = layer_norm(h, blk.ln3_g, blk.ln3_b, cfg.ln_eps)
        g = lin["up"](u, act=1)
        h = lin["down"](g, residual=h)
        if li in keep_blocks:
            trace.block_out[li] = h.copy()
        if steering and site == "residual" and li == cfg.steer_block:
            if cfg.steer_mode == "project":
                h = steer_project(h, row_alpha, direction)
            else:
                h = steer_add(h, row_alpha, resid_norm, direction)
    u = layer_norm(h, P.lnf_g, P.lnf_b, cfg.ln_eps)
    v = f16_linear(u, P.w_out, P.b_out)
    trace.v = v
    return v, trace


def dit_step(model: PreparedModel, x: np.ndarray, seqlens: Sequence[int], kv: List[np.ndarray],
             t_cur, t_next, guidance, row_alpha_req, resid_norm, direction,
             active: Optional[np.ndarray] = None, keep_blocks: Sequence[int] = (),
             text16: Optional[np.ndarray] = None, abar_cur=None, abar_next=None):
    """One denoising step for all requests: model pass on the CFG pair, merge,
    sampler update.  Requests whose `active` flag is false keep their latent.
    cfg.sampler "flow": the model output is a velocity and the update the
    flow-matching Euler step from t_cur to t_next; "ddim": the model output is
    an epsilon prediction (reading) and the update the DDIM step from
    abar_cur to abar_next (per request), t_cur feeding only the time
    embedding."""
    R = len(seqlens)
    seqlens = np.asarray(seqlens, dtype=np.int64)
    Ntot = int(seqlens.sum())
    v, trace = dit_forward(model, x, seqlens, kv, t_cur, row_alpha_req, resid_norm, direction, keep_blocks,
                           text16)
    req = np.repeat(np.arange(R), seqlens)
    w = np.asarray(guidance, F32)[req][:, None]
    v_hat = cfg_merge(v[:Ntot], v[Ntot:], w)
    if getattr(model.cfg, "sampler", "flow") == "ddim":
        x_new = ddim_update(x, v_hat, np.asarray(abar_cur, F32)[req][:, None],
                            np.asarray(abar_next, F32)[req][:, None])
    else:
        tc = np.asarray(t_cur, F32)[req][:, None]
        tn = np.asarray(t_next, F32)[req][:, None]
        x_new = euler_update(x, v_hat, tc, tn)
    if active is not None:
        keep = ~np.asarray(active, bool)[req]
        x_new[keep] = np.asarray(x, F32)[keep]
    trace.v_hat = v_hat
    return x_new, trace


def mean_row_norm(h16: np.ndarray) -> float:
    """Mean over tokens of the per-token L2 norm (the 'mean baseline residual
    norm' that sets the steering unit; reading: mean of norms)."""
    h = np.asarray(h16, F16).astype(F64)
    return float(np.mean(np.sqrt(np.sum(h * h, axis=1))))


def run_sampler(model: PreparedModel, inp, kv=None, resid_norm: float = 0.0,
                steps: Optional[Sequence[int]] = None, keep_blocks: Sequence[int] = (),
                alpha_override: Optional[np.ndarray] = None):
    """Run global steps i (default all N) over every request.

    Request r is active at step i when i >= start_step[r]; a warm request is
    re-noised to t_{start} just before its first step (SoundWeaver, Section 2).
    Returns the final latent and the per-step traces.
    """
    tg = np.asarray(inp.t_grid, F32)
    N = len(tg) - 1
    ddim = getattr(model.cfg, "sampler", "flow") == "ddim"
    ab = ddim_alpha_bars(model.cfg, inp.timesteps) if ddim else None
    if kv is None:
        kv = text_kv(model, inp.text)
    x = np.array(inp.x, dtype=F32, copy=True)
    R = len(inp.seqlens)
    req = np.repeat(np.arange(R), np.asarray(inp.seqlens, dtype=np.int64))
    alpha = inp.alpha if alpha_override is None else alpha_override
    traces = []
    for i in (range(N) if steps is None else steps):
        start = np.asarray(inp.start_step)
        if inp.x0 is not None:
            rn = (start == i) & (start > 0)
            if rn.any():
                rows = rn[req]
                x[rows] = (renoise_vp(inp.x0[rows], inp.eps[rows], ab[i]) if ddim
                           else renoise(inp.x0[rows], inp.eps[rows], tg[i]))
        active = start <= i
        t_cur = np.full(R, tg[i], F32)
        t_next = np.full(R, tg[i + 1], F32)
        x, tr = dit_step(model, x, inp.seqlens, kv, t_cur, t_next, inp.guidance, alpha[i],
                         resid_norm, inp.direction, active, keep_blocks, inp.text,
                         None if ab is None else np.full(R, ab[i], F32),
                         None if ab is None else np.full(R, ab[i + 1], F32))
        traces.append(tr)
    return x, traces


def normwise_rel_err(got: np.ndarray, ref: np.ndarray) -> float:
    """max_i |g_i - o_i| / max_i |o_i| (the step-output parity metric)."""
    got = np.asarray(got, F64)
    ref = np.asarray(ref, F64)
    den = np.max(np.abs(ref))
    return float(np.max(np.abs(got - ref)) / den) if den > 0 else float(np.max(np.abs(got - ref)))
