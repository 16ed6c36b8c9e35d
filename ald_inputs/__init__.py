"""Seeded synthetic workloads for the DiT denoise step.

This module is shared by the oracle and the HIP path, so it holds shapes and
random draws only -- none of the method's arithmetic (no quantization, no
normalisation beyond making the steering direction a unit vector, which is an
input the method receives, not a step it performs).

Shapes follow the five workloads of the audio-latent-diffusion study:
  tiny   : 2 blocks, hidden 256, 4 heads, latent 64 x 64, text 32 x 256, 1 request
  mid    : 16 blocks, hidden 1024, 16 heads, MLP 4096, latent 256, text 128 x 768
  serve  : 24 blocks, hidden 1536, 24 heads, MLP 6144, latent 512, 8 requests
  q4     : 24 blocks, hidden 2048, 32 heads, MLP 8192, latent 1024, 4 requests
  mixed  : the mid model, 32 requests of latent length in {128..1024}
Every request is a classifier-free-guidance pair: B = 2R rows laid out as
[cond rows 0..R-1 | uncond rows 0..R-1]; the uncond rows see a zero text tensor
(the "null prompt" companion of the vLLM audio pipeline page, section 2.4).

Distributions: weights N(0, 0.02) rounded to fp16; biases N(0, 0.02) fp32;
LayerNorm gamma 1 + N(0, 0.02), beta N(0, 0.02); latents and text N(0, 1)
(text stored fp16); steering direction a seeded Gaussian scaled to unit length.
"""
from __future__ import annotations

import dataclasses
from dataclasses import dataclass, field
from typing import Dict, List, Optional, Tuple

import numpy as np

# stream indices of SeedSequence(seed).spawn(...)
_S_PARAMS, _S_LATENT, _S_TEXT, _S_NOISE, _S_DIR, _S_EXTRA = range(6)


@dataclass(frozen=True)
class DiTConfig:
    name: str
    n_blocks: int
    hidden: int
    n_heads: int
    mlp: int
    seq: int            # latent tokens per request (dense workloads)
    channels: int       # latent channels C
    text_tokens: int    # T
    text_dim: int       # D_t
    requests: int       # R; CFG rows B = 2R
    guidance: float
    n_steps: int        # sampler grid size N, t_i = 1 - i/N
    steer_block: int    # 0-based block index whose output is steered
    steer_alpha: float
    steer_steps: Tuple[int, ...]  # steps (0-based, inclusive set) with alpha != 0
    wmode: str          # "w8a8" | "f16" | "q4" | "w8a16"
    seed: int
    ln_eps: float = 1e-5
    steer_mode: str = "add"  # "add" (alpha, residual-norm units) | "project" (beta)
    steer_site: str = "residual"  # "residual" (block output) | "latent" (model input) | "text"
    sampler: str = "flow"   # "flow" (velocity, Euler on t) | "ddim" (epsilon, DDIM on alpha_bar)
    train_steps: int = 1000  # DDIM: training timesteps T of the noise schedule
    beta_1: float = 1e-4     # DDIM: betas linear from beta_1 to beta_T
    beta_T: float = 0.02

    @property
    def steer_dim(self) -> int:
        """Width of the steered tensor: H, C or D_t."""
        return {"residual": self.hidden, "latent": self.channels, "text": self.text_dim}[self.steer_site]

    @property
    def head_dim(self) -> int:
        return self.hidden // self.n_heads

    @property
    def cfg_rows(self) -> int:
        return 2 * self.requests

    @property
    def tokens(self) -> int:
        return self.cfg_rows * self.seq

    def replace(self, **kw) -> "DiTConfig":
        return dataclasses.replace(self, **kw)


TINY = DiTConfig("tiny", 2, 256, 4, 1024, 64, 64, 32, 256, 1, 3.0, 8, 1, 0.5, (0,), "w8a8", 0)
MID = DiTConfig("mid", 16, 1024, 16, 4096, 256, 64, 128, 768, 1, 3.0, 8, 12, 0.5, (2, 3, 4, 5), "w8a8", 1)
SERVE = DiTConfig("serve", 24, 1536, 24, 6144, 512, 64, 128, 768, 8, 3.0, 8, 12, 0.0, (), "w8a8", 2)
Q4 = DiTConfig("q4", 24, 2048, 32, 8192, 1024, 64, 256, 1024, 4, 3.0, 8, 12, 0.0, (), "q4", 3)
MIXED = DiTConfig("mixed", 16, 1024, 16, 4096, 576, 64, 128, 768, 32, 3.0, 16, 12, 0.5, (), "w8a8", 4)
# the DDIM backbone of the warm-start serving pages: 200 steps on a linear-beta schedule
TINY_DDIM = TINY.replace(name="tiny_ddim", n_steps=200, sampler="ddim", seed=5)
MID_DDIM = MID.replace(name="mid_ddim", n_steps=200, sampler="ddim", steer_steps=tuple(range(40, 80)), seed=6)

CONFIGS: Dict[str, DiTConfig] = {c.name: c for c in (TINY, MID, SERVE, Q4, MIXED, TINY_DDIM, MID_DDIM)}

LINEARS = ("qkv", "o", "q", "kv", "ox", "up", "down")


def linear_shapes(cfg: DiTConfig) -> Dict[str, Tuple[int, int]]:
    """(N, K) of every block linear, weight stored [N, K] (output-major)."""
    H, F, Dt = cfg.hidden, cfg.mlp, cfg.text_dim
    return {"qkv": (3 * H, H), "o": (H, H), "q": (H, H), "kv": (2 * H, Dt),
            "ox": (H, H), "up": (F, H), "down": (H, F)}


def _streams(seed: int, n: int = 6):
    return [np.random.default_rng(s) for s in np.random.SeedSequence(seed).spawn(n)]


def _normal_f16(rng, shape, std):
    # draw in fp32 chunks to bound host memory, round once to fp16
    out = np.empty(shape, dtype=np.float16)
    flat = out.reshape(-1)
    step = 1 << 24
    for i in range(0, flat.size, step):
        n = min(step, flat.size - i)
        flat[i:i + n] = (rng.standard_normal(n, dtype=np.float32) * np.float32(std)).astype(np.float16)
    return out


@dataclass
class BlockParams:
    ln1_g: np.ndarray
    ln1_b: np.ndarray
    ln2_g: np.ndarray
    ln2_b: np.ndarray
    ln3_g: np.ndarray
    ln3_b: np.ndarray
    w: Dict[str, np.ndarray]      # fp16 [N, K]
    b: Dict[str, np.ndarray]      # fp32 [N]


@dataclass
class DiTParams:
    w_in: np.ndarray    # fp16 [H, C]
    b_in: np.ndarray    # fp32 [H]
    lnf_g: np.ndarray
    lnf_b: np.ndarray
    w_out: np.ndarray   # fp16 [C, H]
    b_out: np.ndarray   # fp32 [C]
    blocks: List[BlockParams]


def make_params(cfg: DiTConfig) -> DiTParams:
    rng = _streams(cfg.seed)[_S_PARAMS]
    H, C = cfg.hidden, cfg.channels

    def ln():
        g = (1.0 + 0.02 * rng.standard_normal(H)).astype(np.float32)
        b = (0.02 * rng.standard_normal(H)).astype(np.float32)
        return g, b

    w_in = _normal_f16(rng, (H, C), 0.02)
    b_in = (0.02 * rng.standard_normal(H)).astype(np.float32)
    blocks = []
    shapes = linear_shapes(cfg)
    for _ in range(cfg.n_blocks):
        g1, b1 = ln()
        g2, b2 = ln()
        g3, b3 = ln()
        w, b = {}, {}
        for name in LINEARS:
            n, k = shapes[name]
            w[name] = _normal_f16(rng, (n, k), 0.02)
            b[name] = (0.02 * rng.standard_normal(n)).astype(np.float32)
        blocks.append(BlockParams(g1, b1, g2, b2, g3, b3, w, b))
    lnf_g, lnf_b = ln()
    w_out = _normal_f16(rng, (C, H), 0.02)
    b_out = (0.02 * rng.standard_normal(C)).astype(np.float32)
    return DiTParams(w_in, b_in, lnf_g, lnf_b, w_out, b_out, blocks)


@dataclass
class StepInputs:
    """Per-request state for one sampler run.

    x:      fp32 [R*S, C] packed latent state (dense: S per request)
    text:   fp16 [2R, T, D_t]; rows R..2R-1 are zeros (null prompt)
    x0:     fp32 [R*S, C] cached clean latent (warm start) or None
    eps:    fp32 [R*S, C] re-noising draw for warm start
    seqlens: int [R] latent length per request
    guidance: fp32 [R]
    direction: fp32 [H, C or D_t by steering site] unit steering direction
    t_grid: fp32 [N+1]  t_i = 1 - i/N
    alpha:  fp32 [N, R] steering strength per step and request
    start_step: int [R] first step run by each request (0 = cold start)
    """
    x: np.ndarray
    text: np.ndarray
    seqlens: np.ndarray
    guidance: np.ndarray
    direction: np.ndarray
    t_grid: np.ndarray
    alpha: np.ndarray
    start_step: np.ndarray
    x0: Optional[np.ndarray] = None
    eps: Optional[np.ndarray] = None
    timesteps: Optional[np.ndarray] = None  # DDIM: int [N] descending training timesteps


def t_grid(n_steps: int) -> np.ndarray:
    """Uniform flow-matching grid t_i = 1 - i/N, i = 0..N (fp32)."""
    return (1.0 - np.arange(n_steps + 1, dtype=np.float64) / n_steps).astype(np.float32)


def make_inputs(cfg: DiTConfig, seqlens: Optional[np.ndarray] = None) -> StepInputs:
    st = _streams(cfg.seed)
    R, C, T, Dt, H, N = cfg.requests, cfg.channels, cfg.text_tokens, cfg.text_dim, cfg.hidden, cfg.n_steps
    if seqlens is None:
        seqlens = np.full(R, cfg.seq, dtype=np.int64)
    seqlens = np.asarray(seqlens, dtype=np.int64)
    tot = int(seqlens.sum())
    x = st[_S_LATENT].standard_normal((tot, C), dtype=np.float32)
    text = np.zeros((2 * R, T, Dt), dtype=np.float16)
    text[:R] = st[_S_TEXT].standard_normal((R, T, Dt), dtype=np.float32).astype(np.float16)
    g = st[_S_DIR].standard_normal(cfg.steer_dim)
    direction = (g / np.sqrt(np.sum(g * g))).astype(np.float32)
    alpha = np.zeros((N, R), dtype=np.float32)
    for s in cfg.steer_steps:
        if 0 <= s < N:
            alpha[s, :] = cfg.steer_alpha
    tg, ts = t_grid(N), None
    if cfg.sampler == "ddim":
        ts = ddim_timesteps(N, cfg.train_steps)
        tg = np.concatenate([ts / cfg.train_steps, [0.0]]).astype(np.float32)
    return StepInputs(x=x, text=text, seqlens=seqlens,
                      guidance=np.full(R, cfg.guidance, dtype=np.float32),
                      direction=direction, t_grid=tg, alpha=alpha,
                      start_step=np.zeros(R, dtype=np.int64), timesteps=ts)


def ddim_timesteps(n_steps: int, train_steps: int) -> np.ndarray:
    """DDIM grid of N evenly spaced training timesteps, descending:
    (N - 1 - i) * (T / N) for i = 0..N-1 (T a multiple of N); the time
    embedding of grid point i takes t = timesteps[i] / T."""
    assert train_steps % n_steps == 0
    return ((n_steps - 1 - np.arange(n_steps)) * (train_steps // n_steps)).astype(np.int64)


SKIP_ARMS = tuple(range(0, 70, 5))  # warm-start skip percentages 0 %, 5 %, ..., 65 %


def make_ddim_warm_inputs(cfg: DiTConfig, arms_pct: np.ndarray,
                          seqlens: Optional[np.ndarray] = None) -> StepInputs:
    """DDIM requests warm-started at percentage-granular skip arms: request r
    skips k_r = arms_pct[r] * N / 100 steps (N a multiple of 20, so every arm
    is a whole step), is re-noised at grid point k_r from a seeded stand-in
    for a cached clean latent and runs steps k_r..N-1; arm 0 is a cold start."""
    arms_pct = np.asarray(arms_pct, np.int64)
    assert cfg.sampler == "ddim" and cfg.n_steps % 20 == 0
    assert np.all(np.isin(arms_pct, SKIP_ARMS))
    R = len(arms_pct)
    base = make_inputs(cfg.replace(requests=R), seqlens=seqlens)
    st = _streams(cfg.seed)
    tot = int(np.asarray(base.seqlens).sum())
    base.start_step = arms_pct * cfg.n_steps // 100
    base.x0 = st[_S_EXTRA].standard_normal((tot, cfg.channels), dtype=np.float32)
    base.eps = st[_S_NOISE].standard_normal((tot, cfg.channels), dtype=np.float32)
    return base


def make_mixed_inputs(cfg: DiTConfig, requests: Optional[int] = None,
                      seqlens: Optional[np.ndarray] = None,
                      warm: Optional[np.ndarray] = None) -> StepInputs:
    """Warm-start mixed batch: varlen requests, half cold and half warm.

    Cold requests start from N(0,1) noise at step 0.  Warm requests carry a
    seeded stand-in for a cached clean latent x0, a skip fraction p ~ U[0.3, 0.7]
    (start step k = floor(p*N + 1/2)) and their own re-noising draw eps.
    Guidance w_r ~ U[1, 5]; a steering window [a_r, b_r] inside the steps each
    request runs, strength cfg.steer_alpha.
    """
    st = _streams(cfg.seed)
    R = cfg.requests if requests is None else requests
    ex = st[_S_EXTRA]
    if seqlens is None:
        seqlens = ex.integers(128, 1025, size=R)
    seqlens = np.asarray(seqlens, dtype=np.int64)
    R = len(seqlens)
    if warm is None:
        warm = np.arange(R) >= R // 2
    warm = np.asarray(warm, dtype=bool)
    N = cfg.n_steps
    p = ex.uniform(0.3, 0.7, size=R)
    k = np.floor(p * N + 0.5).astype(np.int64)
    start = np.where(warm, k, 0)
    w = ex.uniform(1.0, 5.0, size=R).astype(np.float32)
    alpha = np.zeros((N, R), dtype=np.float32)
    for r in range(R):
        a = int(ex.integers(start[r], N))
        b = int(ex.integers(a, N))
        alpha[a:b + 1, r] = cfg.steer_alpha
    base = make_inputs(cfg.replace(requests=R), seqlens=seqlens)
    tot = int(seqlens.sum())
    x0 = ex.standard_normal((tot, cfg.channels), dtype=np.float32)
    eps = st[_S_NOISE].standard_normal((tot, cfg.channels), dtype=np.float32)
    base.guidance = w
    base.alpha = alpha
    base.start_step = start
    base.x0 = x0
    base.eps = eps
    return base


def cu_seqlens(seqlens: np.ndarray) -> np.ndarray:
    return np.concatenate([[0], np.cumsum(np.asarray(seqlens, dtype=np.int64))]).astype(np.int32)
