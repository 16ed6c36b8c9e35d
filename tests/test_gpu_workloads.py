"""Parity of the denoise step at the serving, 4-bit and mixed warm-start
workload shapes, and invariants at full serving size.

The oracle finishes a reduced-depth model of the serving widths (hidden 1536,
24 heads, MLP 6144, 8 requests x 512 latent tokens = 8192 CFG rows) and of
the 4-bit widths (hidden 2048, MLP 8192, 4 requests x 1024 tokens) in
seconds, so those are checked element by element: the model output of both
CFG rows, the latent's increment over the step and the latent itself, each
within 2e-2 (max |g - o| / max |o|), and at the serving widths the steering's
own effect on the model output (bar 0.1).  The full 24-block serving model and
the full 24-block 4-bit model are checked the same way on one request (1024
and 2048 CFG rows).  The mixed warm-start
batch runs the full 16-block mid-size model on a 4-request packed sub-batch
(lengths 128, 129, 577, 1024; two cold, two warm, one re-noised inside the
checked steps); the full 32-request batch must give each request, bit for
bit, what it gives alone.  At the full 24-block sizes of all 8 serving
requests and of the 4-bit model the graph replay must equal eager execution
bit for bit and the latent stays finite.
"""
import numpy as np
import pytest
import torch

import ald_inputs as I
from audio_latent_diffusion_amd import runtime
from oracle import ald_oracle as O
from tests import _stepcheck as S
from tests._gpu import host, needs_gpu
from tests.test_gpu_step import check_effect, check_steps

pytestmark = [pytest.mark.gpu, needs_gpu]

TOL = S.STEP_TOL
RESID = 20.0
# mean token norm of block 1's output at the serving widths (oracle, unsteered
# pass, one request: 62.4): the steering unit there
RESID_SERVE = 62.0


def _runner(model, inp, resid=RESID, **kw):
    return runtime.StepRunner(model, inp.x, inp.text, inp.seqlens, inp.t_grid, inp.guidance, inp.alpha,
                              inp.direction, resid, start_step=inp.start_step, x0=inp.x0, eps=inp.eps,
                              timesteps=inp.timesteps, **kw)


def _parity(cfg, steps, inp=None, resid=RESID):
    p = I.make_params(cfg)
    inp = I.make_inputs(cfg) if inp is None else inp
    check_steps(runtime.DiTModel(cfg, p), O.prepare_model(cfg, p), inp, steps,
                f"{cfg.name} {cfg.wmode} blocks={cfg.n_blocks} steps={list(steps)}", resid=resid)


@pytest.mark.parametrize("wmode", ["w8a8", "f16", "w8a16"])
def test_serve_widths_two_blocks(wmode):
    """Serving widths, each weight arm on the same inputs; steering (alpha 0.5
    at block 1 in units of its mean token norm) checked in full and on its
    effect."""
    cfg = I.SERVE.replace(n_blocks=2, wmode=wmode, steer_block=1, steer_alpha=0.5, steer_steps=(0,))
    p = I.make_params(cfg)
    check_effect(runtime.DiTModel(cfg, p), O.prepare_model(cfg, p), cfg, I.make_inputs(cfg), 0,
                 f"serve widths {wmode}", resid=RESID_SERVE)


@pytest.mark.parametrize("site,sampler,step", [("text", "flow", 0), ("latent", "ddim", 60), ("residual", "ddim", 199)])
def test_serve_widths_sites_and_ddim(site, sampler, step):
    """Serving widths (2 blocks, W8A8): steering at the text and latent sites,
    and the DDIM sampler in the middle and at the last step of its 200-step
    grid (the last returns the clean estimate)."""
    n = 200 if sampler == "ddim" else 8
    cfg = I.SERVE.replace(n_blocks=2, steer_block=1, steer_alpha=0.5, steer_steps=(step,), steer_site=site,
                          sampler=sampler, n_steps=n)
    _parity(cfg, [step])


def test_q4_widths_one_block():
    """4-bit weights (group 32, fp16 scales) at hidden 2048, 1024 latent tokens."""
    cfg = I.Q4.replace(n_blocks=1, steer_block=0, steer_alpha=0.5, steer_steps=(0,))
    _parity(cfg, [0])


def test_mixed_warm_start_subbatch():
    """Packed varlen requests of the mid-size model, two of them warm-started:
    request 2 is re-noised to t_5 inside the checked steps, request 3 stays
    inactive until step 7."""
    cfg = I.MIXED
    inp = I.make_mixed_inputs(cfg, seqlens=np.array([128, 129, 577, 1024]),
                              warm=np.array([False, False, True, True]))
    inp.start_step = np.array([0, 0, 5, 7])
    _parity(cfg, [5, 6], inp)


@pytest.mark.timeout(900)
def test_serve_full_depth_one_request():
    """The full 24-block serving model (hidden 1536, 24 heads, MLP 6144, W8A8)
    on one request, a CFG pair of 512 latent tokens (1024 rows), steering at
    block 12 active: the step's model output, increment and latent against
    the oracle."""
    cfg = I.SERVE.replace(requests=1, steer_alpha=0.5, steer_steps=(0,))
    _parity(cfg, [0], resid=RESID_SERVE)


@pytest.mark.timeout(900)
def test_q4_full_depth_one_request():
    """The full 24-block 4-bit-weight model (hidden 2048, 32 heads, MLP 8192,
    group-32 weights with fp16 scales) on one request, a CFG pair of 1024
    latent tokens (2048 rows), steering at block 12 active: the step's model
    output, increment and latent against the oracle."""
    cfg = I.Q4.replace(requests=1, steer_alpha=0.5, steer_steps=(0,))
    _parity(cfg, [0])


@pytest.fixture(scope="module")
def serve_params():
    return I.make_params(I.SERVE)


@pytest.mark.parametrize("wmode", ["w8a8", "f16", "w8a16"])
def test_serve_full_size_graph_equals_eager(serve_params, wmode):
    """The full 24-block serving model (8192 CFG rows) in each weight
    precision: two steps replayed as one graph equal the same two steps run
    eagerly, bit for bit."""
    cfg = I.SERVE.replace(wmode=wmode)
    inp = I.make_inputs(cfg)
    model = runtime.DiTModel(cfg, serve_params)
    eager = _runner(model, inp)
    eager.step(0)
    eager.step(1)
    graph = _runner(model, inp)
    graph.capture([0, 1])
    graph.replay()
    a, b = host(eager.x), host(graph.x)
    assert np.all(np.isfinite(a))
    assert a.tobytes() == b.tobytes()
    # the step moved the latent by the guided velocity times the step size
    assert not np.array_equal(a, inp.x)


@pytest.mark.parametrize("wmode", ["w8a8", "f16"])
def test_serve_full_size_requests_independent(serve_params, wmode):
    """The full serving batch (8 requests, 8192 CFG rows: large GEMM tiles)
    against single requests (1024 rows: small tiles), two steps: each request
    comes out bit for bit the same.  int32 accumulators are exact, fp32 ones
    take the same K order in every tile shape, and every other kernel works
    per row or per sequence."""
    cfg = I.SERVE.replace(wmode=wmode)
    model = runtime.DiTModel(cfg, serve_params)
    inp = I.make_inputs(cfg)
    inp.alpha[:2] = 0.5
    packed = _runner(model, inp)
    packed.step(0)
    packed.step(1)
    got = host(packed.x)
    R, L = cfg.requests, cfg.seq
    for r in (0, R - 1):
        one = I.make_inputs(cfg.replace(requests=1))
        one.x = inp.x[r * L:(r + 1) * L]
        one.text = inp.text[[r, R + r]]
        one.guidance = inp.guidance[r:r + 1]
        one.alpha = inp.alpha[:, r:r + 1]
        one.direction = inp.direction
        single = _runner(model, one)
        single.step(0)
        single.step(1)
        assert host(single.x).tobytes() == got[r * L:(r + 1) * L].tobytes(), f"request {r}"


def test_q4_full_size_graph_equals_eager():
    """The full 24-block 4-bit-weight model (hidden 2048, 4 requests x 1024
    latent tokens = 8192 CFG rows): two steps replayed as one graph equal the
    same two steps run eagerly, bit for bit, and the latent stays finite."""
    cfg = I.Q4
    p = I.make_params(cfg)
    inp = I.make_inputs(cfg)
    model = runtime.DiTModel(cfg, p)
    del p
    eager = _runner(model, inp)
    eager.step(0)
    eager.step(1)
    graph = _runner(model, inp)
    graph.capture([0, 1])
    graph.replay()
    a, b = host(eager.x), host(graph.x)
    assert np.all(np.isfinite(a))
    assert a.tobytes() == b.tobytes()
    assert not np.array_equal(a, inp.x)


def test_mixed_full_batch_requests_independent():
    """The full mixed warm-start batch (32 packed requests of 128..1024 latent
    tokens on the mid-size model, about 37k CFG rows per launch, the launch
    shapes the bench times): two steps, the warm half re-noised at the second
    one, steering in both; cold and warm requests give, bit for bit, what each
    gives run alone (its own small launches).  Exact int32 accumulators and
    per-row, per-sequence kernels make the result independent of the batch."""
    cfg = I.MIXED
    model = runtime.DiTModel(cfg, I.make_params(cfg))
    inp = I.make_mixed_inputs(cfg)
    R = len(inp.seqlens)
    warm = np.arange(R) >= R // 2
    inp.start_step = np.where(warm, 1, 0)
    inp.alpha[:2] = 0.5
    packed = _runner(model, inp)
    packed.step(0)
    packed.step(1)
    got = host(packed.x)
    assert np.all(np.isfinite(got))
    cu = np.concatenate([[0], np.cumsum(inp.seqlens)])
    for r in (0, 13, R // 2, R - 1):
        sl = slice(cu[r], cu[r + 1])
        one = I.make_mixed_inputs(cfg.replace(requests=1), seqlens=inp.seqlens[r:r + 1], warm=warm[r:r + 1])
        one.x = inp.x[sl]
        one.x0 = inp.x0[sl]
        one.eps = inp.eps[sl]
        one.text = inp.text[[r, R + r]]
        one.guidance = inp.guidance[r:r + 1]
        one.alpha = inp.alpha[:, r:r + 1]
        one.start_step = inp.start_step[r:r + 1]
        one.direction = inp.direction
        single = _runner(model, one)
        single.step(0)
        single.step(1)
        assert host(single.x).tobytes() == got[sl].tobytes(), f"request {r} (warm {bool(warm[r])})"
