"""End-to-end parity of the denoise step (dit_step / hipGraph) against the oracle.

Every one-step check compares, against the oracle and with the 2e-2 bar
(max |g - o| / max |o|), the model output v of both CFG rows, the latent's
increment over the step and the latent itself; a steered step is also
checked on the steering's own effect (steered minus unsteered model output
against the oracle's, bar 0.1).  Alpha = 0 is bit-identical to the unsteered
pass, graph replay bit-identical to eager, packed varlen requests
bit-identical to one request at a time.
"""
import numpy as np
import pytest
import torch

import ald_inputs as I
from audio_latent_diffusion_amd import runtime
from oracle import ald_oracle as O
from tests import _stepcheck as S
from tests._gpu import host, needs_gpu

pytestmark = [pytest.mark.gpu, needs_gpu]

TOL = S.STEP_TOL
RESID = 5.0
# mean token norm of block 12's output in the mid model's unsteered pass
# (oracle, step 2: 74.8): the steering unit of the workload
RESID_MID = 75.0


def _runner(model, inp, resid=RESID, **kw):
    return runtime.StepRunner(model, inp.x, inp.text, inp.seqlens, inp.t_grid, inp.guidance, inp.alpha,
                              inp.direction, resid, start_step=inp.start_step, x0=inp.x0, eps=inp.eps,
                              timesteps=inp.timesteps, **kw)


def _gpu_steps(model, inp, steps, resid=RESID):
    """GPU latent before the last of `steps`, after it, and its model output."""
    run = _runner(model, inp, resid=resid, keep_velocity=True)
    for i in steps[:-1]:
        run.step(i)
    x_prev = host(run.x).copy()
    run.step(steps[-1])
    return x_prev, host(run.x), host(run.v_out)


def check_steps(model, om, inp, steps, label, resid=RESID):
    """Run `steps` on both sides; assert model output, increment and latent
    of the last step (W8A8: bars from the measured spread of two valid
    oracle evaluations); return (gpu velocity, oracle velocity, the spread
    evaluation's velocity or None)."""
    steps = list(steps)
    xg0, xg, vg = _gpu_steps(model, inp, steps, resid)
    xo0, xo, tr = S.oracle_steps(om, inp, steps, resid)
    bars, trb = S.step_bars(model.cfg.wmode, om, inp, steps, resid, (xo0, xo, tr))
    S.assert_step(S.step_errors(xg0, xg, vg, xo0, xo, tr.v), label, bars)
    return vg, tr.v, None if trb is None else trb.v


def check_effect(model, om, cfg, inp, step, label, resid=RESID):
    """One steered step on both sides (full step checks) and the steering's
    effect on the model output against the oracle's (W8A8: bar twice the
    effect's spread between two valid oracle evaluations, at least
    EFFECT_TOL)."""
    vg_on, vo_on, vb_on = check_steps(model, om, inp, [step], label, resid)
    _, _, vg_off = _gpu_steps(model.with_steer_block(-1), inp, [step], resid)
    om_off = O.PreparedModel(cfg.replace(steer_block=-1), om.params, om.lin)
    _, _, tr_off = S.oracle_steps(om_off, inp, [step], resid)
    err, size = S.effect_error(vg_on, vg_off, vo_on, tr_off.v)
    bar = S.EFFECT_TOL
    if vb_on is not None:
        with S.fp32_layer_norm():
            _, _, trb_off = S.oracle_steps(om_off, inp, [step], resid)
        spread, _ = S.effect_error(vb_on, trb_off.v, vo_on, tr_off.v)
        bar = max(S.EFFECT_TOL, S.SPREAD_FACTOR * spread)
        print(f"{label}: effect spread of two valid oracle evaluations {spread:.2e}")
    print(f"{label}: steering effect {size:.2e} of the output, effect err {err:.2e} (bar {bar:.2e})")
    assert size > 5 * TOL, "the steering effect is too small to check"
    assert err < bar


@pytest.fixture(scope="module")
def tiny():
    cfg = I.TINY
    p = I.make_params(cfg)
    return cfg, p, runtime.DiTModel(cfg, p), O.prepare_model(cfg, p)


def _oracle_steps(om, inp, steps, resid=RESID):
    kv = O.text_kv(om, inp.text)
    x, tr = O.run_sampler(om, inp, kv, resid_norm=resid, steps=steps)
    return x, tr


# A model with no blocks: the velocity is the output projection of the final
# LayerNorm of the input projection, so these check the input projection and
# its time embedding over every row directly.  Serving widths (8192 rows:
# four-wave 128 x 128 tiles), the mid-size step (512 rows: single-wave 64 x 64
# tiles), ragged packed requests at hidden 1088 on both tile kinds (7216
# rows: the last row tile and the last column tile cut short; 284 rows) and
# a latent width of 72.
# Bar: the fp16 rounding of h, the fp32 sums and the time embedding's ~1e-4
# rad argument error move v by a few fp16 ulps of its largest entry.
INPROJ_TOL = 2e-3


@pytest.mark.parametrize("name", ["serve", "mid", "ragged_large", "ragged_small", "width_72"])
def test_input_projection_zero_blocks(name):
    if name in ("serve", "mid"):
        cfg = (I.SERVE if name == "serve" else I.MID).replace(n_blocks=0, steer_block=-1)
        inp = I.make_inputs(cfg)
    elif name == "width_72":  # a latent width other than 64: the generic K loop, its last step half padded
        cfg = I.TINY.replace(n_blocks=0, steer_block=-1, channels=72)
        inp = I.make_inputs(cfg)
    else:
        lens = [1500, 2011, 97] if name == "ragged_large" else [37, 100, 5]
        cfg = I.TINY.replace(n_blocks=0, steer_block=-1, requests=3, hidden=1088, n_heads=17)
        inp = I.make_inputs(cfg, seqlens=np.array(lens))
    p = I.make_params(cfg)
    om = O.prepare_model(cfg, p)
    step = 3  # t = 5/8, not 1: the embedding arguments differ from the first step's
    _, _, vg = _gpu_steps(runtime.DiTModel(cfg, p), inp, [step])
    _, _, tr = S.oracle_steps(om, inp, [step], RESID)
    err = S.rel(vg, tr.v)
    print(f"{name}: input projection (zero blocks) velocity err {err:.2e} (bar {INPROJ_TOL:.0e})")
    assert err < INPROJ_TOL


@pytest.mark.parametrize("wmode", ["w8a8", "f16", "q4", "w8a16"])
def test_tiny_step_parity(wmode):
    """One steered step of the tiny DiT in each weight precision, and the
    steering's effect."""
    cfg = I.TINY.replace(wmode=wmode)
    p = I.make_params(cfg)
    inp = I.make_inputs(cfg)
    check_effect(runtime.DiTModel(cfg, p), O.prepare_model(cfg, p), cfg, inp, 0, f"tiny {wmode}")


def test_tiny_step_projection_steering():
    """Projection steering at block 1 (beta 4: the projection scales only the
    small component along d, so a larger strength makes its effect
    measurable): the step and the effect against the oracle, and beta = 0
    bit-identical to the unsteered pass."""
    cfg = I.TINY.replace(steer_mode="project")
    p = I.make_params(cfg)
    inp = I.make_inputs(cfg)
    inp.alpha[0] = 4.0
    model = runtime.DiTModel(cfg, p)
    check_effect(model, O.prepare_model(cfg, p), cfg, inp, 0, "tiny projection steering")
    inp.alpha[:] = 0
    a = _runner(model, inp)
    a.step(0)
    b = _runner(model.with_steer_block(-1), inp)
    b.step(0)
    assert host(a.x).tobytes() == host(b.x).tobytes()


@pytest.mark.parametrize("site,mode,wmode", [("latent", "add", "w8a8"), ("latent", "project", "w8a8"),
                                             ("text", "add", "w8a8"), ("text", "project", "w8a8"),
                                             ("text", "add", "f16"), ("latent", "add", "w8a16")])
def test_tiny_step_other_sites(site, mode, wmode):
    """Steering at the latent (model input) and text-conditioning sites: one
    steered step and the steering's effect against the oracle; strength 0 is
    bit-identical to the unsteered pass."""
    cfg = I.TINY.replace(steer_site=site, steer_mode=mode, wmode=wmode)
    p = I.make_params(cfg)
    inp = I.make_inputs(cfg)
    # a projection only scales the text's small component along d: a larger
    # strength makes its effect measurable
    inp.alpha[0] = 64.0 if (site, mode) == ("text", "project") else 2.0
    # the site's own norm unit: mean token norm of the latent or of the cond text
    resid = O.mean_row_norm(inp.x.astype(np.float16)) if site == "latent" else \
        O.mean_row_norm(inp.text[:cfg.requests].reshape(-1, cfg.text_dim))
    model = runtime.DiTModel(cfg, p)
    check_effect(model, O.prepare_model(cfg, p), cfg, inp, 0, f"tiny {site} {mode} {wmode}", resid=resid)
    inp.alpha[:] = 0
    a = _runner(model, inp, resid=resid)
    a.step(0)
    b = _runner(model.with_steer_block(-1), inp)
    b.step(0)
    assert host(a.x).tobytes() == host(b.x).tobytes()


def test_text_site_graph_equals_eager(tiny):
    """The text site recomputes the text K/V inside every step: an 8-step
    graph replay equals eager execution bit for bit, before and after new
    strengths are written into device memory."""
    cfg, p, model, om = tiny
    cfg8 = cfg.replace(steer_site="text", steer_steps=(2, 3, 4, 5))
    inp = I.make_inputs(cfg8)
    mt = model.with_config(steer_site="text")
    eager = _runner(mt, inp)
    for i in range(8):
        eager.step(i)
    g = _runner(mt, inp)
    g.capture()
    g.replay()
    assert host(g.x).tobytes() == host(eager.x).tobytes()
    g.x.copy_(torch.from_numpy(inp.x).cuda())
    new_alpha = np.zeros_like(inp.alpha)
    new_alpha[5:8] = -0.3
    g.alpha.copy_(torch.from_numpy(new_alpha).cuda())
    g.replay()
    inp.alpha = new_alpha
    e2 = _runner(mt, inp)
    for i in range(8):
        e2.step(i)
    assert host(g.x).tobytes() == host(e2.x).tobytes()


@pytest.mark.parametrize("steps", [[0, 1], [198, 199]])
def test_tiny_ddim_steps(steps):
    """DDIM sampler (epsilon prediction on the 200-step linear-beta grid):
    the first steps (alpha_bar near 4e-5) and the last two (the last returns
    the clean estimate) against the oracle."""
    cfg = I.TINY_DDIM
    p = I.make_params(cfg)
    inp = I.make_inputs(cfg)
    check_steps(runtime.DiTModel(cfg, p), O.prepare_model(cfg, p), inp, steps, f"tiny ddim steps {steps}")


@pytest.mark.parametrize("site,sampler", [("residual", "flow"), ("text", "ddim"), ("latent", "ddim")])
def test_varlen_warm_start_parity(tiny, site, sampler):
    """Packed requests of different lengths, two of them warm-started at
    later steps, steering at the given site, under either sampler: four
    steps, the last one checked in full."""
    cfg, p, model, _ = tiny
    cfg3 = cfg.replace(requests=3, n_steps=4, steer_site=site, sampler=sampler)
    inp = I.make_mixed_inputs(cfg3, seqlens=np.array([16, 33, 64]), warm=np.array([False, True, True]))
    inp.start_step = np.array([0, 1, 2])
    check_steps(model.with_config(steer_site=site, sampler=sampler, n_steps=4), O.prepare_model(cfg3, p), inp,
                range(4), f"varlen warm start, {site} site, {sampler}")


@pytest.mark.parametrize("site,sampler", [("text", "flow"), ("residual", "ddim")])
def test_mid_step_sites_and_ddim(site, sampler):
    """The full mid-size model (16 blocks, hidden 1024): one steered step with
    text-site steering (K/V recomputed in the step), and one DDIM step."""
    n = 200 if sampler == "ddim" else 8
    step = 60 if sampler == "ddim" else 2
    cfg = I.MID.replace(steer_site=site, sampler=sampler, n_steps=n, steer_steps=(step,))
    p = I.make_params(cfg)
    inp = I.make_inputs(cfg)
    check_steps(runtime.DiTModel(cfg, p), O.prepare_model(cfg, p), inp, [step], f"mid step {step}, {site}, {sampler}")


def test_mid_step_parity():
    """The mid-size model (16 blocks, hidden 1024): one step inside the
    steering span (alpha 0.5 at block 12 in units of that block's mean token
    norm), in full, and the steering's effect on the model output."""
    cfg = I.MID
    p = I.make_params(cfg)
    inp = I.make_inputs(cfg)
    check_effect(runtime.DiTModel(cfg, p), O.prepare_model(cfg, p), cfg, inp, 2, "mid step 2", resid=RESID_MID)


def test_ddim_skip_arms_full_run_graph():
    """Two requests, a cold start and a 10 % skip arm (re-noised at step 20),
    through all 200 DDIM steps: one captured graph equals eager execution bit
    for bit, and the final latent matches the oracle's whole run."""
    cfg = I.TINY_DDIM.replace(n_blocks=1, steer_block=0)
    p = I.make_params(cfg)
    inp = I.make_ddim_warm_inputs(cfg, np.array([0, 10]), seqlens=np.array([40, 24]))
    model = runtime.DiTModel(cfg, p)
    eager = _runner(model, inp)
    for i in range(cfg.n_steps):
        eager.step(i)
    g = _runner(model, inp)
    g.capture()
    g.replay()
    assert host(g.x).tobytes() == host(eager.x).tobytes()
    ref, _ = O.run_sampler(O.prepare_model(cfg, p), inp, resid_norm=RESID)
    err = O.normwise_rel_err(host(g.x), ref)
    print(f"tiny ddim 200 steps, arms 0 % / 10 %: latent err {err:.2e}")
    assert err < TOL


def test_alpha_zero_bit_identical(tiny):
    cfg, p, model, _ = tiny
    inp = I.make_inputs(cfg)
    inp.alpha[:] = 0
    a = _runner(model, inp)
    b = _runner(model.with_steer_block(-1), inp)
    a.step(0)
    b.step(0)
    assert host(a.x).tobytes() == host(b.x).tobytes()
    inp.alpha[:] = 0.5
    c = _runner(model, inp)
    c.step(0)
    assert not np.array_equal(host(c.x), host(a.x))


def test_graph_replay_equals_eager_and_no_recapture(tiny):
    cfg, p, model, om = tiny
    cfg8 = cfg.replace(steer_steps=(2, 3, 4, 5))
    inp = I.make_inputs(cfg8)
    eager = _runner(model, inp)
    for i in range(8):
        eager.step(i)
    g = _runner(model, inp)
    g.capture()
    g.replay()
    assert host(g.x).tobytes() == host(eager.x).tobytes()
    # new steering strengths written into device memory, same graph
    x_init = torch.from_numpy(inp.x).cuda()
    g.x.copy_(x_init)
    new_alpha = np.zeros_like(inp.alpha)
    new_alpha[4:8] = 0.25
    g.alpha.copy_(torch.from_numpy(new_alpha).cuda())
    g.replay()
    inp2 = I.make_inputs(cfg8)
    inp2.alpha = new_alpha
    e2 = _runner(model, inp2)
    for i in range(8):
        e2.step(i)
    assert host(g.x).tobytes() == host(e2.x).tobytes()
    # and the 8-step result matches the oracle sampler
    ref, _ = _oracle_steps(om, inp2, None)
    assert O.normwise_rel_err(host(g.x), ref) < TOL


SITE_SAMPLER = [("residual", "flow"), ("latent", "flow"), ("text", "flow"), ("text", "ddim"), ("latent", "ddim")]


@pytest.mark.parametrize("site,sampler", SITE_SAMPLER)
def test_packed_equals_single_requests(tiny, site, sampler):
    """Three packed requests give, bit for bit, what each gives alone (steered
    at the given site, under either sampler)."""
    cfg, p, model, _ = tiny
    model = model.with_config(steer_site=site, sampler=sampler, n_steps=2)
    cfg = model.cfg
    lens = np.array([40, 64, 17])
    cfg3 = cfg.replace(requests=3)
    inp = I.make_mixed_inputs(cfg3, seqlens=lens, warm=np.zeros(3, bool))
    inp.alpha[:] = 0.5
    packed = _runner(model, inp)
    packed.step(0)
    got = host(packed.x)
    cu = np.concatenate([[0], np.cumsum(lens)])
    T = cfg.text_tokens
    for r in range(3):
        sl = slice(cu[r], cu[r + 1])
        one = I.make_mixed_inputs(cfg.replace(requests=1, n_steps=2), seqlens=lens[r:r + 1], warm=np.zeros(1, bool))
        one.x = inp.x[sl]
        one.text = inp.text[[r, 3 + r]]
        one.guidance = inp.guidance[r:r + 1]
        one.alpha = inp.alpha[:, r:r + 1]
        single = _runner(model, one)
        single.step(0)
        assert host(single.x).tobytes() == got[sl].tobytes(), f"request {r}"


def test_mid_graph_replays_equal_eager():
    """The mid-size model's 8-step loop as one graph (the bench's unit),
    replayed three times with eager work in between: every replay equals the
    eager loop bit for bit."""
    cfg = I.MID
    p = I.make_params(cfg)
    inp = I.make_inputs(cfg)
    model = runtime.DiTModel(cfg, p)
    eager = _runner(model, inp)
    for i in range(cfg.n_steps):
        eager.step(i)
    want = host(eager.x).tobytes()
    g = _runner(model, inp)
    x_init = g.x.clone()
    g.capture()
    for _ in range(3):
        g.x.copy_(x_init)
        g.replay()
        assert host(g.x).tobytes() == want
        torch.randn(1 << 20, device="cuda").sum().item()  # unrelated eager work between replays


@pytest.mark.parametrize("wmode", ["w8a8", "f16", "q4", "w8a16"])
def test_text_site_stacked_kv_bit_identical(tiny, wmode):
    """Text-site steering re-projects the steered text's K/V in the step: with
    the blocks' K/V linears stacked (one launch for every block) the step is
    bit-identical to one launch per block, in every weight precision."""
    cfg, p, _, _ = tiny
    cfg = cfg.replace(wmode=wmode, steer_site="text")
    model = runtime.DiTModel(cfg, p)
    inp = I.make_inputs(cfg)
    unit = float(np.mean(np.linalg.norm(inp.text[:cfg.requests].reshape(-1, cfg.text_dim).astype(np.float64),
                                        axis=1)))
    outs = []
    for m in (model, model.with_stacked_kv(False)):
        run = _runner(m, inp, resid=unit)
        run.step(0)
        outs.append(host(run.x).tobytes())
    assert outs[0] == outs[1]
