"""Pins of the oracle's LayerNorm, GELU, attention, time embedding, steering,
CFG merge and sampler (CPU only)."""
import math

import numpy as np
import pytest
import torch

import ald_inputs as I
from oracle import ald_oracle as O


# ---------------------------------------------------------------- LayerNorm

def test_layer_norm_vs_torch_cpu_and_moments():
    rng = np.random.default_rng(0)
    x = (rng.standard_normal((16, 256)) * 3 + 1).astype(np.float16)
    g = (1 + 0.02 * rng.standard_normal(256)).astype(np.float32)
    b = (0.02 * rng.standard_normal(256)).astype(np.float32)
    y = O.layer_norm(x, g, b).astype(np.float64)
    ref = torch.nn.functional.layer_norm(torch.from_numpy(x.astype(np.float64)), (256,),
                                         torch.from_numpy(g.astype(np.float64)),
                                         torch.from_numpy(b.astype(np.float64)), eps=1e-5).numpy()
    assert np.max(np.abs(y - ref)) <= 2.0 ** -9 * np.max(np.abs(ref))
    y1 = O.layer_norm(x, np.ones(256, np.float32), np.zeros(256, np.float32)).astype(np.float64)
    assert np.allclose(y1.mean(axis=1), 0, atol=2e-3)
    assert np.allclose(y1.var(axis=1), 1, atol=5e-3)


def test_layer_norm_constant_row():
    x = np.full((2, 64), 3.0, np.float16)
    y = O.layer_norm(x, np.ones(64, np.float32), np.full(64, 0.25, np.float32))
    assert np.all(y == np.float16(0.25))   # zero variance: (x - mu) = 0 exactly


# ---------------------------------------------------------------- GELU

def test_gelu_values():
    assert O.gelu(np.array([0.0]))[0] == 0.0
    assert O.gelu(np.array([1.0]))[0] == pytest.approx(0.8413447460685429, abs=1e-15)  # Phi(1)
    x = np.linspace(-6, 6, 101)
    # erf is odd, so gelu(x) - gelu(-x) = x
    assert np.allclose(O.gelu(x) - O.gelu(-x), x, atol=1e-14)
    ref = np.array([0.5 * v * (1 + math.erf(v / math.sqrt(2))) for v in x])
    assert np.allclose(O.gelu(x), ref, atol=1e-15)


# ---------------------------------------------------------------- attention

def _naive_attn(q, k, v, scale):
    Sq, nh, d = q.shape
    Sk = k.shape[0]
    out = np.zeros((Sq, nh, d))
    for h in range(nh):
        for i in range(Sq):
            s = [sum(float(q[i, h, c]) * float(k[j, h, c]) for c in range(d)) * scale for j in range(Sk)]
            m = max(s)
            e = [math.exp(z - m) for z in s]
            z = math.fsum(e)
            for c in range(d):
                out[i, h, c] = math.fsum(e[j] * float(v[j, h, c]) for j in range(Sk)) / z
    return out


def test_attention_naive_loops():
    rng = np.random.default_rng(1)
    q = rng.standard_normal((5, 2, 8)).astype(np.float16)
    k = rng.standard_normal((7, 2, 8)).astype(np.float16)
    v = rng.standard_normal((7, 2, 8)).astype(np.float16)
    got = O.attention(q, k, v, 1 / math.sqrt(8)).astype(np.float64)
    ref = _naive_attn(q, k, v, 1 / math.sqrt(8))
    assert np.max(np.abs(got - ref)) <= 2.0 ** -11 * max(1.0, np.max(np.abs(ref)))


def test_attention_special_cases():
    rng = np.random.default_rng(2)
    q = rng.standard_normal((9, 3, 64)).astype(np.float16)
    v = rng.standard_normal((1, 3, 64)).astype(np.float16)
    k = rng.standard_normal((1, 3, 64)).astype(np.float16)
    # a single key: the softmax weight is exactly 1, output = v
    assert np.array_equal(O.attention(q, k, v, 0.125), np.broadcast_to(v, (9, 3, 64)))
    # identical keys: uniform weights, output = mean of the values
    k = np.broadcast_to(rng.standard_normal((1, 3, 64)).astype(np.float16), (6, 3, 64))
    v = rng.standard_normal((6, 3, 64)).astype(np.float16)
    got = O.attention(q, k, v, 0.125).astype(np.float64)
    ref = np.broadcast_to(v.astype(np.float64).mean(axis=0), got.shape)
    assert np.max(np.abs(got - ref)) <= 2.0 ** -10
    # permuting keys and values together leaves the output unchanged
    k2 = rng.standard_normal((6, 3, 64)).astype(np.float16)
    p = rng.permutation(6)
    a = O.attention(q, k2, v, 0.125).astype(np.float64)
    b = O.attention(q, k2[p], v[p], 0.125).astype(np.float64)
    assert np.max(np.abs(a - b)) <= 2.0 ** -10


def test_attention_varlen_equals_dense_per_sequence():
    rng = np.random.default_rng(3)
    lens = [3, 1, 10]
    tot = sum(lens)
    nh, d = 2, 16
    q = rng.standard_normal((tot, nh * d)).astype(np.float16)
    k = rng.standard_normal((tot, nh * d)).astype(np.float16)
    v = rng.standard_normal((tot, nh * d)).astype(np.float16)
    cu = np.concatenate([[0], np.cumsum(lens)])
    out = O.attention_varlen(q, k, v, cu, cu, nh, 0.25)
    for b in range(3):
        s0, s1 = cu[b], cu[b + 1]
        ref = _naive_attn(q[s0:s1].reshape(-1, nh, d), k[s0:s1].reshape(-1, nh, d),
                          v[s0:s1].reshape(-1, nh, d), 0.25).reshape(s1 - s0, nh * d)
        assert np.max(np.abs(out[s0:s1].astype(np.float64) - ref)) <= 2.0 ** -10


# ---------------------------------------------------------------- time embedding

def test_timestep_embedding_values():
    e = O.timestep_embedding(np.array([0.0, 0.5]), 8)
    assert np.array_equal(e[0], [0, 0, 0, 0, 1, 1, 1, 1])
    # omega_0 = 1: first entry is sin(1000 t), entry H/2 is cos(1000 t)
    assert e[1, 0] == pytest.approx(math.sin(500.0), abs=1e-12)
    assert e[1, 4] == pytest.approx(math.cos(500.0), abs=1e-12)
    # omega_j = 1e4^(-j/(H/2)): j = 2 of H/2 = 4 is 1e-2
    assert e[1, 2] == pytest.approx(math.sin(500.0 * 1e-2), abs=1e-12)
    assert np.allclose(e[:, :4] ** 2 + e[:, 4:] ** 2, 1.0)


# ---------------------------------------------------------------- steering

def test_steer_alpha_zero_is_bit_identical():
    rng = np.random.default_rng(4)
    h = rng.standard_normal((6, 32)).astype(np.float16)
    h[0, 0] = np.float16(-0.0)
    h[1, 3] = np.float16(np.nan)
    d = rng.standard_normal(32)
    d = (d / np.linalg.norm(d)).astype(np.float32)
    out = O.steer_add(h, np.zeros(6, np.float32), 7.5, d)
    assert out.tobytes() == h.tobytes()     # -0.0 and NaN bits kept
    alpha = np.array([0, 0.5, 0, 0.25, 0, 1.0], np.float32)
    out = O.steer_add(h, alpha, 7.5, d)
    for i in (0, 2, 4):
        assert out[i].tobytes() == h[i].tobytes()


def test_steer_closed_form_and_linearity():
    rng = np.random.default_rng(5)
    h = rng.standard_normal((4, 64)).astype(np.float16)
    d = rng.standard_normal(64)
    d = (d / np.linalg.norm(d)).astype(np.float32)
    hn = 3.0
    delta = {}
    for a in (0.25, 0.5, 1.0):
        out = O.steer_add(h, np.full(4, a, np.float32), hn, d).astype(np.float64)
        delta[a] = out - h.astype(np.float64)
        # rank-one update along d with magnitude alpha * ||h_bar||
        assert np.allclose(delta[a], a * hn * d.astype(np.float64)[None, :], atol=2.0 ** -8)
        assert np.allclose(np.linalg.norm(delta[a], axis=1), a * hn, rtol=2e-3)
    assert np.allclose(delta[1.0], 2 * delta[0.5], atol=2.0 ** -8)
    assert np.allclose(delta[0.5], 2 * delta[0.25], atol=2.0 ** -8)


def test_steer_project_beta_zero_and_orthogonal_rows_untouched():
    rng = np.random.default_rng(6)
    h = rng.standard_normal((5, 32)).astype(np.float16)
    h[0, 1] = np.float16(-0.0)
    d = np.zeros(32, np.float32)
    d[3] = 1.0                                   # d_hat = e_3
    out = O.steer_project(h, np.zeros(5, np.float32), d)
    assert out.tobytes() == h.tobytes()          # beta = 0: bit-identical
    h[2, 3] = 0                                  # row 2 orthogonal to d_hat
    out = O.steer_project(h, np.full(5, 0.75, np.float32), d)
    assert out[2].tobytes() == h[2].tobytes()    # h . d_hat = 0: nothing moves
    # along e_3 only coordinate 3 changes, scaled by 1 + beta (one rounding)
    rest = np.delete(np.arange(32), 3)
    assert np.array_equal(out[:, rest], h[:, rest])
    assert np.array_equal(out[:, 3], (h[:, 3].astype(np.float64) * 1.75).astype(np.float16))


def test_steer_project_scales_the_component_along_the_direction():
    rng = np.random.default_rng(7)
    h = rng.standard_normal((4, 64)).astype(np.float16)
    d = rng.standard_normal(64)
    d = (d / np.linalg.norm(d)).astype(np.float32)
    d64 = d.astype(np.float64)
    h64 = h.astype(np.float64)
    par = h64 @ d64                               # component along d_hat
    orth = h64 - par[:, None] * d64[None, :]
    for beta in (-0.5, 0.5, 2.0):
        out = O.steer_project(h, np.full(4, beta, np.float32), d).astype(np.float64)
        assert np.allclose(out @ d64, (1 + beta) * par, atol=2e-2)
        assert np.allclose(out - (out @ d64)[:, None] * d64[None, :], orth, atol=2.0 ** -7)
    # beta = -1 removes the component (up to the fp16 rounding of the result)
    out = O.steer_project(h, np.full(4, -1.0, np.float32), d).astype(np.float64)
    assert np.all(np.abs(out @ d64) < 2e-2)


def test_steer_latent_zero_rows_and_closed_forms():
    """Latent site: rows with strength 0 are the unsteered fp16 input; on a zero
    latent the add gives fp16(a * n * d) exactly; along a basis direction only
    that channel moves; projection of an orthogonal row is a no-op."""
    rng = np.random.default_rng(8)
    x = rng.standard_normal((6, 64)).astype(np.float32)
    d = np.zeros(64, np.float32)
    d[5] = 1.0
    a = np.array([0, 0.5, 0, -0.25, 1.0, 0], np.float32)
    out = O.steer_latent(x, a, 4.0, d)
    assert out.dtype == np.float16
    zero = a == 0
    assert out[zero].tobytes() == x[zero].astype(np.float16).tobytes()
    rest = np.delete(np.arange(64), 5)
    assert np.array_equal(out[:, rest], x[:, rest].astype(np.float16))
    assert np.array_equal(out[:, 5], (x[:, 5].astype(np.float64) + 4.0 * a).astype(np.float16))
    z = O.steer_latent(np.zeros((2, 64), np.float32), np.array([0.5, -2.0], np.float32), 3.0, d)
    assert z[0, 5] == np.float16(1.5) and z[1, 5] == np.float16(-6.0) and not z[:, rest].any()
    # projection: x + b (x . d) d scales channel 5 by (1 + b), one rounding of the fp32 state
    p = O.steer_latent(x, a, 4.0, d, mode="project")
    assert np.array_equal(p[:, 5], (x[:, 5].astype(np.float64) * (1 + a.astype(np.float64))).astype(np.float16))
    x[1, 5] = 0
    assert O.steer_latent(x, a, 4.0, d, mode="project")[1].tobytes() == x[1].astype(np.float16).tobytes()


def test_steer_text_only_cond_rows_of_each_request():
    """Text site: request r's cond rows [r*T, (r+1)*T) get strength alpha[r];
    the null-prompt rows and every row of a request with alpha 0 stay bitwise."""
    rng = np.random.default_rng(9)
    R, T, D = 3, 4, 32
    t = rng.standard_normal((2 * R * T, D)).astype(np.float16)
    d = rng.standard_normal(D)
    d = (d / np.linalg.norm(d)).astype(np.float32)
    a = np.array([0.5, 0.0, -1.0], np.float32)
    out = O.steer_text(t, R, T, a, 2.0, d)
    assert out[R * T:].tobytes() == t[R * T:].tobytes()
    assert out[T:2 * T].tobytes() == t[T:2 * T].tobytes()
    for r in (0, 2):
        rows = slice(r * T, (r + 1) * T)
        ref = (t[rows].astype(np.float64) + float(a[r]) * 2.0 * d.astype(np.float64)).astype(np.float16)
        assert np.array_equal(out[rows], ref)
    pr = O.steer_text(t, R, T, a, 2.0, d, mode="project")
    assert pr[R * T:].tobytes() == t[R * T:].tobytes()
    assert np.array_equal(pr[:T], O.steer_project(t[:T], np.full(T, 0.5, np.float32), d))


def test_mean_row_norm():
    h = np.array([[3, 4, 0], [0, 0, 1]], np.float16)
    assert O.mean_row_norm(h) == pytest.approx(3.0)   # (5 + 1) / 2


# ---------------------------------------------------------------- CFG merge

def test_cfg_special_values_and_affinity():
    rng = np.random.default_rng(6)
    c = rng.standard_normal((5, 64)).astype(np.float16)
    u = rng.standard_normal((5, 64)).astype(np.float16)
    assert np.array_equal(O.cfg_merge(c, u, 1.0), c.astype(np.float32))
    assert np.array_equal(O.cfg_merge(c, u, 0.0), u.astype(np.float32))
    cf, uf = c.astype(np.float64), u.astype(np.float64)
    for w in (3.0, 1.5, 4.75):
        assert np.allclose(O.cfg_merge(c, u, w), cf + (w - 1) * (cf - uf), rtol=1e-6, atol=1e-5)
    assert np.array_equal(O.cfg_merge(c, c, 3.0), c.astype(np.float32))


# ---------------------------------------------------------------- sampler

def test_euler_closed_form_and_constant_field():
    rng = np.random.default_rng(7)
    x0 = rng.standard_normal((10, 64)).astype(np.float32)
    eps = rng.standard_normal((10, 64)).astype(np.float32)
    # the exact velocity of the straight path x_t = (1-t) x0 + t eps is eps - x0;
    # Euler on any grid from t = 1 to 0 integrates it exactly (up to fp32 rounding)
    tg = 1 - np.arange(9) / 8
    x = eps.copy()
    for i in range(8):
        x = O.euler_update(x, eps - x0, tg[i], tg[i + 1])
    assert np.allclose(x, x0, atol=1e-5)
    y = O.euler_update(x0, eps, 1.0, 0.875)
    assert np.array_equal(y, (x0 + np.float32(-0.125) * eps).astype(np.float32))


def test_renoise_endpoints_and_path():
    rng = np.random.default_rng(8)
    x0 = rng.standard_normal((4, 64)).astype(np.float32)
    eps = rng.standard_normal((4, 64)).astype(np.float32)
    assert np.array_equal(O.renoise(x0, eps, 0.0), x0)
    assert np.array_equal(O.renoise(x0, eps, 1.0), eps)
    # warm start at t_k then exact-velocity Euler reaches x0
    N, k = 16, 6
    tg = 1 - np.arange(N + 1) / N
    x = O.renoise(x0, eps, tg[k])
    for i in range(k, N):
        x = O.euler_update(x, eps - x0, tg[i], tg[i + 1])
    assert np.allclose(x, x0, atol=1e-5)


# ---------------------------------------------------------------- DDIM sampler

def test_ddpm_alpha_bar_closed_forms():
    T, b1, bT = 1000, 1e-4, 0.02
    ab = O.ddpm_alpha_bar(T, b1, bT)
    assert ab.shape == (T,)
    assert ab[0] == pytest.approx(1 - b1, rel=1e-15)
    db = (bT - b1) / (T - 1)
    assert ab[1] == pytest.approx((1 - b1) * (1 - b1 - db), rel=1e-15)
    assert ab[T - 1] / ab[T - 2] == pytest.approx(1 - bT, rel=1e-12)   # last beta is beta_T
    assert np.all(np.diff(ab) < 0) and 0 < ab[-1] < 1e-4              # almost pure noise at T


def test_ddim_timesteps_grid():
    ts = I.ddim_timesteps(200, 1000)
    assert ts[0] == 995 and ts[-1] == 0 and len(ts) == 200 and np.all(np.diff(ts) == -5)
    ab = O.ddim_alpha_bars(I.TINY_DDIM, ts)
    assert ab.shape == (201,) and ab[-1] == 1.0 and np.all(np.diff(ab) > 0)


def test_ddim_update_closed_forms():
    """With the true noise as the prediction, a DDIM step moves the forward
    sample sqrt(a) x0 + sqrt(1-a) eps to the forward sample at a'; a' = a is
    the identity; a' = 1 returns the clean estimate."""
    rng = np.random.default_rng(21)
    x0 = rng.standard_normal((8, 64))
    eps = rng.standard_normal((8, 64))
    a, an = np.float32(0.3), np.float32(0.55)
    x = (np.sqrt(np.float64(a)) * x0 + np.sqrt(1 - np.float64(a)) * eps).astype(np.float32)
    e32 = eps.astype(np.float32)
    got = O.ddim_update(x, e32, a, an).astype(np.float64)
    want = np.sqrt(np.float64(an)) * x0 + np.sqrt(1 - np.float64(an)) * eps
    assert np.allclose(got, want, atol=2e-6)
    assert np.allclose(O.ddim_update(x, e32, a, a), x, rtol=0, atol=1e-6)
    x0_hat = (x.astype(np.float64) - np.sqrt(1 - np.float64(a)) * e32) / np.sqrt(np.float64(a))
    assert np.array_equal(O.ddim_update(x, e32, a, np.float32(1.0)), x0_hat.astype(np.float32))


def test_ddim_exact_noise_trajectory_recovers_x0():
    """200 DDIM steps on the linear-beta grid with the prediction fixed to the
    noise that made the start: the run ends at the clean latent."""
    rng = np.random.default_rng(22)
    x0 = rng.standard_normal((4, 64)).astype(np.float32)
    eps = rng.standard_normal((4, 64)).astype(np.float32)
    ab = O.ddim_alpha_bars(I.TINY_DDIM, I.ddim_timesteps(200, 1000))
    x = O.renoise_vp(x0, eps, ab[0])
    for i in range(200):
        x = O.ddim_update(x, eps, ab[i], ab[i + 1])
    assert np.allclose(x, x0, atol=1e-4)


def test_renoise_vp_endpoints_and_variance():
    rng = np.random.default_rng(23)
    x0 = rng.standard_normal((2000, 64)).astype(np.float32)
    eps = rng.standard_normal((2000, 64)).astype(np.float32)
    assert np.array_equal(O.renoise_vp(x0, eps, np.float32(1.0)), x0)
    assert np.array_equal(O.renoise_vp(x0, eps, np.float32(0.0)), eps)
    assert np.var(O.renoise_vp(x0, eps, np.float32(0.37))) == pytest.approx(1.0, abs=0.02)


def test_skip_arms_are_whole_steps():
    cfg = I.TINY_DDIM
    inp = I.make_ddim_warm_inputs(cfg, np.array([0, 5, 35, 65]))
    assert inp.start_step.tolist() == [0, 10, 70, 130]


def test_skip_start_step():
    assert O.skip_start_step(0.3, 16) == 5      # 4.8 + 0.5 -> 5
    assert O.skip_start_step(0.7, 16) == 11     # 11.2 + 0.5 -> 11
    assert O.skip_start_step(0.5, 8) == 4
    assert O.skip_start_step(0.0, 8) == 0
