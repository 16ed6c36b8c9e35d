"""Long latent sequences (latent length >= 4096, long-form clips) and
continuous-batching varlen packs with long members.

Attention rows are independent, so at lengths where the oracle's full
score matrix is too large the check takes sampled query rows of every
sequence against all of that sequence's keys (bar 2^-8 per element as in the
short-sequence attention tests).  The tiny model's full step at a 4096-token
latent is checked element by element on the output latent (bar 2e-2).
"""
import numpy as np
import pytest

import ald_inputs as I
from audio_latent_diffusion_amd import binding as B
from audio_latent_diffusion_amd import runtime
from oracle import ald_oracle as O
from tests._gpu import dev, f16_close, host, needs_gpu

pytestmark = [pytest.mark.gpu, needs_gpu]


def rng(seed):
    return np.random.default_rng(seed)


def _sampled_ref(q, k, v, nh, cu_q, cu_k, rows_per_seq, seed):
    """Oracle rows for a sample of query rows of every sequence."""
    r = np.random.default_rng(seed)
    picks, refs = [], []
    for b in range(len(cu_q) - 1):
        q0, q1, k0, k1 = int(cu_q[b]), int(cu_q[b + 1]), int(cu_k[b]), int(cu_k[b + 1])
        if q1 == q0:
            continue
        n = min(rows_per_seq, q1 - q0)
        rows = np.unique(np.concatenate([r.choice(np.arange(q0, q1), n, replace=False), [q0, q1 - 1]]))
        sub_cu_q = np.array([0, len(rows)])
        sub_cu_k = np.array([0, k1 - k0])
        refs.append(O.attention_varlen(q[rows], k[k0:k1], v[k0:k1], sub_cu_q, sub_cu_k, nh, 0.125))
        picks.append(rows)
    return np.concatenate(picks), np.concatenate(refs)


@pytest.mark.parametrize("S,nh", [(4096, 4), (8192, 2)])
def test_attention_long_dense_sampled(S, nh):
    r = rng(S + nh)
    W = nh * 64
    Bn = 2  # a CFG pair
    q = r.standard_normal((Bn * S, W)).astype(np.float16)
    k = r.standard_normal((Bn * S, W)).astype(np.float16)
    v = r.standard_normal((Bn * S, W)).astype(np.float16)
    out = host(B.attn_fwd(dev(q), dev(k), dev(v), nh, Bn, S, S))
    cu = np.arange(Bn + 1) * S
    rows, ref = _sampled_ref(q, k, v, nh, cu, cu, 48, S)
    f16_close(out[rows], ref, rtol=2.0 ** -8, atol_frac=2.0 ** -8)


def test_attention_long_varlen_pack_sampled():
    """Continuous-batching pack: long and short members, one of them empty."""
    r = rng(11)
    lens = [4096, 1, 0, 2500, 8192, 129]
    nh = 2
    W = nh * 64
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    q = r.standard_normal((cu[-1], W)).astype(np.float16)
    k = r.standard_normal((cu[-1], W)).astype(np.float16)
    v = r.standard_normal((cu[-1], W)).astype(np.float16)
    out = host(B.attn_fwd(dev(q), dev(k), dev(v), nh, len(lens), cu_seqlens_q=dev(cu), cu_seqlens_k=dev(cu),
                          max_sq=max(lens), max_sk=max(lens)))
    rows, ref = _sampled_ref(q, k, v, nh, cu, cu, 40, 12)
    f16_close(out[rows], ref, rtol=2.0 ** -8, atol_frac=2.0 ** -8)


def test_tiny_model_long_latent_step():
    """Tiny model (2 blocks, hidden 256), one request with a 4096-token latent,
    steering active: the step's output latent against the oracle."""
    cfg = I.TINY.replace(seq=4096)
    p = I.make_params(cfg)
    inp = I.make_inputs(cfg)
    run = runtime.StepRunner(runtime.DiTModel(cfg, p), inp.x, inp.text, inp.seqlens, inp.t_grid, inp.guidance,
                             inp.alpha, inp.direction, 5.0, start_step=inp.start_step, x0=inp.x0, eps=inp.eps)
    run.step(0)
    got = host(run.x)
    ref, _ = O.run_sampler(O.prepare_model(cfg, p), inp, resid_norm=5.0, steps=[0])
    err = O.normwise_rel_err(got, ref)
    print(f"tiny, latent 4096: err {err:.2e}")
    assert err < 2e-2
