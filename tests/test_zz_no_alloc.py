"""dit_step_static, the step entry point that allocates nothing, against
dit_step with a caller workspace, through the C ABI.

Both run the same kernels on the same inputs, so their results must be
identical bit for bit.  Two calls in a row share the device's scratch array:
the first a steered step of the mid-size model (one request of 256 latent
tokens), the second a smaller packed step of the tiny model, which runs on
what the first call left in the array.
"""
import ctypes

import numpy as np
import pytest
import torch

import ald_inputs as I
from audio_latent_diffusion_amd import _lib as L
from audio_latent_diffusion_amd import runtime
from tests._gpu import host, needs_gpu

pytestmark = [pytest.mark.gpu, needs_gpu]


def _runner(model, inp, resid):
    return runtime.StepRunner(model, inp.x, inp.text, inp.seqlens, inp.t_grid, inp.guidance, inp.alpha,
                              inp.direction, resid, start_step=inp.start_step, x0=inp.x0, eps=inp.eps,
                              timesteps=inp.timesteps, keep_velocity=True)


def _static_step(run, i):
    m = run.model
    L.check("dit_step_static", L.lib().dit_step_static(ctypes.byref(m.c_cfg), ctypes.byref(m.c_weights),
                                                       ctypes.byref(run._args[i]),
                                                       torch.cuda.current_stream().cuda_stream))


def _compare(model, inp, steps, resid):
    ws = _runner(model, inp, resid)
    st = _runner(model, inp, resid)
    need = model.workspace_size(st.n_tok, st.R)
    assert need <= L.ALD_STATIC_SCRATCH_BYTES
    for i in steps:
        ws.step(i)
        _static_step(st, i)
    assert np.all(np.isfinite(host(st.x)))
    assert host(st.x).tobytes() == host(ws.x).tobytes()
    assert host(st.v_out).tobytes() == host(ws.v_out).tobytes()
    return need


def test_static_step_equals_workspace_step_on_two_calls():
    mid = I.MID
    m1 = runtime.DiTModel(mid, I.make_params(mid))
    need1 = _compare(m1, I.make_inputs(mid), [2, 3], 75.0)  # steps inside the steering span
    del m1
    tiny = I.TINY.replace(requests=2)
    m2 = runtime.DiTModel(tiny, I.make_params(tiny))
    inp = I.make_mixed_inputs(tiny, seqlens=np.array([40, 17]), warm=np.zeros(2, bool))
    need2 = _compare(m2, inp, [0], 5.0)
    assert need2 < need1


def test_static_step_refuses_more_than_its_scratch():
    """A step that needs more than the array is refused before any launch."""
    cfg = I.SERVE
    model = runtime.DiTModel(cfg.replace(n_blocks=1, steer_block=0), I.make_params(cfg.replace(n_blocks=1,
                                                                                           steer_block=0)))
    inp = I.make_inputs(cfg.replace(n_blocks=1, steer_block=0))
    run = runtime.StepRunner(model, inp.x, inp.text, inp.seqlens, inp.t_grid, inp.guidance, inp.alpha,
                             inp.direction, 1.0)
    assert model.workspace_size(run.n_tok, run.R) > L.ALD_STATIC_SCRATCH_BYTES
    x_before = host(run.x).copy()
    m = run.model
    rc = L.lib().dit_step_static(ctypes.byref(m.c_cfg), ctypes.byref(m.c_weights), ctypes.byref(run._args[0]),
                                 torch.cuda.current_stream().cuda_stream)
    assert rc == L.ALD_E_WORKSPACE
    assert host(run.x).tobytes() == x_before.tobytes()
