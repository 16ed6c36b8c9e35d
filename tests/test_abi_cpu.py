"""The C ABI on the CPU: the library loads, exports every declared entry
point, and its host-side validation rejects bad arguments before any launch
(no GPU needed: every device entry point called here fails validation, so
nothing touches HIP; the host-only schedule helper runs for real)."""
import ctypes
import os
import re

import numpy as np
import pytest

from audio_latent_diffusion_amd import _lib as L

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ald.h")

FAKE = 0x10000  # a 16-byte aligned non-null "device" address, never dereferenced on the host


def header_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\*?\s*([a-z_][a-z0-9_]*)\s*\(", src, flags=re.M)
    return sorted(set(names))


def test_header_lists_the_binding_exports():
    assert header_functions() == sorted(L.EXPORTS)


def test_library_exports_every_declared_symbol():
    lib = L.lib()
    for name in header_functions():
        assert hasattr(lib, name), name
    assert lib.ald_version() == 202
    assert lib.ald_strerror(L.ALD_E_WORKSPACE) == b"workspace too small"


def test_gemm_validation():
    lib = L.lib()
    # null weights
    assert lib.w8a8_linear(FAKE, 64, 4, 64, None, FAKE, 8, None, None, 0, 0, FAKE, 8, FAKE, FAKE, None, 0,
                           None) == L.ALD_E_INVALID
    # K not a multiple of 16
    assert lib.w8a8_linear(FAKE, 72, 4, 24, FAKE, FAKE, 8, None, None, 0, 0, FAKE, 8, FAKE, FAKE, None, 0,
                           None) == L.ALD_E_INVALID
    # misaligned activation pointer
    assert lib.w8a8_linear(FAKE + 2, 64, 4, 64, FAKE, FAKE, 8, None, None, 0, 0, FAKE, 8, FAKE, FAKE, None, 0,
                           None) == L.ALD_E_INVALID
    # unknown flag, bad activation
    assert lib.w8a8_linear(FAKE, 64, 4, 64, FAKE, FAKE, 8, None, None, 0, 0, FAKE, 8, FAKE, FAKE, None, 4,
                           None) == L.ALD_E_INVALID
    assert lib.w8a8_linear(FAKE, 64, 4, 64, FAKE, FAKE, 8, None, None, 0, 7, FAKE, 8, FAKE, FAKE, None, 0,
                           None) == L.ALD_E_INVALID
    # K beyond the register-resident quantizer
    assert lib.w8a8_linear(FAKE, 16384, 4, 16384, FAKE, FAKE, 8, None, None, 0, 0, FAKE, 8, FAKE, FAKE, None, 0,
                           None) == L.ALD_E_UNSUPPORTED
    # empty problems are a no-op success
    assert lib.w8a8_linear(None, 64, 0, 64, None, None, 8, None, None, 0, 0, None, 8, None, None, None, 0,
                           None) == L.ALD_OK
    assert lib.q4_linear(FAKE, 64, 4, 48, FAKE, FAKE, 8, None, None, 0, 0, FAKE, 8, None) == L.ALD_E_UNSUPPORTED
    # 8-bit weight-only: K must be whole 64-element slices; a missing scale is invalid
    assert lib.q8w_linear(FAKE, 96, 4, 96, FAKE, FAKE, 8, None, None, 0, 0, FAKE, 8, None) == L.ALD_E_UNSUPPORTED
    assert lib.q8w_linear(FAKE, 64, 4, 64, FAKE, None, 8, None, None, 0, 0, FAKE, 8, None) == L.ALD_E_INVALID
    assert lib.q8w_linear(FAKE, 60, 4, 64, FAKE, FAKE, 8, None, None, 0, 0, FAKE, 8, None) == L.ALD_E_INVALID
    assert lib.q8w_linear(None, 64, 0, 64, None, None, 8, None, None, 0, 0, None, 8, None) == L.ALD_OK
    assert lib.f16_linear(FAKE, 64, 4, 64, None, 8, None, None, 0, 0, FAKE, 8, None) == L.ALD_E_INVALID
    assert lib.quantize_q4(FAKE, 4, 48, FAKE, FAKE, None) == L.ALD_E_UNSUPPORTED
    assert lib.quantize_rows_q8(FAKE, 64, 4, 60, FAKE, 64, FAKE, None) == L.ALD_E_INVALID


def test_attention_and_elementwise_validation():
    lib = L.lib()
    assert lib.attn_fwd(FAKE, FAKE, FAKE, 128, 128, 2, 128, 1, 8, 8, None, None, 0, 0, 0.1, FAKE, 128,
                        None) == L.ALD_E_UNSUPPORTED  # head_dim 128
    assert lib.attn_fwd(FAKE, FAKE, FAKE, 64, 64, 2, 64, 1, 8, 8, None, None, 0, 0, 0.1, FAKE, 128,
                        None) == L.ALD_E_INVALID      # stride narrower than n_heads * 64
    assert lib.attn_fwd(None, FAKE, FAKE, 128, 128, 2, 64, 1, 8, 8, None, None, 0, 0, 0.1, FAKE, 128,
                        None) == L.ALD_E_INVALID
    assert lib.steer_add(FAKE, 64, 4, 64, 4, 1, None, FAKE, 1.0, FAKE, 9, None) == L.ALD_E_INVALID
    assert lib.steer_add(FAKE, 64, 4, 64, 0, 1, None, FAKE, 1.0, FAKE, 0, None) == L.ALD_E_INVALID
    assert lib.steer_add(FAKE, 16384, 4, 16384, 1, 1, None, FAKE, 1.0, FAKE, 0, None) == L.ALD_E_UNSUPPORTED
    assert lib.steer_latent(FAKE, FAKE, 8, 64, 8, 1, None, FAKE, 1.0, FAKE, 0, None) == L.ALD_E_INVALID  # in place
    assert lib.steer_latent(FAKE, FAKE + 4096, 8, 1024, 8, 1, None, FAKE, 1.0, FAKE, 0, None) == L.ALD_E_UNSUPPORTED
    assert lib.steer_latent(FAKE, FAKE + 4096, 8, 62, 8, 1, None, FAKE, 1.0, FAKE, 0, None) == L.ALD_E_INVALID
    assert lib.steer_latent(FAKE, FAKE + 4096, 8, 64, 8, 1, None, FAKE, 1.0, FAKE, 2, None) == L.ALD_E_INVALID
    assert lib.steer_latent(None, None, 0, 64, 8, 1, None, None, 1.0, None, 0, None) == L.ALD_OK
    assert lib.cfg_merge(FAKE, 10, 64, 0, None, FAKE, FAKE, None) == L.ALD_E_INVALID
    assert lib.sampler_update(5, FAKE, FAKE, None, None, 10, 64, 10, None, FAKE, FAKE, None, None) == L.ALD_E_INVALID
    assert lib.sampler_update(L.ALD_RENOISE, FAKE, None, None, FAKE, 10, 64, 10, None, FAKE, None, None,
                              None) == L.ALD_E_INVALID
    # latent kernels index vectors of 4 values with 32-bit arithmetic
    big = 1 << 27  # 2^27 tokens x 64 channels = 2^31 vectors of 4
    assert lib.cfg_merge(FAKE, big, 64, big, None, FAKE, FAKE, None) == L.ALD_E_UNSUPPORTED
    assert lib.sampler_update(L.ALD_EULER, FAKE, FAKE, None, None, big, 64, big, None, FAKE, FAKE, None,
                              None) == L.ALD_E_UNSUPPORTED


def _cfg(**kw):
    d = dict(n_blocks=2, hidden=256, n_heads=4, head_dim=64, mlp=1024, channels=64, text_tokens=32, text_dim=256,
             wmode=L.ALD_W8A8, steer_block=1, ln_eps=1e-5, steer_mode=L.ALD_STEER_ADD,
             steer_site=L.ALD_SITE_RESIDUAL, sampler=L.ALD_SAMPLER_FLOW)
    d.update(kw)
    return L.dit_config(**d)


def _weights(n):
    arr = (L.dit_block_weights * n)()
    for i in range(n):
        b = arr[i]
        for nm in ("ln1_g", "ln1_b", "ln2_g", "ln2_b", "ln3_g", "ln3_b"):
            setattr(b, nm, FAKE)
        for nm in ("qkv", "o", "q", "kv", "ox", "up", "down"):
            setattr(b, nm, L.dit_linear(FAKE, FAKE, FAKE))
    w = L.dit_weights(ctypes.cast(arr, ctypes.POINTER(L.dit_block_weights)), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE)
    return w, arr


def test_workspace_size():
    lib = L.lib()
    c = _cfg()
    n = lib.dit_workspace_size(ctypes.byref(c), 64, 1)
    M, H, F = 128, 256, 1024
    assert n >= 2 * M * H + 2 * M * 3 * H + 2 * M * H * 2 + M * F
    assert lib.dit_workspace_size(ctypes.byref(c), 128, 1) > n
    bad = _cfg(head_dim=128)
    assert lib.dit_workspace_size(ctypes.byref(bad), 64, 1) == 0


def test_step_validation():
    lib = L.lib()
    c = _cfg()
    w, arr = _weights(2)
    a = L.dit_step_args(x=FAKE, text_kv=FAKE, R=1, seq=64, n_tok=64, max_seq=64, t_cur=FAKE, t_next=FAKE,
                        guidance=FAKE, alpha=FAKE, resid_norm=1.0, direction=FAKE)
    need = lib.dit_workspace_size(ctypes.byref(c), 64, 1)
    assert lib.dit_step(ctypes.byref(c), ctypes.byref(w), ctypes.byref(a), FAKE, need - 1,
                        None) == L.ALD_E_WORKSPACE
    bad = _cfg(head_dim=32, n_heads=8)
    assert lib.dit_step(ctypes.byref(bad), ctypes.byref(w), ctypes.byref(a), FAKE, need, None) == L.ALD_E_UNSUPPORTED
    bad = _cfg(steer_mode=7)
    assert lib.dit_step(ctypes.byref(bad), ctypes.byref(w), ctypes.byref(a), FAKE, need, None) == L.ALD_E_INVALID
    bad = _cfg(steer_site=3)
    assert lib.dit_step(ctypes.byref(bad), ctypes.byref(w), ctypes.byref(a), FAKE, need, None) == L.ALD_E_INVALID
    bad = _cfg(sampler=2)
    assert lib.dit_step(ctypes.byref(bad), ctypes.byref(w), ctypes.byref(a), FAKE, need, None) == L.ALD_E_INVALID
    # the DDIM sampler reads alpha_bar, which these args do not give
    dd = _cfg(sampler=L.ALD_SAMPLER_DDIM)
    assert lib.dit_step(ctypes.byref(dd), ctypes.byref(w), ctypes.byref(a), FAKE, need, None) == L.ALD_E_INVALID
    # the text site reads the raw text, which these args do not give
    txt = _cfg(steer_site=L.ALD_SITE_TEXT)
    need_t = lib.dit_workspace_size(ctypes.byref(txt), 64, 1)
    assert need_t > need  # steered text, its codes and one block's K/V
    assert lib.dit_step(ctypes.byref(txt), ctypes.byref(w), ctypes.byref(a), FAKE, need_t, None) == L.ALD_E_INVALID
    lat = _cfg(steer_site=L.ALD_SITE_LATENT)
    assert lib.dit_workspace_size(ctypes.byref(lat), 64, 1) == need + 64 * 64 * 4
    assert lib.dit_step(ctypes.byref(lat), ctypes.byref(w), ctypes.byref(a), FAKE, need, None) == L.ALD_E_WORKSPACE
    assert lib.dit_workspace_size(ctypes.byref(_cfg(steer_site=L.ALD_SITE_LATENT, steer_block=-1)), 64, 1) == need
    bad = _cfg(steer_block=2)
    assert lib.dit_step(ctypes.byref(bad), ctypes.byref(w), ctypes.byref(a), FAKE, need, None) == L.ALD_E_INVALID
    bad = _cfg(wmode=7)
    assert lib.dit_step(ctypes.byref(bad), ctypes.byref(w), ctypes.byref(a), FAKE, need, None) == L.ALD_E_INVALID
    # W8A16 needs the widths in whole 64-element slices
    bad = _cfg(wmode=L.ALD_W8A16, text_dim=96)
    assert lib.dit_step(ctypes.byref(bad), ctypes.byref(w), ctypes.byref(a), FAKE, need, None) == L.ALD_E_UNSUPPORTED
    a2 = L.dit_step_args(x=FAKE, text_kv=FAKE, R=1, seq=60, n_tok=64, max_seq=64, t_cur=FAKE, t_next=FAKE,
                         guidance=FAKE, alpha=FAKE, resid_norm=1.0, direction=FAKE)
    assert lib.dit_step(ctypes.byref(c), ctypes.byref(w), ctypes.byref(a2), FAKE, need, None) == L.ALD_E_INVALID
    a3 = L.dit_step_args(x=FAKE, text_kv=FAKE, R=1, seq=64, n_tok=64, max_seq=64, t_cur=FAKE, t_next=FAKE,
                         guidance=FAKE, alpha=None, resid_norm=1.0, direction=FAKE)
    assert lib.dit_step(ctypes.byref(c), ctypes.byref(w), ctypes.byref(a3), FAKE, need, None) == L.ALD_E_INVALID
    a4 = L.dit_step_args(x=FAKE, text_kv=FAKE, R=2, seq=0, cu_seqlens=FAKE, row_req=None, n_tok=64, max_seq=64,
                         t_cur=FAKE, t_next=FAKE, guidance=FAKE, alpha=FAKE, resid_norm=1.0, direction=FAKE)
    assert lib.dit_step(ctypes.byref(c), ctypes.byref(w), ctypes.byref(a4), FAKE, need, None) == L.ALD_E_INVALID
    arr[1].qkv = L.dit_linear(None, FAKE, FAKE)
    assert lib.dit_step(ctypes.byref(c), ctypes.byref(w), ctypes.byref(a), FAKE, need, None) == L.ALD_E_INVALID
    h = ctypes.c_void_p()
    assert lib.dit_graph_capture(ctypes.byref(c), ctypes.byref(w), ctypes.byref(a), 0, FAKE, need, FAKE,
                                 ctypes.byref(h)) == L.ALD_E_INVALID
    assert lib.dit_graph_launch(None, None) == L.ALD_E_INVALID
    n = ctypes.c_size_t()
    assert lib.dit_graph_nodes(None, ctypes.byref(n)) == L.ALD_E_INVALID
    assert lib.dit_graph_destroy(None) == L.ALD_E_INVALID


def test_attention_scale_must_be_finite_and_positive():
    """The softmax's running reference maximum is kept in units of the scaled
    score: a zero, negative or non-finite scale is rejected before launch."""
    lib = L.lib()
    for scale in (0.0, -0.125, float("nan"), float("inf")):
        assert lib.attn_fwd(FAKE, FAKE, FAKE, 128, 128, 2, 64, 1, 8, 8, None, None, 0, 0, scale, FAKE, 128,
                            None) == L.ALD_E_INVALID, scale


def test_text_kv_required_only_where_read():
    """text_kv is read unless the step steers the text site (which recomputes
    the K/V from the steered text): NULL is invalid at the residual site and
    passes validation at the text site (here the step then stops at the
    too-small workspace, before any launch)."""
    lib = L.lib()
    w, arr = _weights(2)
    a = L.dit_step_args(x=FAKE, text_kv=None, R=1, seq=64, n_tok=64, max_seq=64, t_cur=FAKE, t_next=FAKE,
                        guidance=FAKE, alpha=FAKE, resid_norm=1.0, direction=FAKE, text=FAKE)
    c = _cfg()
    need = lib.dit_workspace_size(ctypes.byref(c), 64, 1)
    assert lib.dit_step(ctypes.byref(c), ctypes.byref(w), ctypes.byref(a), FAKE, need, None) == L.ALD_E_INVALID
    txt = _cfg(steer_site=L.ALD_SITE_TEXT)
    need_t = lib.dit_workspace_size(ctypes.byref(txt), 64, 1)
    assert lib.dit_step(ctypes.byref(txt), ctypes.byref(w), ctypes.byref(a), FAKE, need_t - 1,
                        None) == L.ALD_E_WORKSPACE


def test_w8a16_stacked_text_kv_weight_bytes_checked():
    """The 8-bit weight-only GEMM addresses its weights with 32-bit byte
    offsets: stacked text K/V linears of n_blocks * 2H * D_t >= 2^32 bytes have
    no kernel, and the text-site step says so before any launch (one block's
    K/V linear, 2H * D_t bytes, is fine)."""
    lib = L.lib()
    nb, H, Dt = 32, 8192, 8192
    c = _cfg(n_blocks=nb, hidden=H, n_heads=H // 64, mlp=H, text_dim=Dt, text_tokens=32, wmode=L.ALD_W8A16,
             steer_site=L.ALD_SITE_TEXT, steer_block=0)
    assert nb * 2 * H * Dt >= 1 << 32
    w, arr = _weights(nb)
    w.kv_all = L.dit_linear(FAKE, FAKE, FAKE)
    a = L.dit_step_args(x=FAKE, text_kv=None, R=1, seq=32, n_tok=32, max_seq=32, t_cur=FAKE, t_next=FAKE,
                        guidance=FAKE, alpha=FAKE, resid_norm=1.0, direction=FAKE, text=FAKE)
    need = lib.dit_workspace_size(ctypes.byref(c), 32, 1)
    assert need > 0
    assert lib.dit_step(ctypes.byref(c), ctypes.byref(w), ctypes.byref(a), FAKE, need, None) == L.ALD_E_UNSUPPORTED
    # the same weights as one q8w_linear call are rejected the same way
    assert lib.q8w_linear(FAKE, Dt, 64, Dt, FAKE, FAKE, nb * 2 * H, None, None, 0, 0, FAKE, nb * 2 * H,
                          None) == L.ALD_E_UNSUPPORTED


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(L, "_lib", None)
    monkeypatch.setattr(L, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(ImportError):
        L.lib()


def test_ddim_alpha_bar_host_helper_matches_oracle():
    """The library's schedule helper (host C++) and the oracle's schedule are
    independent codes of the same linear-beta product; they agree to fp32."""
    from audio_latent_diffusion_amd import binding as B
    from oracle import ald_oracle as O
    import ald_inputs as I
    cfg = I.TINY_DDIM
    ts = I.ddim_timesteps(200, 1000)
    got = B.ddim_alpha_bar(cfg.train_steps, cfg.beta_1, cfg.beta_T, ts)
    ref = O.ddim_alpha_bars(cfg, ts)
    assert got.shape == ref.shape and got[-1] == 1.0
    assert np.allclose(got, ref, rtol=2.0 ** -23, atol=0)
    lib = L.lib()
    out = np.empty(3, np.float32)
    bad_ts = np.array([0, 1000], np.int32)
    assert lib.ddim_alpha_bar(1000, 1e-4, 0.02, bad_ts.ctypes.data_as(ctypes.c_void_p), 2,
                              out.ctypes.data_as(ctypes.c_void_p)) == L.ALD_E_INVALID
    assert lib.ddim_alpha_bar(1, 1e-4, 0.02, None, 0, out.ctypes.data_as(ctypes.c_void_p)) == L.ALD_E_INVALID
    assert lib.ddim_alpha_bar(1000, 1e-4, 0.02, None, 0, out.ctypes.data_as(ctypes.c_void_p)) == L.ALD_OK
    assert out[0] == 1.0
    # sampler ops: an unknown op and a DDIM update without its prediction are rejected
    assert lib.sampler_update(4, FAKE, FAKE, None, None, 10, 64, 10, None, FAKE, FAKE, None, None) == L.ALD_E_INVALID
    assert lib.sampler_update(L.ALD_DDIM, FAKE, None, None, None, 10, 64, 10, None, FAKE, FAKE, None,
                              None) == L.ALD_E_INVALID
    assert lib.sampler_update(L.ALD_RENOISE_VP, FAKE, None, FAKE, None, 10, 64, 10, None, FAKE, None, None,
                              None) == L.ALD_E_INVALID


def test_bench_refuses_more_than_one_gpu():
    """bench.py measures one GPU: --gpus above 1 exits with a message before
    any device work."""
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120, cwd=root)
    assert r.returncode != 0
    assert "one GPU" in r.stderr
