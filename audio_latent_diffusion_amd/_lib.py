"""ctypes declarations of libald.so (the C ABI in include/ald.h).

Loading fails loudly when the library has not been built: there is no
fallback path of any kind.
"""
from __future__ import annotations

import ctypes
import os
from ctypes import POINTER, c_double, c_float, c_int, c_int64, c_size_t, c_uint, c_void_p

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libald.so")

ALD_OK, ALD_E_INVALID, ALD_E_UNSUPPORTED, ALD_E_WORKSPACE, ALD_E_LAUNCH = 0, -1, -2, -3, -4
ALD_W8A8, ALD_F16, ALD_Q4, ALD_W8A16 = 0, 1, 2, 3
ALD_ACT_NONE, ALD_ACT_GELU = 0, 1
ALD_PREQUANT = 1
ALD_EULER, ALD_RENOISE, ALD_DDIM, ALD_RENOISE_VP = 0, 1, 2, 3
ALD_SAMPLER_FLOW, ALD_SAMPLER_DDIM = 0, 1
SAMPLERS = {"flow": ALD_SAMPLER_FLOW, "ddim": ALD_SAMPLER_DDIM}
ALD_STEER_ADD, ALD_STEER_PROJECT = 0, 1
STEER_MODES = {"add": ALD_STEER_ADD, "project": ALD_STEER_PROJECT}
ALD_SITE_RESIDUAL, ALD_SITE_LATENT, ALD_SITE_TEXT = 0, 1, 2
STEER_SITES = {"residual": ALD_SITE_RESIDUAL, "latent": ALD_SITE_LATENT, "text": ALD_SITE_TEXT}

ALD_STATIC_SCRATCH_BYTES = 64 << 20  # scratch array of dit_step_static, per device

WMODES = {"w8a8": ALD_W8A8, "f16": ALD_F16, "q4": ALD_Q4, "w8a16": ALD_W8A16}

# every extern "C" entry point of include/ald.h
EXPORTS = (
    "ald_strerror", "ald_version", "quantize_rows_q8", "quantize_q4", "ln_quant", "ln_f16",
    "w8a8_linear", "q8w_linear", "q4_linear", "f16_linear", "attn_fwd", "steer_add", "steer_latent", "cfg_merge",
    "sampler_update", "ddim_alpha_bar", "dit_workspace_size", "dit_text_kv", "dit_step", "dit_step_static", "dit_graph_capture",
    "dit_graph_launch", "dit_graph_nodes", "dit_graph_destroy",
)


class AldError(RuntimeError):
    def __init__(self, fn: str, code: int, msg: str):
        super().__init__(f"{fn} failed: {msg} (code {code})")
        self.code = code


class dit_config(ctypes.Structure):
    _fields_ = [("n_blocks", c_int), ("hidden", c_int), ("n_heads", c_int), ("head_dim", c_int),
                ("mlp", c_int), ("channels", c_int), ("text_tokens", c_int), ("text_dim", c_int),
                ("wmode", c_int), ("steer_block", c_int), ("ln_eps", c_float), ("steer_mode", c_int),
                ("steer_site", c_int), ("sampler", c_int)]


class dit_linear(ctypes.Structure):
    _fields_ = [("w", c_void_p), ("scale", c_void_p), ("bias", c_void_p)]


class dit_block_weights(ctypes.Structure):
    _fields_ = [("ln1_g", c_void_p), ("ln1_b", c_void_p), ("ln2_g", c_void_p), ("ln2_b", c_void_p),
                ("ln3_g", c_void_p), ("ln3_b", c_void_p),
                ("qkv", dit_linear), ("o", dit_linear), ("q", dit_linear), ("kv", dit_linear),
                ("ox", dit_linear), ("up", dit_linear), ("down", dit_linear)]


class dit_weights(ctypes.Structure):
    _fields_ = [("blocks", POINTER(dit_block_weights)), ("w_in", c_void_p), ("b_in", c_void_p),
                ("lnf_g", c_void_p), ("lnf_b", c_void_p), ("w_out", c_void_p), ("b_out", c_void_p),
                ("kv_all", dit_linear)]


class dit_step_args(ctypes.Structure):
    _fields_ = [("x", c_void_p), ("text_kv", c_void_p), ("R", c_int), ("seq", c_int),
                ("cu_seqlens", c_void_p), ("row_req", c_void_p), ("n_tok", c_int64), ("max_seq", c_int),
                ("t_cur", c_void_p), ("t_next", c_void_p), ("guidance", c_void_p), ("alpha", c_void_p),
                ("resid_norm", c_float), ("direction", c_void_p), ("active", c_void_p),
                ("renoise", c_void_p), ("x0", c_void_p), ("eps", c_void_p), ("v_out", c_void_p),
                ("block_norms", c_void_p), ("text", c_void_p), ("abar_cur", c_void_p),
                ("abar_next", c_void_p)]


_lib = None


def _declare(lib):
    V, I, I64, F = c_void_p, c_int, c_int64, c_float
    sig = {
        "ald_strerror": (ctypes.c_char_p, [I]),
        "ald_version": (I, []),
        "quantize_rows_q8": (I, [V, I64, I, I, V, I64, V, V]),
        "quantize_q4": (I, [V, I, I, V, V, V]),
        "ln_quant": (I, [V, I64, I, I, V, V, F, V, V, V, V]),
        "ln_f16": (I, [V, I64, I, I, V, V, F, V, I64, V]),
        "w8a8_linear": (I, [V, I64, I, I, V, V, I, V, V, I64, I, V, I64, V, V, V, c_uint, V]),
        "q4_linear": (I, [V, I64, I, I, V, V, I, V, V, I64, I, V, I64, V]),
        "q8w_linear": (I, [V, I64, I, I, V, V, I, V, V, I64, I, V, I64, V]),
        "f16_linear": (I, [V, I64, I, I, V, I, V, V, I64, I, V, I64, V]),
        "attn_fwd": (I, [V, V, V, I64, I64, I, I, I, I, I, V, V, I, I, F, V, I64, V]),
        "steer_add": (I, [V, I64, I, I, I, I, V, V, F, V, I, V]),
        "steer_latent": (I, [V, V, I64, I, I, I, V, V, F, V, I, V]),
        "cfg_merge": (I, [V, I64, I, I, V, V, V, V]),
        "sampler_update": (I, [I, V, V, V, V, I64, I, I, V, V, V, V, V]),
        "ddim_alpha_bar": (I, [I, c_double, c_double, V, I, V]),
        "dit_workspace_size": (c_size_t, [POINTER(dit_config), I64, I]),
        "dit_text_kv": (I, [POINTER(dit_config), POINTER(dit_weights), V, I, V, V, c_size_t, V]),
        "dit_step": (I, [POINTER(dit_config), POINTER(dit_weights), POINTER(dit_step_args), V, c_size_t, V]),
        "dit_step_static": (I, [POINTER(dit_config), POINTER(dit_weights), POINTER(dit_step_args), V]),
        "dit_graph_capture": (I, [POINTER(dit_config), POINTER(dit_weights), POINTER(dit_step_args), I, V,
                                  c_size_t, V, POINTER(c_void_p)]),
        "dit_graph_launch": (I, [V, V]),
        "dit_graph_nodes": (I, [V, POINTER(c_size_t)]),
        "dit_graph_destroy": (I, [V]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args


def lib():
    """The loaded libald.so (built by __graft_entry__.build())."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build the HIP library first "
                              "(python -c 'import __graft_entry__ as g; g.build()')")
        l = ctypes.CDLL(LIB_PATH)
        _declare(l)
        _lib = l
    return _lib


def check(fn: str, code: int) -> None:
    if code != ALD_OK:
        raise AldError(fn, code, lib().ald_strerror(code).decode())
