"""Thin Python binding of the C ABI, one function per entry point, same names.

Argument marshalling only: shapes and dtypes are read from torch tensors,
outputs are allocated when not given, and the call is enqueued on torch's
current stream.  Every computation happens inside libald.so.
"""
from __future__ import annotations

import ctypes
from typing import Optional

import numpy as np
import torch

from . import _lib as L


def _p(t: Optional[torch.Tensor]):
    return None if t is None else t.data_ptr()


def _stream():
    return torch.cuda.current_stream().cuda_stream


def _dev(t: torch.Tensor, dtype=None, name="tensor"):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if t.dim() >= 1 and t.stride(-1) != 1:
        raise ValueError(f"{name} must have unit stride in its last dimension")
    return t


def _ld(t: torch.Tensor) -> int:
    return t.stride(0) if t.dim() == 2 else t.shape[-1]


def quantize_rows_q8(x, q=None, scale=None):
    _dev(x, torch.float16, "x")
    M, K = x.shape
    q = torch.empty((M, K), dtype=torch.int8, device=x.device) if q is None else q
    scale = torch.empty(M, dtype=torch.float32, device=x.device) if scale is None else scale
    L.check("quantize_rows_q8", L.lib().quantize_rows_q8(_p(x), _ld(x), M, K, _p(q), _ld(q), _p(scale), _stream()))
    return q, scale


def quantize_q4(w, packed=None, scales=None):
    _dev(w, torch.float16, "w")
    N, K = w.shape
    packed = torch.empty((N, K // 2), dtype=torch.uint8, device=w.device) if packed is None else packed
    scales = torch.empty((N, K // 32), dtype=torch.float16, device=w.device) if scales is None else scales
    L.check("quantize_q4", L.lib().quantize_q4(_p(w.contiguous()), N, K, _p(packed), _p(scales), _stream()))
    return packed, scales


def ln_quant(x, gamma, beta, eps=1e-5, u_out=None, q=None, scale=None):
    _dev(x, torch.float16, "x")
    M, H = x.shape
    q = torch.empty((M, H), dtype=torch.int8, device=x.device) if q is None else q
    scale = torch.empty(M, dtype=torch.float32, device=x.device) if scale is None else scale
    L.check("ln_quant", L.lib().ln_quant(_p(x), _ld(x), M, H, _p(gamma), _p(beta), float(eps), _p(u_out), _p(q),
                                         _p(scale), _stream()))
    return q, scale


def ln_f16(x, gamma, beta, eps=1e-5, y=None):
    _dev(x, torch.float16, "x")
    M, H = x.shape
    y = torch.empty((M, H), dtype=torch.float16, device=x.device) if y is None else y
    L.check("ln_f16", L.lib().ln_f16(_p(x), _ld(x), M, H, _p(gamma), _p(beta), float(eps), _p(y), _ld(y),
                                     _stream()))
    return y


def w8a8_linear(x, wq, w_scale, bias=None, residual=None, act=0, y=None, xq=None, x_scale=None, acc=None,
                prequant=False, want_y=True):
    N, K = wq.shape
    if prequant:
        M = xq.shape[0]
    else:
        _dev(x, torch.float16, "x")
        M = x.shape[0]
    dev = wq.device
    xq = torch.empty((M, K), dtype=torch.int8, device=dev) if xq is None else xq
    x_scale = torch.empty(M, dtype=torch.float32, device=dev) if x_scale is None else x_scale
    if y is None and want_y:
        y = torch.empty((M, N), dtype=torch.float16, device=dev)
    L.check("w8a8_linear", L.lib().w8a8_linear(
        _p(x), _ld(x) if x is not None else 0, M, K, _p(wq), _p(w_scale), N, _p(bias), _p(residual),
        _ld(residual) if residual is not None else 0, act, _p(y), _ld(y) if y is not None else 0, _p(xq),
        _p(x_scale), _p(acc), L.ALD_PREQUANT if prequant else 0, _stream()))
    return y


def q8w_linear(x, wq, w_scale, bias=None, residual=None, act=0, y=None):
    """fp16 x times int8 weights [N, K] with fp32 per-channel scales."""
    _dev(x, torch.float16, "x")
    M, K = x.shape
    N = wq.shape[0]
    y = torch.empty((M, N), dtype=torch.float16, device=x.device) if y is None else y
    L.check("q8w_linear", L.lib().q8w_linear(_p(x), _ld(x), M, K, _p(wq), _p(w_scale), N, _p(bias), _p(residual),
                                             _ld(residual) if residual is not None else 0, act, _p(y), _ld(y),
                                             _stream()))
    return y


def q4_linear(x, wq4, w_scale, bias=None, residual=None, act=0, y=None):
    _dev(x, torch.float16, "x")
    M, K = x.shape
    N = wq4.shape[0]
    y = torch.empty((M, N), dtype=torch.float16, device=x.device) if y is None else y
    L.check("q4_linear", L.lib().q4_linear(_p(x), _ld(x), M, K, _p(wq4), _p(w_scale), N, _p(bias), _p(residual),
                                           _ld(residual) if residual is not None else 0, act, _p(y), _ld(y),
                                           _stream()))
    return y


def f16_linear(x, w, bias=None, residual=None, act=0, y=None):
    _dev(x, torch.float16, "x")
    M, K = x.shape
    N = w.shape[0]
    y = torch.empty((M, N), dtype=torch.float16, device=x.device) if y is None else y
    L.check("f16_linear", L.lib().f16_linear(_p(x), _ld(x), M, K, _p(w), N, _p(bias), _p(residual),
                                             _ld(residual) if residual is not None else 0, act, _p(y), _ld(y),
                                             _stream()))
    return y


def attn_fwd(q, k, v, n_heads, batch, Sq=0, Sk=0, cu_seqlens_q=None, cu_seqlens_k=None, max_sq=0, max_sk=0,
             scale=0.125, out=None, head_dim=64):
    """q/k/v are 2-D token-major views [tokens, >= n_heads*64] (row strides may differ
    from the width, e.g. column slices of a fused QKV buffer)."""
    _dev(q, torch.float16, "q")
    rows = q.shape[0]
    if out is None:
        out = torch.zeros((rows, n_heads * 64), dtype=torch.float16, device=q.device)
    if k.stride(0) != v.stride(0):
        raise ValueError("k and v must share a row stride")
    L.check("attn_fwd", L.lib().attn_fwd(_p(q), _p(k), _p(v), q.stride(0), k.stride(0), n_heads, head_dim, batch,
                                         Sq, Sk, _p(cu_seqlens_q), _p(cu_seqlens_k), max_sq, max_sk, float(scale),
                                         _p(out), out.stride(0), _stream()))
    return out


def steer_add(h, alpha, resid_norm, direction, rows_per_req=1, R=1, row_req=None, mode=L.ALD_STEER_ADD):
    _dev(h, torch.float16, "h")
    M, H = h.shape
    L.check("steer_add", L.lib().steer_add(_p(h), _ld(h), M, H, rows_per_req, R, _p(row_req), _p(alpha),
                                           float(resid_norm), _p(direction), mode, _stream()))
    return h


def steer_latent(x, alpha, resid_norm, direction, rows_per_req=1, R=1, row_req=None, mode=L.ALD_STEER_ADD,
                 out=None):
    """Steered copy of the fp32 latent x [n_tok, C] (the model's input at the latent site)."""
    _dev(x, torch.float32, "x")
    n_tok, C = x.shape
    out = torch.empty_like(x) if out is None else out
    L.check("steer_latent", L.lib().steer_latent(_p(x), _p(out), n_tok, C, rows_per_req, R, _p(row_req), _p(alpha),
                                                 float(resid_norm), _p(direction), mode, _stream()))
    return out


def cfg_merge(v, w, rows_per_req=1, row_req=None, v_hat=None):
    _dev(v, torch.float16, "v")
    n2, C = v.shape
    n_tok = n2 // 2
    v_hat = torch.empty((n_tok, C), dtype=torch.float32, device=v.device) if v_hat is None else v_hat
    L.check("cfg_merge", L.lib().cfg_merge(_p(v), n_tok, C, rows_per_req, _p(row_req), _p(w), _p(v_hat),
                                           _stream()))
    return v_hat


def ddim_alpha_bar(T, beta_1, beta_T, timesteps):
    """alpha_bar of the linear-beta schedule at the grid timesteps, then 1 (host, fp32 [n + 1])."""
    ts = np.ascontiguousarray(np.asarray(timesteps, np.int32))
    out = np.empty(len(ts) + 1, np.float32)
    L.check("ddim_alpha_bar", L.lib().ddim_alpha_bar(int(T), float(beta_1), float(beta_T),
                                                     ts.ctypes.data_as(ctypes.c_void_p), len(ts),
                                                     out.ctypes.data_as(ctypes.c_void_p)))
    return out


def sampler_update(op, x, t_cur, t_next=None, v_hat=None, x0=None, eps=None, rows_per_req=1, row_req=None,
                   active=None):
    _dev(x, torch.float32, "x")
    n_tok, C = x.shape
    L.check("sampler_update", L.lib().sampler_update(op, _p(x), _p(v_hat), _p(x0), _p(eps), n_tok, C, rows_per_req,
                                                     _p(row_req), _p(t_cur), _p(t_next), _p(active), _stream()))
    return x
