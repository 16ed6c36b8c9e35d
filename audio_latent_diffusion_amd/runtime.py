"""Device-resident DiT model and step runner over the C ABI.

DiTModel uploads the fp16 weights, packs the block linears on the GPU
(per-output-channel int8 for W8A8 and W8A16, group-32 int4 for q4) and releases the
fp16 copies afterwards, so the lower precision replaces the footprint
instead of adding to it (aria, Section III-A, runtime).  StepRunner owns
the latent state, the per-step device arrays (t, steering strength,
guidance) and the workspace, enqueues dit_step, and captures the step loop
once as a hipGraph whose per-step values live in device memory (aria:
the denoising loop is captured once and replayed as one GPU graph; the
steering strength is refreshed each step without re-capture).

torch provides device memory and the stream; all arithmetic runs in
libald.so.
"""
from __future__ import annotations

import ctypes
from typing import List, Optional, Sequence

import numpy as np
import torch

from . import _lib as L
from . import binding as B


def _t(a, dtype, device):
    if isinstance(a, torch.Tensor):  # weights already drawn on a device
        return a.to(device=device, dtype=dtype).contiguous()
    return torch.from_numpy(np.ascontiguousarray(a)).to(device=device, dtype=dtype)


class DiTModel:
    """Weights of one DiT on the device, in the precision of cfg.wmode."""

    def __init__(self, cfg, params, device="cuda"):
        self.cfg = cfg
        self.device = torch.device(device)
        self.wmode = L.WMODES[cfg.wmode]
        dev = self.device
        f16, f32 = torch.float16, torch.float32
        self.keep = []  # tensors referenced by the ctypes structs
        self.w_in = _t(params.w_in, f16, dev)
        self.b_in = _t(params.b_in, f32, dev)
        self.lnf_g = _t(params.lnf_g, f32, dev)
        self.lnf_b = _t(params.lnf_b, f32, dev)
        self.w_out = _t(params.w_out, f16, dev)
        self.b_out = _t(params.b_out, f32, dev)
        self.blocks = []
        for blk in params.blocks:
            d = {}
            for nm in ("ln1_g", "ln1_b", "ln2_g", "ln2_b", "ln3_g", "ln3_b"):
                d[nm] = _t(getattr(blk, nm), f32, dev)
            for name, w16 in blk.w.items():
                wt = _t(w16, f16, dev)
                bias = _t(blk.b[name], f32, dev)
                if self.wmode in (L.ALD_W8A8, L.ALD_W8A16):
                    q, s = B.quantize_rows_q8(wt)
                    d[name] = (q, s, bias)
                elif self.wmode == L.ALD_Q4:
                    q, s = B.quantize_q4(wt)
                    d[name] = (q, s, bias)
                else:
                    d[name] = (wt, None, bias)
                del wt  # free-after-pack: the fp16 copy is released once packed
            self.blocks.append(d)
        # the blocks' text K/V linears stacked along N (per-row formats stack
        # as they are), for one-launch re-projection of a steered text
        if self.blocks:
            kvs = [d["kv"] for d in self.blocks]
            self.kv_all = tuple(None if kvs[0][i] is None else torch.cat([k[i] for k in kvs]).contiguous()
                                for i in range(3))
        else:
            self.kv_all = None
        self.stack_kv = True
        torch.cuda.synchronize(dev)
        self._build_structs()

    def _build_structs(self):
        cfg = self.cfg
        self.c_cfg = L.dit_config(cfg.n_blocks, cfg.hidden, cfg.n_heads, cfg.hidden // cfg.n_heads, cfg.mlp,
                                  cfg.channels, cfg.text_tokens, cfg.text_dim, self.wmode, cfg.steer_block,
                                  cfg.ln_eps, L.STEER_MODES[cfg.steer_mode], L.STEER_SITES[cfg.steer_site],
                                  L.SAMPLERS[cfg.sampler])
        arr = (L.dit_block_weights * max(1, cfg.n_blocks))()
        for i, d in enumerate(self.blocks):
            bw = arr[i]
            for nm in ("ln1_g", "ln1_b", "ln2_g", "ln2_b", "ln3_g", "ln3_b"):
                setattr(bw, nm, d[nm].data_ptr())
            for name in ("qkv", "o", "q", "kv", "ox", "up", "down"):
                w, s, b = d[name]
                setattr(bw, name, L.dit_linear(w.data_ptr(), None if s is None else s.data_ptr(), b.data_ptr()))
        self.c_blocks = arr
        kv_all = L.dit_linear(None, None, None)
        if self.kv_all is not None and self.stack_kv:
            w, s, b = self.kv_all
            kv_all = L.dit_linear(w.data_ptr(), None if s is None else s.data_ptr(), b.data_ptr())
        self.c_weights = L.dit_weights(ctypes.cast(arr, ctypes.POINTER(L.dit_block_weights)), self.w_in.data_ptr(),
                                       self.b_in.data_ptr(), self.lnf_g.data_ptr(), self.lnf_b.data_ptr(),
                                       self.w_out.data_ptr(), self.b_out.data_ptr(), kv_all)

    def with_steer_block(self, steer_block: int) -> "DiTModel":
        """Same weights, another steered block (-1: none)."""
        return self.with_config(steer_block=steer_block)

    def with_config(self, **kw) -> "DiTModel":
        """Same weights, other step settings (steering, sampler, grid size)."""
        other = object.__new__(DiTModel)
        other.__dict__.update(self.__dict__)
        other.cfg = self.cfg.replace(**kw)
        other._build_structs()
        return other

    def with_stacked_kv(self, on: bool) -> "DiTModel":
        """Same weights, with or without the stacked text K/V linears handed
        to the step (a text-site step then re-projects the steered text in one
        launch, or in one per block)."""
        other = object.__new__(DiTModel)
        other.__dict__.update(self.__dict__)
        other.stack_kv = bool(on)
        other._build_structs()
        return other

    def workspace_size(self, n_tok: int, R: int) -> int:
        return int(L.lib().dit_workspace_size(ctypes.byref(self.c_cfg), n_tok, R))

    def text_kv(self, text16: torch.Tensor, ws: Optional[torch.Tensor] = None) -> torch.Tensor:
        """Step-invariant text keys/values [n_blocks, rows, 2H] from text [rows, D_t]."""
        cfg = self.cfg
        text16 = text16.reshape(-1, cfg.text_dim).contiguous()
        rows = text16.shape[0]
        kv = torch.empty((max(1, cfg.n_blocks), rows, 2 * cfg.hidden), dtype=torch.float16, device=self.device)
        need = rows * cfg.text_dim + rows * 4 + 1024
        if ws is None or ws.numel() < need:
            ws = torch.empty(need, dtype=torch.uint8, device=self.device)
        L.check("dit_text_kv", L.lib().dit_text_kv(ctypes.byref(self.c_cfg), ctypes.byref(self.c_weights),
                                                   text16.data_ptr(), rows, kv.data_ptr(), ws.data_ptr(),
                                                   ws.numel(), B._stream()))
        return kv


class StepRunner:
    """Latent state and per-step device arrays for R requests.

    Dense requests (all of length `seq`) or packed varlen requests
    (`seqlens`).  Per-step arrays are [n_steps, R] so step i reads row i; the
    host may rewrite them between graph replays without re-capture.  With the
    DDIM sampler, `timesteps` (int [N], descending) gives the grid: t_grid
    then feeds only the time embedding and alpha_bar comes from the model's
    noise schedule.
    """

    def __init__(self, model: DiTModel, x0_latent: np.ndarray, text16: np.ndarray, seqlens: Sequence[int],
                 t_grid: np.ndarray, guidance: np.ndarray, alpha: np.ndarray, direction: np.ndarray,
                 resid_norm: float, start_step: Optional[np.ndarray] = None, x0: Optional[np.ndarray] = None,
                 eps: Optional[np.ndarray] = None, keep_velocity: bool = False,
                 timesteps: Optional[np.ndarray] = None):
        cfg = model.cfg
        dev = model.device
        self.model = model
        self.R = R = len(seqlens)
        self.seqlens = np.asarray(seqlens, dtype=np.int64)
        self.n_tok = int(self.seqlens.sum())
        self.dense = bool(np.all(self.seqlens == self.seqlens[0]))
        self.seq = int(self.seqlens[0]) if self.dense else 0
        self.max_seq = int(self.seqlens.max())
        N = len(t_grid) - 1
        self.n_steps = N
        f32 = torch.float32
        self.x = _t(x0_latent, f32, dev).reshape(self.n_tok, cfg.channels).contiguous()
        self.text = _t(text16, torch.float16, dev).reshape(-1, cfg.text_dim).contiguous()
        self.kv = model.text_kv(self.text)
        tg = np.asarray(t_grid, np.float32)
        self.t_cur = _t(np.repeat(tg[:-1, None], R, axis=1), f32, dev).contiguous()
        self.t_next = _t(np.repeat(tg[1:, None], R, axis=1), f32, dev).contiguous()
        self.abar_cur = self.abar_next = None
        if cfg.sampler == "ddim":
            if timesteps is None:
                raise ValueError("the DDIM sampler needs the grid timesteps")
            ab = B.ddim_alpha_bar(cfg.train_steps, cfg.beta_1, cfg.beta_T, timesteps)
            self.abar_cur = _t(np.repeat(ab[:-1, None], R, axis=1), f32, dev).contiguous()
            self.abar_next = _t(np.repeat(ab[1:, None], R, axis=1), f32, dev).contiguous()
        self.guidance = _t(np.asarray(guidance, np.float32).reshape(R), f32, dev)
        self.alpha = _t(np.asarray(alpha, np.float32).reshape(N, R), f32, dev).contiguous()
        self.direction = _t(direction, f32, dev)
        self.resid_norm = float(resid_norm)
        start = np.zeros(R, np.int64) if start_step is None else np.asarray(start_step, np.int64)
        self.start = start
        steps = np.arange(N)[:, None]
        self.active = _t((steps >= start[None, :]).astype(np.uint8), torch.uint8, dev).contiguous()
        self.renoise = None
        if x0 is not None and np.any(start > 0):
            self.renoise = _t(((steps == start[None, :]) & (start[None, :] > 0)).astype(np.uint8), torch.uint8,
                              dev).contiguous()
            self.x0 = _t(x0, f32, dev).reshape(self.n_tok, cfg.channels).contiguous()
            self.eps = _t(eps, f32, dev).reshape(self.n_tok, cfg.channels).contiguous()
        cu = np.concatenate([[0], np.cumsum(self.seqlens)]).astype(np.int32)
        self.cu = _t(cu, torch.int32, dev)
        self.row_req = _t(np.repeat(np.arange(R), self.seqlens).astype(np.int32), torch.int32, dev)
        self.ws_bytes = model.workspace_size(self.n_tok, R)
        self.ws = torch.empty(self.ws_bytes, dtype=torch.uint8, device=dev)
        self.v_out = (torch.empty((2 * self.n_tok, cfg.channels), dtype=torch.float16, device=dev)
                      if keep_velocity else None)
        self.block_norms = None
        self.graph = None
        self._graphs = []
        self._args = [self._make_args(i) for i in range(N)]

    def _make_args(self, i: int) -> L.dit_step_args:
        R = self.R
        a = L.dit_step_args()
        a.x = self.x.data_ptr()
        a.text_kv = self.kv.data_ptr()
        a.R = R
        a.seq = self.seq
        a.cu_seqlens = None if self.dense else self.cu.data_ptr()
        a.row_req = None if self.dense else self.row_req.data_ptr()
        a.n_tok = self.n_tok
        a.max_seq = self.max_seq
        a.t_cur = self.t_cur[i].data_ptr()
        a.t_next = self.t_next[i].data_ptr()
        a.guidance = self.guidance.data_ptr()
        a.alpha = self.alpha[i].data_ptr()
        a.resid_norm = self.resid_norm
        a.direction = self.direction.data_ptr()
        a.active = None if not np.any(self.start > 0) else self.active[i].data_ptr()
        a.renoise = None if self.renoise is None else self.renoise[i].data_ptr()
        a.x0 = None if self.renoise is None else self.x0.data_ptr()
        a.eps = None if self.renoise is None else self.eps.data_ptr()
        a.v_out = None if self.v_out is None else self.v_out.data_ptr()
        a.block_norms = None if self.block_norms is None else self.block_norms.data_ptr()
        a.text = self.text.data_ptr()
        a.abar_cur = None if self.abar_cur is None else self.abar_cur[i].data_ptr()
        a.abar_next = None if self.abar_next is None else self.abar_next[i].data_ptr()
        return a

    def collect_block_norms(self, enable: bool = True):
        """Per-row L2 norms of the steered block's output (steering calibration)."""
        self.block_norms = (torch.empty(2 * self.n_tok, dtype=torch.float32, device=self.x.device)
                            if enable else None)
        self._args = [self._make_args(i) for i in range(self.n_steps)]

    def step(self, i: int) -> None:
        m = self.model
        L.check("dit_step", L.lib().dit_step(ctypes.byref(m.c_cfg), ctypes.byref(m.c_weights),
                                             ctypes.byref(self._args[i]), self.ws.data_ptr(), self.ws_bytes,
                                             B._stream()))

    def capture_graph(self, steps: Sequence[int]) -> ctypes.c_void_p:
        """Capture the given steps as one hipGraph on a side stream and return
        its handle (owned by this runner, destroyed with it)."""
        steps = list(steps)
        arr = (L.dit_step_args * len(steps))(*[self._args[i] for i in steps])
        m = self.model
        handle = ctypes.c_void_p()
        s = torch.cuda.Stream(device=self.x.device)
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            L.check("dit_graph_capture", L.lib().dit_graph_capture(
                ctypes.byref(m.c_cfg), ctypes.byref(m.c_weights), arr, len(steps), self.ws.data_ptr(),
                self.ws_bytes, s.cuda_stream, ctypes.byref(handle)))
        torch.cuda.current_stream().wait_stream(s)
        self._graphs.append(handle)
        return handle

    def graph_nodes(self, handle: ctypes.c_void_p) -> int:
        """Kernel launches recorded in a captured graph."""
        n = ctypes.c_size_t()
        L.check("dit_graph_nodes", L.lib().dit_graph_nodes(handle, ctypes.byref(n)))
        return int(n.value)

    def launch_graph(self, handle: ctypes.c_void_p) -> None:
        L.check("dit_graph_launch", L.lib().dit_graph_launch(handle, B._stream()))

    def capture(self, steps: Optional[Sequence[int]] = None) -> None:
        """Capture the given steps (default all) as the runner's graph."""
        self.graph = self.capture_graph(range(self.n_steps) if steps is None else steps)

    def replay(self) -> None:
        self.launch_graph(self.graph)

    def destroy_graph(self) -> None:
        for h in self._graphs:
            if h.value:
                L.lib().dit_graph_destroy(h)
        self._graphs = []
        self.graph = None

    def __del__(self):
        try:
            self.destroy_graph()
        except Exception:
            pass
