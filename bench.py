"""Denoise-step throughput of the DiT hot path on one MI355X.

Headline workload (the serving batch): 24 DiT blocks, hidden 1536, 24 heads,
MLP 6144 (GELU), 8 requests as 16 CFG rows (cond + null-prompt companion) of
512 latent tokens x 64 channels (8192 rows per launch), cross-attention to
128 text tokens of dim 768, W8A8 block linears (per-output-channel int8
weights, per-token dynamic activation scales, int32 accumulation), fp16
attention, guidance 3, 8 Euler steps on the uniform t grid captured once as
one hipGraph, the steering node present at block 12 (strength 0 in every
step, read from device memory).  Synthetic seeded inputs; random weights of
that architecture drawn on the device.

One timed unit is one replay of the 8-step graph: the latent restarts from
its initial noise before each replay; the text K/V projection, done once per
request outside the step loop (0.7 % of a request's work), is not repeated.
`value` is denoise steps per second from the median of per-replay HIP-event
times (each replay bracketed by events on the stream it runs on), over
exactly --steps timed steps after --warmup untimed ones.

The JSON line also carries: the roofline of the dominant kernel (the W8A8
GEMM over the serving block's six launches with the step's own epilogues,
timed live with HIP events inside a graph); the GEMM alone at those shapes
against the vendor library; a steering-overhead A/B (no steering node,
strength 0 in every step, an active span); the mid-size model's loop and its
variants; the tiny model's one-step graph; per-kernel rooflines; launches per
step against the floor of an empty launch; and the CPU oracle on the host
cores (the serving step extrapolated from one of its 24 blocks).

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu]
"""
from __future__ import annotations

import argparse
import json
import os
import statistics
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

INT8_PEAK_TOPS = 5000.0      # MI355X dense int8 MFMA, TOP/s
FP16_PEAK_TFLOPS = 2500.0    # MI355X dense fp16 MFMA, TFLOP/s
HBM_PEAK_GBS = 8000.0        # MI355X HBM3E, GB/s

# the pages' end-to-end figures (RTX 3070, warm generation of a 10 s stereo
# clip with 8 sampling steps, text encoder and decoder included): context only
PAGES_CONTEXT = {
    "source": "A Quantized Native Runtime for On-Device Semantic Audio Generation (Chinese summary, results table)",
    "hardware": "RTX 3070 8 GB",
    "seconds_per_10s_clip": {"small_runtime": 0.13, "small_pytorch": 0.146, "medium_runtime": 0.37,
                             "medium_pytorch": 0.443},
    "note": "whole clips including text encoding and decoding on another GPU; not a per-step or like-for-like "
            "figure",
}


def _events_time(fn, iters, stream):
    import torch
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for _ in range(iters):
        fn()
    end.record(stream)
    end.synchronize()
    return start.elapsed_time(end) / iters  # ms


def _median(xs):
    return float(statistics.median(xs))


MIX_SHAPES = lambda H, F: [(H, 3 * H), (H, H), (H, H), (H, H), (H, F), (F, H)]  # (K, N) per block
MIX_NAMES = ("qkv", "o", "q", "ox", "up", "down")
# the epilogue each block linear runs in the step: residual add in place (o,
# ox, down), GELU (up), plain (qkv, q)
MIX_EPI = {"qkv": "plain", "o": "residual", "q": "plain", "ox": "residual", "up": "gelu", "down": "residual"}


def gemm_mix(M, H, F, epilogues=True, seed=0):
    """The W8A8 GEMM launches of one DiT block at M rows (qkv, o, q, ox, up,
    down), pre-quantized inputs, with the step's epilogues (bias everywhere,
    in-place residual for o, ox and down, GELU for up) or the plain one;
    returns one callable per launch, each enqueued through the C ABI on
    torch's current stream."""
    import torch
    from audio_latent_diffusion_amd import binding as B
    g = torch.Generator(device="cuda").manual_seed(seed)
    calls = []
    for name, (K, N) in zip(MIX_NAMES, MIX_SHAPES(H, F)):
        xq = torch.randint(-127, 128, (M, K), dtype=torch.int8, device="cuda", generator=g)
        wq = torch.randint(-127, 128, (N, K), dtype=torch.int8, device="cuda", generator=g)
        xs = torch.rand(M, device="cuda", generator=g) * 1e-2
        ws = torch.rand(N, device="cuda", generator=g) * 1e-3
        b = torch.randn(N, device="cuda", generator=g) * 0.02
        y = torch.randn((M, N), device="cuda", generator=g).half()
        epi = MIX_EPI[name] if epilogues else "plain"
        res = y if epi == "residual" else None
        act = 1 if epi == "gelu" else 0
        calls.append(lambda xq=xq, wq=wq, xs=xs, ws=ws, b=b, y=y, res=res, act=act: B.w8a8_linear(
            None, wq, ws, bias=b, residual=res, act=act, y=y, xq=xq, x_scale=xs, prequant=True))
    return calls


def _graph_of(fns, reps):
    """fns captured `reps` times into one graph on a side stream."""
    import torch
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for f in fns:
            f()
    torch.cuda.synchronize()
    gr = torch.cuda.CUDAGraph()
    with torch.cuda.graph(gr, stream=s):
        for _ in range(reps):
            for f in fns:
                f()
    gr.replay()
    torch.cuda.synchronize()
    return gr


def gemm_mix_timing(M, H, F, epilogues=True, reps=20, replays=5):
    """Per-launch times of one block's six W8A8 GEMMs at M rows, each shape
    captured `reps` times into a graph (the step runs them inside a graph;
    launched one by one from Python, short kernels would time the host) and
    timed with HIP events on the stream the graph replays on; returns
    per-shape launch times, ops and algorithmic bytes."""
    import torch
    calls = gemm_mix(M, H, F, epilogues)
    out = {}
    for name, (K, N), f in zip(MIX_NAMES, MIX_SHAPES(H, F), calls):
        gr = _graph_of([f], reps)
        ms = [_events_time(gr.replay, 1, torch.cuda.current_stream()) / reps for _ in range(replays)]
        epi = MIX_EPI[name] if epilogues else "plain"
        byts = M * K + N * K + 2 * M * N + 4 * (M + 2 * N) + (2 * M * N if epi == "residual" else 0)
        out[name] = {"M": M, "K": K, "N": N, "epilogue": epi, "us": round(_median(ms) * 1e3, 2),
                     "ops": 2.0 * M * N * K, "bytes": byts}
        del gr
    del calls
    torch.cuda.synchronize()
    return out


def mix_roofline(per_shape):
    """Algorithmic ops (and bytes) per launch over the average launch time of the mix."""
    n = len(per_shape)
    us = sum(v["us"] for v in per_shape.values()) / n
    ops = sum(v["ops"] for v in per_shape.values()) / n
    byts = sum(v["bytes"] for v in per_shape.values()) / n
    tops = ops / (us * 1e-6) / 1e12
    return {"avg_launch_us": round(us, 2), "algorithmic_ops_per_launch": ops, "algorithmic_bytes_per_launch": byts,
            "achieved": round(tops, 1), "frac": round(tops / INT8_PEAK_TOPS, 4),
            "per_shape": {k: {kk: vv for kk, vv in v.items() if kk not in ("ops", "bytes")} |
                          {"tops": round(v["ops"] / (v["us"] * 1e-6) / 1e12, 1),
                           "frac_int8_peak": round(v["ops"] / (v["us"] * 1e-6) / 1e12 / INT8_PEAK_TOPS, 4)}
                          for k, v in per_shape.items()}}


def graph_floor_us(n=200, replays=5):
    """Time per launch, inside a captured graph like the step's, of a kernel
    that does no work (zero-strength steering of one row: one workgroup reads
    the strength and exits): the floor every launch of the step pays."""
    import torch
    from audio_latent_diffusion_amd import binding as B
    h = torch.zeros((1, 64), dtype=torch.float16, device="cuda")
    a = torch.zeros(1, device="cuda")
    d = torch.zeros(64, device="cuda")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        B.steer_add(h, a, 1.0, d)
    torch.cuda.synchronize()
    gr = torch.cuda.CUDAGraph()
    with torch.cuda.graph(gr, stream=s):
        for _ in range(n):
            B.steer_add(h, a, 1.0, d)
    gr.replay()
    torch.cuda.synchronize()
    ms = _events_time(gr.replay, replays, torch.cuda.current_stream())
    del gr
    return ms * 1e3 / n


def serve_gemm(iters=20):
    """W8A8 GEMM at the serving-batch shapes (8192 tokens, hidden 1536)."""
    import torch
    from audio_latent_diffusion_amd import binding as B
    out = {}
    g = torch.Generator(device="cuda").manual_seed(1)
    total_ops, total_ms = 0.0, 0.0
    for name, (M, K, N) in {"qkv": (8192, 1536, 4608), "o": (8192, 1536, 1536), "up": (8192, 1536, 6144),
                            "down": (8192, 6144, 1536)}.items():
        xq = torch.randint(-127, 128, (M, K), dtype=torch.int8, device="cuda", generator=g)
        wq = torch.randint(-127, 128, (N, K), dtype=torch.int8, device="cuda", generator=g)
        xs = torch.rand(M, device="cuda", generator=g) * 1e-2
        ws = torch.rand(N, device="cuda", generator=g) * 1e-3
        y = torch.empty((M, N), dtype=torch.float16, device="cuda")
        fn = lambda: B.w8a8_linear(None, wq, ws, xq=xq, x_scale=xs, y=y, prequant=True)  # noqa: E731
        for _ in range(3):
            fn()
        ms = _events_time(fn, iters, torch.cuda.current_stream())
        # with the per-token quantization of an fp16 input in front (two launches)
        x = torch.randn((M, K), dtype=torch.float16, device="cuda", generator=g)
        fq = lambda: B.w8a8_linear(x, wq, ws, xq=xq, x_scale=xs, y=y)  # noqa: E731
        for _ in range(3):
            fq()
        ms_q = _events_time(fq, iters, torch.cuda.current_stream())
        # the vendor library on the same operands (hipBLASLt behind torch._int_mm:
        # int32 output, no dequantization epilogue), for comparison
        wt = wq.t()
        fv = lambda: torch._int_mm(xq, wt)  # noqa: E731
        for _ in range(3):
            fv()
        ms_v = _events_time(fv, iters, torch.cuda.current_stream())
        ops = 2.0 * M * N * K
        out[name] = {"M": M, "K": K, "N": N, "ms": round(ms, 4), "tops": round(ops / ms / 1e9, 1),
                     "frac_int8_peak": round(ops / ms / 1e9 / INT8_PEAK_TOPS, 4),
                     "quant_plus_gemm_ms": round(ms_q, 4), "vendor_int_mm_ms": round(ms_v, 4)}
        total_ops += ops
        total_ms += ms
    tops = total_ops / total_ms / 1e9
    res = {"shapes": out, "tops": round(tops, 1), "frac_int8_peak": round(tops / INT8_PEAK_TOPS, 4)}
    # a long square launch, where the fixed start and finish of a round amortize
    M = K = N = 8192
    xq = torch.randint(-127, 128, (M, K), dtype=torch.int8, device="cuda", generator=g)
    wq = torch.randint(-127, 128, (N, K), dtype=torch.int8, device="cuda", generator=g)
    xs = torch.rand(M, device="cuda", generator=g) * 1e-2
    ws = torch.rand(N, device="cuda", generator=g) * 1e-3
    y = torch.empty((M, N), dtype=torch.float16, device="cuda")
    fn = lambda: B.w8a8_linear(None, wq, ws, xq=xq, x_scale=xs, y=y, prequant=True)  # noqa: E731
    for _ in range(2):
        fn()
    ms = _events_time(fn, 5, torch.cuda.current_stream())
    ops = 2.0 * M * N * K
    res["square_8192"] = {"ms": round(ms, 4), "tops": round(ops / ms / 1e9, 1),
                          "frac_int8_peak": round(ops / ms / 1e9 / INT8_PEAK_TOPS, 4)}
    return res


def _timed(fn, iters=10):
    import torch
    for _ in range(2):
        fn()
    torch.cuda.synchronize()
    return _events_time(fn, iters, torch.cuda.current_stream())


def _entry(kind, ms, work, peak, unit, **extra):
    """One kernel's roofline: algorithmic work per launch over the launch time."""
    achieved = work / (ms / 1e3) / (1e9 if unit == "GB/s" else 1e12)
    d = {"bound": kind, "avg_launch_us": round(ms * 1e3, 2), "achieved": round(achieved, 1), "peak": peak,
         "unit": unit, "frac": round(achieved / peak, 4)}
    d.update(extra)
    return d


def kernel_rooflines():
    """Per-kernel rooflines at the large workload shapes, each kernel launched
    through the C ABI on torch's current stream and timed there with HIP
    events: flash attention (serving and 4-bit-model shapes), the fp16- and
    4-bit-weight GEMMs (serving and 4-bit-model launch mixes), and the
    HBM-bound kernels on stress shapes larger than the 256 MB last-level
    cache (same row widths as the serving model)."""
    import torch
    from audio_latent_diffusion_amd import binding as B
    from audio_latent_diffusion_amd import _lib as L
    g = torch.Generator(device="cuda").manual_seed(7)
    out = {}

    # attention: self-attention of the serving batch (16 rows x 512 tokens,
    # 24 heads), of the 4-bit model (8 rows x 1024 tokens, 32 heads) and of a
    # long-form clip on the mid-size model (a CFG pair of 8192 tokens, 16 heads)
    for name, (Bn, S, nh) in {"attn_serve": (16, 512, 24), "attn_q4": (8, 1024, 32),
                              "attn_long": (2, 8192, 16)}.items():
        qkv = torch.randn((Bn * S, 3 * nh * 64), dtype=torch.float16, device="cuda", generator=g)
        o = torch.empty((Bn * S, nh * 64), dtype=torch.float16, device="cuda")
        q, k, v = qkv[:, :nh * 64], qkv[:, nh * 64:2 * nh * 64], qkv[:, 2 * nh * 64:]
        ms = _timed(lambda: B.attn_fwd(q, k, v, nh, Bn, S, S, out=o))
        out[name] = _entry("mfma", ms, 4.0 * Bn * nh * S * S * 64, FP16_PEAK_TFLOPS, "TFLOP/s",
                           shape=f"batch {Bn} x {S} tokens x {nh} heads, head dim 64")
        del qkv, o

    # fp16-weight and 8-bit weight-only GEMMs (serving block mix), 4-bit-weight
    # GEMMs (4-bit model mix); all three run fp16 MFMAs
    for name, M, shapes, kind in (("f16_gemm_serve", 8192, MIX_SHAPES(1536, 6144), "f16"),
                                  ("q8w_gemm_serve", 8192, MIX_SHAPES(1536, 6144), "q8w"),
                                  ("q4_gemm", 8192, MIX_SHAPES(2048, 8192), "q4")):
        launches, flops = [], 0.0
        for K, N in shapes:
            x = torch.randn((M, K), dtype=torch.float16, device="cuda", generator=g)
            w = (0.02 * torch.randn((N, K), device="cuda", generator=g)).half()
            b = torch.zeros(N, device="cuda")
            y = torch.empty((M, N), dtype=torch.float16, device="cuda")
            if kind == "q4":
                p, sc = B.quantize_q4(w)
                launches.append(lambda x=x, p=p, sc=sc, b=b, y=y: B.q4_linear(x, p, sc, b, y=y))
            elif kind == "q8w":
                p, sc = B.quantize_rows_q8(w)
                launches.append(lambda x=x, p=p, sc=sc, b=b, y=y: B.q8w_linear(x, p, sc, b, y=y))
            else:
                launches.append(lambda x=x, w=w, b=b, y=y: B.f16_linear(x, w, b, y=y))
            flops += 2.0 * M * N * K

        def mix(launches=launches):
            for f in launches:
                f()
        ms = _timed(mix, 5) / len(shapes)
        out[name] = _entry("mfma", ms, flops / len(shapes), FP16_PEAK_TFLOPS, "TFLOP/s",
                           shape=f"M {M}, per-block launch mix (K, N) {shapes}")
        del launches

    # HBM-bound kernels on stress shapes
    M, H, F = 1 << 18, 1536, 6144
    x = torch.randn((M, H), dtype=torch.float16, device="cuda", generator=g)
    gam = torch.ones(H, device="cuda")
    bet = torch.zeros(H, device="cuda")
    q = torch.empty((M, H), dtype=torch.int8, device="cuda")
    s = torch.empty(M, device="cuda")
    ms = _timed(lambda: B.ln_quant(x, gam, bet, q=q, scale=s))
    out["ln_quant"] = _entry("hbm", ms, 3.0 * M * H + 4.0 * M, HBM_PEAK_GBS, "GB/s", shape=f"{M} x {H}")
    alpha = torch.full((1,), 0.5, device="cuda")
    d = torch.randn(H, device="cuda", generator=g)
    d /= d.norm()
    ms = _timed(lambda: B.steer_add(x, alpha, 1.0, d))
    out["steer_add"] = _entry("hbm", ms, 4.0 * M * H, HBM_PEAK_GBS, "GB/s", shape=f"{M} x {H}")
    beta = torch.full((1,), 1e-3, device="cuda")  # small: repeated amplification stays finite
    ms = _timed(lambda: B.steer_add(x, beta, 1.0, d, mode=L.ALD_STEER_PROJECT))
    out["steer_project"] = _entry("hbm", ms, 4.0 * M * H, HBM_PEAK_GBS, "GB/s", shape=f"{M} x {H}")
    del x, q
    Mf = M // 4
    xf = torch.randn((Mf, F), dtype=torch.float16, device="cuda", generator=g)
    qf = torch.empty((Mf, F), dtype=torch.int8, device="cuda")
    sf = torch.empty(Mf, device="cuda")
    ms = _timed(lambda: B.quantize_rows_q8(xf, q=qf, scale=sf))
    out["act_quant"] = _entry("hbm", ms, 3.0 * Mf * F + 4.0 * Mf, HBM_PEAK_GBS, "GB/s", shape=f"{Mf} x {F}")
    del xf, qf
    n_tok, C = 1 << 22, 64
    v = torch.randn((2 * n_tok, C), dtype=torch.float16, device="cuda", generator=g)
    w = torch.full((1,), 3.0, device="cuda")
    vh = torch.empty((n_tok, C), device="cuda")
    ms = _timed(lambda: B.cfg_merge(v, w, rows_per_req=n_tok, v_hat=vh))
    out["cfg_merge"] = _entry("hbm", ms, 8.0 * n_tok * C, HBM_PEAK_GBS, "GB/s", shape=f"{n_tok} x {C}")
    del v
    xs = torch.randn((n_tok, C), device="cuda", generator=g)
    tc = torch.full((1,), 1.0, device="cuda")
    tn = torch.full((1,), 0.875, device="cuda")
    ms = _timed(lambda: B.sampler_update(L.ALD_EULER, xs, tc, tn, v_hat=vh, rows_per_req=n_tok))
    out["sampler_euler"] = _entry("hbm", ms, 12.0 * n_tok * C, HBM_PEAK_GBS, "GB/s", shape=f"{n_tok} x {C}")
    ab = torch.full((1,), 0.3, device="cuda")
    abn = torch.full((1,), 0.35, device="cuda")
    vh.normal_(generator=g)
    ms = _timed(lambda: B.sampler_update(L.ALD_DDIM, xs, ab, abn, v_hat=vh, rows_per_req=n_tok))
    out["sampler_ddim"] = _entry("hbm", ms, 12.0 * n_tok * C, HBM_PEAK_GBS, "GB/s", shape=f"{n_tok} x {C}")
    # latent-site steering: a steered fp32 copy of the latent (4 B read + 4 B written per value)
    dl = torch.randn(C, device="cuda", generator=g)
    dl /= dl.norm()
    xl = torch.empty_like(xs)
    ms = _timed(lambda: B.steer_latent(xs, alpha, 1.0, dl, rows_per_req=n_tok, out=xl))
    out["steer_latent"] = _entry("hbm", ms, 8.0 * n_tok * C, HBM_PEAK_GBS, "GB/s", shape=f"{n_tok} x {C}")
    del xs, vh, xl
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return out


def device_params(cfg, seed):
    """Random weights of cfg's architecture, drawn on the GPU with a seeded
    generator (the same distributions as the seeded host draws: weights
    N(0, 0.02) in fp16, biases N(0, 0.02), LayerNorm gain 1 + N(0, 0.02) and
    shift N(0, 0.02)); for timing runs of the large models, whose host draws
    would take minutes."""
    import torch
    import ald_inputs as I
    g = torch.Generator(device="cuda").manual_seed(seed)
    H, C = cfg.hidden, cfg.channels

    def nrm(shape, s=0.02):
        return torch.randn(shape, generator=g, device="cuda") * s

    def ln():
        return 1.0 + nrm(H), nrm(H)

    shapes = I.linear_shapes(cfg)
    blocks = []
    for _ in range(cfg.n_blocks):
        (g1, b1), (g2, b2), (g3, b3) = ln(), ln(), ln()
        w = {n: nrm(shapes[n]).half() for n in I.LINEARS}
        b = {n: nrm(shapes[n][0]) for n in I.LINEARS}
        blocks.append(I.BlockParams(g1, b1, g2, b2, g3, b3, w, b))
    lg, lb = ln()
    return I.DiTParams(nrm((H, C)).half(), nrm(H), lg, lb, nrm((C, H)).half(), nrm(C), blocks)


class Loop:
    """A step runner whose whole sampler loop is captured once as one graph
    (plus, when a step count needs one, a graph of the loop's first k steps);
    each replay restarts the latent from its initial noise."""

    def __init__(self, model, inp, resid):
        from audio_latent_diffusion_amd import runtime
        self.run = runtime.StepRunner(model, inp.x, inp.text, inp.seqlens, inp.t_grid, inp.guidance, inp.alpha,
                                      inp.direction, resid, start_step=inp.start_step, x0=inp.x0, eps=inp.eps,
                                      timesteps=inp.timesteps)
        self.n = self.run.n_steps
        self.x_init = self.run.x.clone()
        self.graphs = {self.n: self.run.capture_graph(range(self.n))}

    def schedule(self, steps):
        """Replays (each a step count) that add up to exactly `steps` steps."""
        sched = [self.n] * (steps // self.n)
        if steps % self.n:
            sched.append(steps % self.n)
        for k in sched:
            if k not in self.graphs:
                self.graphs[k] = self.run.capture_graph(range(k))
        return sched

    def replay(self, k, stream, ev=None):
        self.run.x.copy_(self.x_init)
        if ev is not None:
            ev[0].record(stream)
        self.run.launch_graph(self.graphs[k])
        if ev is not None:
            ev[1].record(stream)

    def event_times(self, sched):
        """ms per step of each replay, from HIP events around the graph launch."""
        import torch
        stream = torch.cuda.current_stream()
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in sched]
        for k, ev in zip(sched, evs):
            self.replay(k, stream, ev)
        torch.cuda.synchronize()
        return [ev[0].elapsed_time(ev[1]) / k for k, ev in zip(sched, evs)]

    def timed(self, steps, warmup):
        """Exactly `steps` timed steps after `warmup` untimed ones: median of
        the per-replay event times, and the wall clock around them with a
        device synchronisation on both sides."""
        import torch
        stream = torch.cuda.current_stream()
        warm, sched = self.schedule(warmup), self.schedule(steps)
        for k in warm:
            self.replay(k, stream)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        per_step = self.event_times(sched)
        wall = time.perf_counter() - t0
        med = _median(per_step)
        ok = bool(torch.isfinite(self.run.x).all().item())
        return {"steps": steps, "replays": len(sched), "median_ms_per_step": round(med, 4),
                "steps_per_s": round(1e3 / med, 2), "wall_steps_per_s": round(steps / wall, 2),
                "min_ms_per_step": round(min(per_step), 4), "max_ms_per_step": round(max(per_step), 4),
                "finite": ok}

    def launches_per_step(self):
        return self.run.graph_nodes(self.graphs[self.n]) / self.n

    def close(self):
        self.run.destroy_graph()


def steering_ab(model, inp, resid, span_alpha, span_steps, replays):
    """The same loop three ways, replays interleaved so that drift in the
    chip's clock falls on all three alike: no steering node (steer_block -1),
    the node with strength 0 in every step, and strength `span_alpha` in
    `span_steps` (the node reads the strength from device memory at run
    time).  Median ms per step of each, and the differences."""
    import dataclasses
    zero = np.zeros_like(inp.alpha)
    span = np.zeros_like(inp.alpha)
    span[list(span_steps), :] = span_alpha
    arms = {"no_node": Loop(model.with_steer_block(-1), dataclasses.replace(inp, alpha=zero), resid),
            "alpha_zero": Loop(model, dataclasses.replace(inp, alpha=zero), resid),
            "active_span": Loop(model, dataclasses.replace(inp, alpha=span), resid)}
    times = {k: [] for k in arms}
    for loop in arms.values():
        loop.event_times([loop.n])
    for _ in range(replays):
        for k, loop in arms.items():
            times[k] += loop.event_times([loop.n])
    out = {k: round(_median(v), 4) for k, v in times.items()}
    base = out["no_node"]
    res = {"median_ms_per_step": out,
           "steps_per_s": {k: round(1e3 / v, 2) for k, v in out.items()},
           "overhead_vs_no_node_pct": {k: round(100.0 * (v - base) / base, 2) for k, v in out.items()
                                       if k != "no_node"},
           "launches_per_step": {k: loop.launches_per_step() for k, loop in arms.items()},
           "replays_each": replays, "span": {"alpha": span_alpha, "steps": list(span_steps)}}
    for loop in arms.values():
        loop.close()
    return res


def loop_rate(model, inp, resid, replays):
    """steps/s of whole replays of the run's full sampler loop as one graph
    (median of the per-replay event times)."""
    loop = Loop(model, inp, resid)
    r = loop.timed(replays * loop.n, loop.n)
    r["launches_per_step"] = loop.launches_per_step()
    loop.close()
    return r


def mixed_warm_start(resid, replays=5):
    """The warm-start serving batch: 32 packed requests of 128..1024 latent
    tokens on the mid-size architecture, half of them warm-started (re-noised
    at a skipped step), 16 Euler steps as one graph; request-steps/s and
    token-steps/s over the rows each step actually advances."""
    import ald_inputs as I
    from audio_latent_diffusion_amd import runtime
    cfg = I.MIXED
    inp = I.make_mixed_inputs(cfg)
    model = runtime.DiTModel(cfg, I.make_params(cfg))
    r = loop_rate(model, inp, resid, replays)
    active = cfg.n_steps - np.asarray(inp.start_step)
    req_steps = int(active.sum())
    tok_steps = int((np.asarray(inp.seqlens) * active).sum())
    sec = r["median_ms_per_step"] * cfg.n_steps / 1e3
    del model
    return {"workload": f"{len(inp.seqlens)} packed requests, latent lengths 128..1024 (total "
                        f"{int(np.sum(inp.seqlens))} tokens), half warm-started, {cfg.n_steps} Euler steps as one "
                        f"hipGraph, W8A8", "request_steps_per_s": round(req_steps / sec, 1),
            "token_steps_per_s": round(tok_steps / sec), "active_request_steps": req_steps,
            "ms_per_loop": round(sec * 1e3, 2), "replays": r["replays"], "finite": r["finite"]}


def variant_loops(model, resid):
    """The mid-size model's loop under other settings: the DDIM sampler over
    the 200-step grid (the warm-start pages' backbone setting, steering in
    steps 40-79), and steering at the latent and text sites (8 Euler steps;
    the text site re-projects the steered text's K/V in every step)."""
    import ald_inputs as I
    out = {}
    cfg = I.MID_DDIM
    r = loop_rate(model.with_config(sampler="ddim", n_steps=cfg.n_steps), I.make_inputs(cfg), resid, 3)
    out["ddim_200"] = dict(workload="DDIM sampler, 200 steps as one hipGraph, steering alpha 0.5 at block 12 "
                                    "in steps 40-79", **r)
    for site in ("latent", "text"):
        cfg = I.MID.replace(steer_site=site)
        inp = I.make_inputs(cfg)
        unit = float(np.mean(np.linalg.norm(inp.x, axis=1))) if site == "latent" else \
            float(np.mean(np.linalg.norm(inp.text[:cfg.requests].reshape(-1, cfg.text_dim).astype(np.float64), axis=1)))
        r = loop_rate(model.with_config(steer_site=site), inp, unit, 30)
        out[f"steer_{site}_site"] = dict(workload=f"8 Euler steps as one hipGraph, steering alpha 0.5 at the "
                                                  f"{site} site in steps 2-5", **r)
    return out


def other_arms(params, inp, replays=5):
    """The serving model with fp16 and 8-bit weight-only weights on the same
    inputs as the W8A8 headline, and the 4-bit-weight model (24 blocks,
    hidden 2048, 4 requests as 8 CFG rows of 1024 tokens); 8 Euler steps as
    one graph each, and the six block linears' algorithmic work times the
    rate."""
    import torch
    import ald_inputs as I
    from audio_latent_diffusion_amd import runtime
    out = {}

    def lin_ops(cfg):
        tokens = 2 * cfg.requests * cfg.seq
        return 2.0 * tokens * sum(n * k for name, (n, k) in I.linear_shapes(cfg).items() if name != "kv") * \
            cfg.n_blocks

    for arm in ("f16", "w8a16"):
        cfg = I.SERVE.replace(wmode=arm)
        model = runtime.DiTModel(cfg, params)
        r = loop_rate(model, inp, 1.0, replays)
        out[f"serve_{arm}"] = dict(workload=f"serving model, {arm} weights, 8 Euler steps as one hipGraph",
                                   linear_ops_per_step=lin_ops(cfg),
                                   linear_tflops=round(lin_ops(cfg) * r["steps_per_s"] / 1e12, 1), **r)
        del model
        torch.cuda.empty_cache()
    cfg = I.Q4
    qp = device_params(cfg, cfg.seed)
    model = runtime.DiTModel(cfg, qp)
    del qp
    torch.cuda.empty_cache()
    r = loop_rate(model, I.make_inputs(cfg), 1.0, replays)
    out["q4_model"] = dict(workload="24 blocks, hidden 2048, 4 requests x CFG pair of 1024 latent tokens (8192 "
                                    "rows), 4-bit weights (group 32), 8 Euler steps as one hipGraph",
                           linear_ops_per_step=lin_ops(cfg),
                           linear_tflops=round(lin_ops(cfg) * r["steps_per_s"] / 1e12, 1), **r)
    del model
    torch.cuda.empty_cache()
    return out


def _source_hash(path):
    import hashlib
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def _oracle_threads():
    try:
        from threadpoolctl import threadpool_info
        return max([d.get("num_threads", 1) for d in threadpool_info()] or [1])
    except Exception:
        return None


def _oracle_step_seconds(cfg, inp=None, steps=(0,)):
    """Wall seconds of the oracle's step(s) on cfg's model (text K/V and
    weight packing excluded)."""
    import ald_inputs as I
    from oracle import ald_oracle as O
    om = O.prepare_model(cfg, I.make_params(cfg))
    inp = I.make_inputs(cfg) if inp is None else inp
    kv = O.text_kv(om, inp.text)
    t0 = time.perf_counter()
    O.run_sampler(om, inp, kv, resid_norm=1.0, steps=list(steps))
    return time.perf_counter() - t0


def cpu_baseline():
    """The oracle as it stands (fp64 numpy, BLAS matmuls) on the host cores.

    value: the headline workload, extrapolated -- one step of the serving
    model cut to one of its 24 blocks over the full batch (8 requests, 8192
    CFG rows), times 24 (the input and output projections, CFG merge and
    Euler update, under 1 % of the work, are counted 24 times).  Beside it:
    the 4-bit-weight model the same way, a full step of the mid-size model,
    the tiny model on all threads and on one, and one global step of a
    4-request packed sub-batch of the mixed warm-start workload (lengths 128,
    129, 577, 1024; two cold, two warm, one re-noised in that step)."""
    import ald_inputs as I
    cores = len(os.sched_getaffinity(0))
    legs = {}
    t_serve = _oracle_step_seconds(I.SERVE.replace(n_blocks=1, steer_block=0))
    legs["q4_model_x24"] = {"seconds_one_block": round((t4 := _oracle_step_seconds(
        I.Q4.replace(n_blocks=1, steer_block=0))), 2), "steps_per_s": round(1.0 / (24 * t4), 5),
        "extrapolated": True}
    t_mid = _oracle_step_seconds(I.MID, steps=(2,))
    legs["mid_step"] = {"seconds": round(t_mid, 2), "steps_per_s": round(1.0 / t_mid, 4)}
    legs["tiny_step"] = tiny_oracle_rates()
    cfg = I.MIXED
    sub = I.make_mixed_inputs(cfg, seqlens=np.array([128, 129, 577, 1024]),
                              warm=np.array([False, False, True, True]))
    sub.start_step = np.array([0, 0, 5, 7])
    t_mix = _oracle_step_seconds(cfg, sub, steps=(7,))
    legs["mixed_subbatch_step"] = {"seconds": round(t_mix, 2), "request_steps_per_s": round(4 / t_mix, 4),
                                   "token_steps_per_s": round(int(np.sum(sub.seqlens)) / t_mix, 1)}
    return {"value": round(1.0 / (24 * t_serve), 5), "unit": "steps/s", "cores": cores, "kind": "oracle",
            "sample": f"one step of the serving model cut to 1 of its 24 blocks (8 requests, 8192 CFG rows, "
                      f"W8A8) took {t_serve:.1f} s; value = 1 / (24 x that), an extrapolation to the full "
                      f"24-block step",
            "blas_threads": _oracle_threads(), "seconds_one_block": round(t_serve, 2), "extrapolated": True,
            "legs": legs}


def tiny_oracle_rates(reps=3):
    """The oracle on one step of the tiny DiT (2 blocks, hidden 256, a CFG pair
    of 64 latent tokens), on all host threads and on one: steps/s each."""
    import ald_inputs as I
    from oracle import ald_oracle as O
    cfg = I.TINY
    params = I.make_params(cfg)
    inp = I.make_inputs(cfg)
    om = O.prepare_model(cfg, params)
    kv = O.text_kv(om, inp.text)

    def rate():
        t0 = time.perf_counter()
        for _ in range(reps):
            O.dit_step(om, inp.x, inp.seqlens, kv, np.full(1, inp.t_grid[0], np.float32),
                       np.full(1, inp.t_grid[1], np.float32), inp.guidance, inp.alpha[0], 5.0, inp.direction)
        return round(reps / (time.perf_counter() - t0), 2)

    res = {"all_threads_steps_per_s": rate()}
    try:
        from threadpoolctl import threadpool_limits
        with threadpool_limits(limits=1):
            res["one_thread_steps_per_s"] = rate()
    except Exception:
        res["one_thread_steps_per_s"] = None
    return res


GEMM_SOURCE = os.path.join(ROOT, "audio_latent_diffusion_amd", "csrc", "gemm_dma.hip")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "gemm_w8a8_serve_mix_traffic.txt")


def measured_traffic():
    """HBM bytes per GEMM launch from the committed rocprofv3 counter summary
    (FETCH_SIZE and WRITE_SIZE of the serving launch mix, each scaled by what
    the same counter reads for a plain copy of known size); None when the
    file is missing or the kernel source changed since the counters were
    taken."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    vals = {}
    with open(TRAFFIC_FILE) as f:
        for ln in f:
            parts = ln.split()
            if len(parts) == 2 and not ln.startswith("#"):
                vals[parts[0]] = parts[1]
    try:
        if vals["source_sha256"] != _source_hash(GEMM_SOURCE):
            return None
        copy_bytes = float(vals["copy_bytes"])
        fetch_factor = float(vals["copy_fetch_kib_per_dispatch"]) * 1024.0 / copy_bytes
        write_factor = float(vals["copy_write_kib_per_dispatch"]) * 1024.0 / copy_bytes
        return (float(vals["gemm_fetch_kib_per_dispatch"]) * 1024.0 / fetch_factor +
                float(vals["gemm_write_kib_per_dispatch"]) * 1024.0 / write_factor)
    except (KeyError, ValueError, ZeroDivisionError):
        return None


def counter_legs(legs, reps):
    """Workloads for the rocprofv3 runs: the headline loop (two replays),
    the serving block's W8A8 GEMM mix
    with the step's epilogues (the roofline's kernel), the same mix at the
    mid-size model's 512 rows, the plain-epilogue serving GEMMs, the
    per-kernel legs, and a plain device copy of known size that calibrates
    FETCH_SIZE / WRITE_SIZE."""
    import torch
    if "serve_step" in legs:
        # the headline loop itself: two replays of the serving W8A8 8-step graph
        import ald_inputs as I
        from audio_latent_diffusion_amd import runtime
        cfg = I.SERVE
        params = device_params(cfg, cfg.seed)
        model = runtime.DiTModel(cfg, params)
        del params
        loop = Loop(model, I.make_inputs(cfg), 1.0)
        loop.timed(2 * loop.n, loop.n)
        loop.close()
        del model
        torch.cuda.empty_cache()
    if "serve_mix" in legs:
        for f in gemm_mix(8192, 1536, 6144):
            for _ in range(reps):
                f()
    if "mid_mix" in legs:
        for f in gemm_mix(512, 1024, 4096):
            for _ in range(reps):
                f()
    if "serve" in legs:
        print(json.dumps({"w8a8_gemm_serve": serve_gemm(iters=reps)}))
    if "kernels" in legs:
        kernel_rooflines()
    if "copy" in legs:
        # an elementwise kernel that reads one buffer and writes another, both
        # larger than the 256 MB last-level cache
        n = 256 << 20  # 256 Mi fp32 = 1 GiB each way
        a = torch.ones(n, dtype=torch.float32, device="cuda")
        b = torch.empty_like(a)
        for _ in range(reps):
            torch.mul(a, 1.0, out=b)
        print(f"copy leg: {n * 4} bytes read and written per dispatch")
    torch.cuda.synchronize()


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=400, help="timed denoise steps (8 per replay)")
    ap.add_argument("--warmup", type=int, default=80, help="untimed denoise steps")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--leg", default="", help="profiling legs only (serve_step,serve_mix,mid_mix,serve,kernels,"
                                              "copy) for rocprofv3 runs")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on one GPU only; --gpus N > 1 is not supported. The step shards by request "
              "(each GPU would hold the weights and run its own requests' CFG pairs with no per-step "
              "exchange), and no multi-GPU path is built.", file=sys.stderr)
        sys.exit(2)
    if args.steps < 1 or args.warmup < 0:
        print("--steps must be at least 1 and --warmup at least 0", file=sys.stderr)
        sys.exit(2)
    if args.leg == "serve_loop":  # the headline loop's timing alone (for A/B runs of two builds)
        import ald_inputs as I
        from audio_latent_diffusion_amd import runtime
        cfg = I.SERVE
        params = device_params(cfg, cfg.seed)
        model = runtime.DiTModel(cfg, params)
        del params
        loop = Loop(model, I.make_inputs(cfg), 1.0)
        print(json.dumps(loop.timed(args.steps, args.warmup)))
        loop.close()
        return
    if args.leg:
        counter_legs(args.leg.split(","), 20)
        return

    import torch
    import ald_inputs as I
    from audio_latent_diffusion_amd import runtime

    def log(msg):
        print(f"[bench] {msg}", file=sys.stderr, flush=True)

    # ---- headline: the serving batch, W8A8, 8 steps as one graph ----
    cfg = I.SERVE
    params = device_params(cfg, cfg.seed)
    inp = I.make_inputs(cfg)
    model = runtime.DiTModel(cfg, params)
    loop = Loop(model, inp, 1.0)  # strength 0 in every step: the steering unit is never used
    head = loop.timed(args.steps, args.warmup)
    launches = loop.launches_per_step()
    loop.close()
    log(f"serving W8A8 step: {head['steps_per_s']} steps/s (median of {head['replays']} replays)")
    steer_serve = steering_ab(model, inp, 62.0, 0.5, (2, 3, 4, 5), 5)
    log("serving steering A/B done")
    del model
    torch.cuda.empty_cache()
    arms = other_arms(params, inp)
    del params
    torch.cuda.empty_cache()
    log("serving fp16 / 8-bit weight-only arms and the 4-bit model done")

    # ---- the W8A8 GEMM: the serving block's launch mix with its epilogues ----
    serve_mix = mix_roofline(gemm_mix_timing(8192, 1536, 6144, epilogues=True))
    traffic = measured_traffic()
    serve_plain = serve_gemm()
    floor_us = graph_floor_us()
    log(f"serving GEMM mix: {serve_mix['frac']} of the int8 peak")

    # ---- mid-size model (16 blocks, hidden 1024, one CFG pair of 256 tokens) ----
    mcfg = I.MID
    mparams = I.make_params(mcfg)
    minp = I.make_inputs(mcfg)
    mmodel = runtime.DiTModel(mcfg, mparams)
    zero = I.make_inputs(mcfg)
    zero.alpha[:] = 0
    cal = runtime.StepRunner(mmodel, zero.x, zero.text, zero.seqlens, zero.t_grid, zero.guidance, zero.alpha,
                             zero.direction, 0.0)
    cal.collect_block_norms()
    norms = []
    for i in range(mcfg.n_steps):
        cal.step(i)
        norms.append(cal.block_norms.double().mean().item())
    resid = float(np.mean(norms))  # steering unit: mean token norm of block 12's output, unsteered run
    del cal
    mloop = Loop(mmodel, minp, resid)
    mid = mloop.timed(50 * mloop.n, 10 * mloop.n)
    mid["launches_per_step"] = mloop.launches_per_step()
    mid["us_per_launch"] = round(mid["median_ms_per_step"] * 1e3 / mid["launches_per_step"], 2)
    mid["graph_noop_launch_us"] = round(floor_us, 2)
    mloop.close()
    mid["steering_ab"] = steering_ab(mmodel, minp, resid, mcfg.steer_alpha, mcfg.steer_steps, 30)
    mid["gemm_mix_m512"] = mix_roofline(gemm_mix_timing(512, 1024, 4096, epilogues=True))
    variants = variant_loops(mmodel, resid)
    variants["warm_start_mixed"] = mixed_warm_start(resid)
    del mmodel
    torch.cuda.empty_cache()
    log("mid-size loops done")

    # ---- tiny model: one step as its own graph ----
    tcfg = I.TINY.replace(n_steps=1)
    tmodel = runtime.DiTModel(tcfg, I.make_params(tcfg))
    tiny = loop_rate(tmodel, I.make_inputs(tcfg), 5.0, 200)
    del tmodel

    kernels = kernel_rooflines()
    log("per-kernel legs done")

    # the serving step's algorithmic work: int8 GEMM ops of the six block
    # linears (the text K/V projection is hoisted) and attention flops
    M, H, F, S, T, nh = cfg.tokens, cfg.hidden, cfg.mlp, cfg.seq, cfg.text_tokens, cfg.n_heads
    int8_ops = cfg.n_blocks * sum(2.0 * M * N * K for K, N in MIX_SHAPES(H, F))
    attn_flops = cfg.n_blocks * cfg.cfg_rows * nh * 4.0 * 64 * (S * S + S * T)
    step_s = head["median_ms_per_step"] / 1e3
    gemm_block_us = sum(v["us"] for v in serve_mix["per_shape"].values())
    line = {
        "metric": "DiT denoise steps/s (CFG batch) + W8A8 GEMM % of int8 MFMA peak on 1 GPU",
        "value": head["steps_per_s"],
        "unit": "steps/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["median_ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8",
        "data": "synthetic",
        "config": {"workload": "serving batch: 24-block DiT, hidden 1536, 24 heads, MLP 6144, 8 requests x CFG "
                               "pair = 16 rows x 512 latent tokens x 64 channels (8192 rows), text 128 x 768, W8A8 "
                               "block linears, fp16 attention, 8 Euler steps as one hipGraph, steering node at "
                               "block 12 with strength 0",
                   "global_batch": cfg.cfg_rows, "seq_len": cfg.seq, "parallelism": "none",
                   "denoise_steps_per_replay": cfg.n_steps, "attention_dtype": "fp16",
                   "timing": "median of per-replay HIP-event times; each replay restarts the latent from its "
                             "noise and reuses the request's text K/V (projected once per request, 0.7 % of its "
                             "work)"},
        "wall_steps_per_s": head["wall_steps_per_s"],
        "timing": head,
        "launches_per_step": launches,
        "roofline": {"bound": "mfma", "kernel": "W8A8 GEMM (int8 MFMA): the serving block's six launches "
                                                "(M 8192; qkv, o, q, ox, up, down) with the step's epilogues",
                     "achieved": serve_mix["achieved"], "peak": INT8_PEAK_TOPS, "unit": "TOP/s",
                     "frac": serve_mix["frac"], "traffic": None if traffic is None else round(traffic),
                     "avg_launch_us": serve_mix["avg_launch_us"],
                     "algorithmic_ops_per_launch": serve_mix["algorithmic_ops_per_launch"],
                     "algorithmic_bytes_per_launch": serve_mix["algorithmic_bytes_per_launch"],
                     "per_shape": serve_mix["per_shape"]},
        "step_rates": {"int8_gemm_tops": round(int8_ops / step_s / 1e12, 1),
                       "attention_tflops": round(attn_flops / step_s / 1e12, 2),
                       "int8_gemm_ops_per_step": int8_ops, "attention_flops_per_step": attn_flops,
                       "gemm_share_of_step": round(cfg.n_blocks * gemm_block_us * 1e-6 / step_s, 3)},
        "steering_ab": steer_serve,
        "w8a8_gemm_serve": serve_plain,
        "mid_model": dict(workload="mid-size DiT, 16 blocks, hidden 1024, 16 heads, MLP 4096, one CFG pair of 256 "
                                   "latent tokens (512 rows), text 128 x 768, W8A8, 8 Euler steps as one hipGraph, "
                                   "steering alpha 0.5 at block 12 in steps 2-5", **mid),
        "tiny_one_step_graph": dict(workload="tiny DiT, 2 blocks, hidden 256, one CFG pair of 64 latent tokens, "
                                             "W8A8, one step as its own hipGraph", **tiny),
        "loop_variants": {**variants, **arms},
        "kernels": kernels,
        "context_pages": PAGES_CONTEXT,
    }
    if not args.no_cpu:
        line["cpu_baseline"] = cpu_baseline()
        log("CPU oracle done")
    print(json.dumps(line))


if __name__ == "__main__":
    main()
