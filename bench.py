"""Denoise-step throughput of the DiT hot path on one MI355X.

Workload (mid-size DiT): 16 blocks, hidden 1024, 16 heads, MLP 4096 (GELU),
latent 256 x 64, cross-attention to 128 text tokens of dim 768, one request
as a CFG pair (batch 2, guidance 3), W8A8 weights with per-token dynamic
activation scales, 8 Euler steps on the uniform t grid captured once as one
hipGraph, steering (alpha 0.5 at block 12) active in steps 2-5 only.
Synthetic seeded inputs and random weights of that shape.

One timed unit is one replay of the 8-step graph (a whole sampler pass of a
fresh request: the latent is reset from its initial noise first); `value` is
denoise steps per second.  The JSON line also carries the roofline of the
dominant kernel (the W8A8 GEMM, timed live with HIP events on its own launch
stream at the step's shapes), the W8A8 GEMM at the serving-batch shapes
(hidden 1536, 8192 tokens) as % of the int8 MFMA peak, per-kernel rooflines
(attention, fp16- and 4-bit-weight GEMMs at the large workload shapes; the
HBM-bound kernels on stress shapes beyond the last-level cache), and the CPU
oracle timed on a bounded sample on the host cores.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

INT8_PEAK_TOPS = 5000.0      # MI355X dense int8 MFMA, TOP/s
FP16_PEAK_TFLOPS = 2500.0    # MI355X dense fp16 MFMA, TFLOP/s
HBM_PEAK_GBS = 8000.0        # MI355X HBM3E, GB/s


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


MIX_SHAPES = lambda H, F: [(H, 3 * H), (H, H), (H, H), (H, H), (H, F), (F, H)]  # (K, N) per block


def gemm_mix(cfg):
    """The W8A8 GEMM launches of one DiT block at M = 2 R S tokens (qkv, o, q,
    ox, up, down), pre-quantized inputs, each launched through the C ABI on
    torch's current stream; returns a callable that enqueues the six."""
    import torch
    from audio_latent_diffusion_amd import binding as B
    M = cfg.tokens
    g = torch.Generator(device="cuda").manual_seed(0)
    bufs = []
    for K, N in MIX_SHAPES(cfg.hidden, cfg.mlp):
        xq = torch.randint(-127, 128, (M, K), dtype=torch.int8, device="cuda", generator=g)
        wq = torch.randint(-127, 128, (N, K), dtype=torch.int8, device="cuda", generator=g)
        xs = torch.rand(M, device="cuda", generator=g) * 1e-2
        ws = torch.rand(N, device="cuda", generator=g) * 1e-3
        y = torch.empty((M, N), dtype=torch.float16, device="cuda")
        bufs.append((xq, wq, xs, ws, y))

    def run_mix():
        for xq, wq, xs, ws, y in bufs:
            B.w8a8_linear(None, wq, ws, xq=xq, x_scale=xs, y=y, prequant=True)
    return run_mix


def gemm_mix_timing(cfg, iters=50, replays=5):
    """Average launch time of the W8A8 GEMM over the step's per-block launch
    mix, with the algorithmic ops and bytes per launch.  The launches are
    captured into a graph, as the step runs them (launched one by one from
    Python, these short kernels would time the host instead), and the graph's
    replays are timed with HIP events on torch's current stream, the stream
    they run on."""
    import torch
    run_mix = gemm_mix(cfg)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        run_mix()
    torch.cuda.synchronize()
    gr = torch.cuda.CUDAGraph()
    with torch.cuda.graph(gr, stream=s):
        for _ in range(iters):
            run_mix()
    gr.replay()
    torch.cuda.synchronize()
    ms_mix = _events_time(gr.replay, replays, torch.cuda.current_stream()) / iters
    del gr
    M = cfg.tokens
    shapes = MIX_SHAPES(cfg.hidden, cfg.mlp)
    ops = sum(2.0 * M * N * K for K, N in shapes)
    byts = sum(M * K + N * K + 2 * M * N + 4 * (M + N) for K, N in shapes)
    return ms_mix / len(shapes), ops / len(shapes), byts / len(shapes)


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


def cpu_baseline(cfg, params, inp, resid, budget_s=20.0):
    """The oracle, as it stands, on the host cores: denoise steps of the same
    workload, as many whole steps as fit the budget (at least one)."""
    from oracle import ald_oracle as O
    try:
        from threadpoolctl import threadpool_info
        threads = max([d.get("num_threads", 1) for d in threadpool_info()] or [1])
    except Exception:
        threads = len(os.sched_getaffinity(0))
    om = O.prepare_model(cfg, params)
    kv = O.text_kv(om, inp.text)
    x = inp.x
    t0 = time.perf_counter()
    n = 0
    while True:
        i = n % cfg.n_steps
        x, _ = O.dit_step(om, x, inp.seqlens, kv, np.full(1, inp.t_grid[i], np.float32),
                          np.full(1, inp.t_grid[i + 1], np.float32), inp.guidance, inp.alpha[i], resid,
                          inp.direction)
        n += 1
        if time.perf_counter() - t0 >= budget_s or n >= cfg.n_steps:
            break
    dt = time.perf_counter() - t0
    out = {"value": round(n / dt, 4), "unit": "steps/s", "cores": int(threads), "kind": "oracle",
           "sample": f"{n} denoise step(s) of the mid-size DiT (same shapes, CFG pair) in {dt:.1f} s; "
                     f"fp64 numpy oracle with BLAS matmuls, text K/V and weight packing excluded"}
    out["tiny_step"] = tiny_oracle_rates()
    return out


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
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "gemm_w8a8_mid_launch_mix_traffic.txt")


def _source_hash(path):
    import hashlib
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def measured_traffic():
    """HBM bytes per GEMM launch from the committed rocprofv3 counter summary
    (FETCH_SIZE and WRITE_SIZE of the launch-mix leg, each scaled by what the
    same counter reads for a plain copy of known size); None when the file is
    missing or the kernel source changed since the counters were taken."""
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
    """Workloads for the rocprofv3 --pmc runs: the GEMM launch mix of the
    step (same shapes and stream as the roofline timing), the W8A8 GEMMs at
    the serving shapes, and a plain device copy of known size that
    calibrates FETCH_SIZE / WRITE_SIZE."""
    import torch
    import ald_inputs as I
    if "gemm" in legs:
        run_mix = gemm_mix(I.MID)
        for _ in range(reps):
            run_mix()
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


def loop_rate(model, inp, resid, replays):
    """steps/s of whole replays of the run's full sampler loop as one graph."""
    import torch
    from audio_latent_diffusion_amd import runtime
    run = runtime.StepRunner(model, inp.x, inp.text, inp.seqlens, inp.t_grid, inp.guidance, inp.alpha,
                             inp.direction, resid, timesteps=inp.timesteps)
    n = run.n_steps
    x_init = run.x.clone()
    graph = run.capture_graph(range(n))
    run.x.copy_(x_init)
    run.launch_graph(graph)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(replays):
        run.x.copy_(x_init)
        run.launch_graph(graph)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ok = bool(torch.isfinite(run.x).all().item())
    run.destroy_graph()
    return {"steps_per_s": round(replays * n / wall, 2), "ms_per_loop": round(wall * 1e3 / replays, 2),
            "finite": ok}


def mixed_warm_start(resid, replays=2):
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
    sec = r["ms_per_loop"] / 1e3
    del model
    return {"workload": f"{len(inp.seqlens)} packed requests, latent lengths 128..1024 (total "
                        f"{int(np.sum(inp.seqlens))} tokens), half warm-started, {cfg.n_steps} Euler steps as one "
                        f"hipGraph, W8A8", "request_steps_per_s": round(req_steps / sec, 1),
            "token_steps_per_s": round(tok_steps / sec), "active_request_steps": req_steps,
            "ms_per_loop": r["ms_per_loop"], "finite": r["finite"]}


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


def large_model_loops(replays=2):
    """Step rates of the other model sizes: the serving model (24 blocks,
    hidden 1536, 8 requests as 16 CFG rows of 512 latent tokens) with fp16,
    W8A8 and 8-bit weight-only weights side by side on the same inputs, and
    the 4-bit-weight model (24 blocks, hidden 2048, 4 requests as 8 CFG rows of
    1024 tokens); 8 Euler steps as one graph each."""
    import torch
    import ald_inputs as I
    from audio_latent_diffusion_amd import runtime
    out = {}
    for cfg, arms in ((I.SERVE, ("w8a8", "f16", "w8a16")), (I.Q4, ("q4",))):
        params = device_params(cfg, cfg.seed)
        inp = I.make_inputs(cfg)
        tokens = 2 * cfg.requests * cfg.seq
        # the six block linears of the step (the text K/V projection is hoisted)
        lin_ops = 2.0 * tokens * sum(n * k for name, (n, k) in I.linear_shapes(cfg).items() if name != "kv") \
            * cfg.n_blocks
        for arm in arms:
            model = runtime.DiTModel(cfg.replace(wmode=arm), params)
            r = loop_rate(model, inp, 1.0, replays)
            key = f"serve_{arm}" if cfg is I.SERVE else "q4_model"
            out[key] = dict(
                workload=f"{cfg.n_blocks} blocks, hidden {cfg.hidden}, {cfg.requests} requests x CFG pair of "
                         f"{cfg.seq} latent tokens ({tokens} rows), {arm} weights, 8 Euler steps as one hipGraph",
                linear_ops_per_step=lin_ops,
                linear_rate=round(lin_ops * r["steps_per_s"] / 1e12, 1),
                linear_rate_unit="TOP/s" if arm == "w8a8" else "TFLOP/s", **r)
            del model
            torch.cuda.empty_cache()
        del params
        torch.cuda.empty_cache()
    return out


def variant_loops(model, resid):
    """The mid-size model's loop under other settings: the DDIM sampler over
    the 200-step grid (the warm-start pages' backbone setting, steering in
    steps 40-79), and steering at the latent and text sites (8 Euler steps;
    the text site re-projects the steered text's K/V in every step)."""
    import ald_inputs as I
    out = {}
    cfg = I.MID_DDIM
    r = loop_rate(model.with_config(sampler="ddim", n_steps=cfg.n_steps), I.make_inputs(cfg), resid, 2)
    out["ddim_200"] = dict(workload="DDIM sampler, 200 steps as one hipGraph, steering alpha 0.5 at block 12 "
                                    "in steps 40-79", **r)
    for site in ("latent", "text"):
        cfg = I.MID.replace(steer_site=site)
        inp = I.make_inputs(cfg)
        unit = float(np.mean(np.linalg.norm(inp.x, axis=1))) if site == "latent" else \
            float(np.mean(np.linalg.norm(inp.text[:cfg.requests].reshape(-1, cfg.text_dim).astype(np.float64), axis=1)))
        r = loop_rate(model.with_config(steer_site=site), inp, unit, 20)
        out[f"steer_{site}_site"] = dict(workload=f"8 Euler steps as one hipGraph, steering alpha 0.5 at the "
                                                  f"{site} site in steps 2-5", **r)
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=160, help="timed denoise steps")
    ap.add_argument("--warmup", type=int, default=16, help="untimed denoise steps")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--cpu-budget", type=float, default=20.0)
    ap.add_argument("--leg", default="", help="counter legs only (gemm,serve,kernels,copy) for rocprofv3 runs")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on one GPU only; --gpus N > 1 is not supported. The step shards by request "
              "(each GPU would hold the weights and run its own requests' CFG pairs with no per-step "
              "exchange), and no multi-GPU path is built.", file=sys.stderr)
        sys.exit(2)
    if args.leg:
        counter_legs(args.leg.split(","), 20)
        return

    import torch
    import ald_inputs as I
    from audio_latent_diffusion_amd import runtime

    cfg = I.MID
    params = I.make_params(cfg)
    inp = I.make_inputs(cfg)
    model = runtime.DiTModel(cfg, params)

    # steering unit: mean per-token residual norm at the steered block over the
    # 8 steps of the alpha = 0 run (a calibration input, outside the timed region)
    zero = I.make_inputs(cfg)
    zero.alpha[:] = 0
    cal = runtime.StepRunner(model, zero.x, zero.text, zero.seqlens, zero.t_grid, zero.guidance, zero.alpha,
                             zero.direction, 0.0)
    cal.collect_block_norms()
    norms = []
    for i in range(cfg.n_steps):
        cal.step(i)
        norms.append(cal.block_norms.double().mean().item())
    resid = float(np.mean(norms))
    del cal

    # the whole 8-step sampler loop is one graph; a partial graph of the first
    # K mod 8 steps makes the timed count exactly K denoise steps
    run = runtime.StepRunner(model, inp.x, inp.text, inp.seqlens, inp.t_grid, inp.guidance, inp.alpha,
                             inp.direction, resid)
    x_init = run.x.clone()
    full_graph = run.capture_graph(range(cfg.n_steps))

    def replay(graph):
        run.x.copy_(x_init)  # a fresh request: the latent restarts from its noise
        run.launch_graph(graph)

    def schedule(k):
        sched = [full_graph] * (k // cfg.n_steps)
        if k % cfg.n_steps:
            sched.append(run.capture_graph(range(k % cfg.n_steps)))
        return sched

    warm, timed = schedule(args.warmup), schedule(args.steps)
    for gr in warm:
        replay(gr)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    start.record(stream)
    for gr in timed:
        replay(gr)
    end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ev_ms = start.elapsed_time(end)
    steps_per_s = args.steps / wall
    ok = bool(torch.isfinite(run.x).all().item())

    variants = variant_loops(model, resid)
    variants["warm_start_mixed"] = mixed_warm_start(resid)
    variants.update(large_model_loops())
    ms_launch, ops_launch, bytes_launch = gemm_mix_timing(cfg)
    floor_us = graph_floor_us()
    achieved = ops_launch / (ms_launch / 1e3) / 1e12
    traffic = measured_traffic()
    serve = serve_gemm()
    kernels = kernel_rooflines()

    # the step's algorithmic work: int8 GEMM ops of the block linears (the text
    # K/V projection is hoisted out of the step) and attention flops
    M, H, F, S, T, nh = cfg.tokens, cfg.hidden, cfg.mlp, cfg.seq, cfg.text_tokens, cfg.n_heads
    int8_ops = cfg.n_blocks * sum(2.0 * M * N * K for K, N in MIX_SHAPES(H, F))
    attn_flops = cfg.n_blocks * cfg.cfg_rows * nh * 4.0 * 64 * (S * S + S * T)
    step_s = 1.0 / steps_per_s
    line = {
        "metric": "DiT denoise steps/s (CFG batch) + W8A8 GEMM % of int8 MFMA peak on 1 GPU",
        "value": round(steps_per_s, 2),
        "unit": "steps/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall * 1e3 / args.steps, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8",
        "data": "synthetic",
        "config": {"workload": "mid-size DiT, 16 blocks, hidden 1024, 16 heads, MLP 4096, latent 256x64, "
                               "text 128x768, CFG batch 2, W8A8, 8 Euler steps as one hipGraph, "
                               "steering alpha 0.5 at block 12 in steps 2-5",
                   "global_batch": cfg.cfg_rows, "seq_len": cfg.seq, "parallelism": "none",
                   "denoise_steps_per_replay": cfg.n_steps, "attention_dtype": "fp16"},
        "event_steps_per_s": round(args.steps / (ev_ms / 1e3), 2),
        "finite": ok,
        "roofline": {"bound": "mfma", "kernel": "W8A8 GEMM (int8 MFMA), the step's launch mix at M = 512",
                     "achieved": round(achieved, 2), "peak": INT8_PEAK_TOPS, "unit": "TOP/s",
                     "frac": round(achieved / INT8_PEAK_TOPS, 4),
                     "traffic": None if traffic is None else round(traffic),
                     "avg_launch_us": round(ms_launch * 1e3, 2),
                     "graph_noop_launch_us": round(floor_us, 2),
                     "algorithmic_ops_per_launch": ops_launch, "algorithmic_bytes_per_launch": bytes_launch},
        "step_rates": {"int8_gemm_tops": round(int8_ops / step_s / 1e12, 1),
                       "attention_tflops": round(attn_flops / step_s / 1e12, 2),
                       "int8_gemm_ops_per_step": int8_ops, "attention_flops_per_step": attn_flops},
        "w8a8_gemm_serve": serve,
        "loop_variants": variants,
        "kernels": kernels,
    }
    if not args.no_cpu:
        line["cpu_baseline"] = cpu_baseline(cfg, params, inp, resid, args.cpu_budget)
    print(json.dumps(line))


if __name__ == "__main__":
    main()
