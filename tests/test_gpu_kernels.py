"""Per-kernel parity of the HIP path (through the C ABI) against the oracle.

Bit-exact: int8 codes, per-row scales, int32 accumulators, q4 codes/scales.
Floating point: tolerances derived from one fp16 rounding after fp32
accumulation (see tests/_gpu.py).  Shapes cover tiny, ragged (not a tile
multiple in M, N or K), several tiles, and the mid/serve workload shapes.
"""
import math

import numpy as np
import pytest
import torch

from audio_latent_diffusion_amd import binding as B
from audio_latent_diffusion_amd import _lib as L
from oracle import ald_oracle as O
from tests._gpu import dev, f16_close, host, needs_gpu

pytestmark = [pytest.mark.gpu, needs_gpu]


def rng(seed):
    return np.random.default_rng(seed)


# ------------------------------------------------------------- quantizers

@pytest.mark.parametrize("M,K", [(1, 8), (7, 136), (64, 256), (33, 1024), (5, 6144), (3, 8192)])
def test_quantize_rows_bit_exact(M, K):
    r = rng(M * 1000 + K)
    x = (r.standard_normal((M, K)) * r.uniform(0.01, 30, (M, 1))).astype(np.float16)
    x[0, : min(8, K)] = [0.5, 1.5, 2.5, -0.5, 3.5, -2.5, 126.5, 127][: min(8, K)]
    if M > 2:
        x[2] = 0
    q, s = B.quantize_rows_q8(dev(x))
    qo, so = O.quantize_rows_q8(x)
    assert np.array_equal(host(q), qo)
    assert host(s).tobytes() == so.tobytes()


def test_quantize_rows_strided_input():
    x = rng(1).standard_normal((20, 96)).astype(np.float16)
    xt = dev(x)
    q, s = B.quantize_rows_q8(xt[:, 16:80])
    qo, so = O.quantize_rows_q8(x[:, 16:80])
    assert np.array_equal(host(q), qo) and np.array_equal(host(s), so)


@pytest.mark.parametrize("N,K", [(1, 32), (5, 96), (130, 256), (1536, 1536)])
def test_quantize_q4_bit_exact(N, K):
    w = (0.02 * rng(N + K).standard_normal((N, K))).astype(np.float16)
    w[0, :32] = 0
    p, s = B.quantize_q4(dev(w))
    po, so = O.quantize_q4(w)
    assert np.array_equal(host(p), po)
    assert np.array_equal(host(s).view(np.uint16), so.view(np.uint16))


# 5003 rows: more than 1024 four-row workgroups, so LayerNorm + quantization
# walks two rows per wave, with a ragged second round
@pytest.mark.parametrize("M,H", [(1, 64), (13, 256), (128, 1024), (40, 1536), (9, 2048), (5003, 1536)])
def test_ln_quant(M, H):
    r = rng(M + H)
    x = (r.standard_normal((M, H)) * 2 + 0.5).astype(np.float16)
    g = (1 + 0.02 * r.standard_normal(H)).astype(np.float32)
    b = (0.02 * r.standard_normal(H)).astype(np.float32)
    u = torch.empty((M, H), dtype=torch.float16, device="cuda")
    q, s = B.ln_quant(dev(x), dev(g), dev(b), 1e-5, u_out=u)
    uo = O.layer_norm(x, g, b, 1e-5)
    ug = host(u)
    f16_close(ug, uo, rtol=2.0 ** -10, atol_frac=2.0 ** -11)
    # the codes are bit-exactly the quantization of the fp16 row they came from
    qo, so = O.quantize_rows_q8(ug)
    assert np.array_equal(host(q), qo)
    assert np.array_equal(host(s), so)
    y = B.ln_f16(dev(x), dev(g), dev(b), 1e-5)
    assert np.array_equal(host(y), ug)


def _extreme_rows(H, r):
    """fp16 rows at the edges of the format and of the statistics: a large
    common offset (variance far below the mean squared), a constant row
    (zero variance), values near the fp16 maximum, subnormals only, one
    spike in a row of zeros (at the first, a middle and the last column),
    alternating signs, negative zeros."""
    rows = [1000.0 + r.standard_normal(H), np.full(H, 3.0), 60000.0 * np.sign(r.standard_normal(H)),
            6e-8 * r.integers(-900, 900, H), np.eye(1, H, 0)[0] * 7.0, np.eye(1, H, H // 2 + 3)[0] * -300.0,
            np.eye(1, H, H - 1)[0] * 0.001, np.where(np.arange(H) % 2 == 0, 1.0, -1.0) * 512.0, np.full(H, -0.0),
            r.standard_normal(H) * 1e-3 + 65000.0 * (np.arange(H) == 5)]
    return np.stack(rows).astype(np.float16)


# Rows at the edges of fp16 and of the statistics, through LayerNorm +
# quantization (codes bit-exact against the quantization of the GPU's own
# fp16 row, LayerNorm within the bar above) and through the activation
# quantizer alone (bit-exact)
@pytest.mark.parametrize("H", [256, 1536, 6144])
def test_row_kernels_extreme_values(H):
    r = rng(H + 3)
    x = _extreme_rows(H, r)
    g = (1 + 0.02 * r.standard_normal(H)).astype(np.float32)
    b = (0.02 * r.standard_normal(H)).astype(np.float32)
    u = torch.empty(x.shape, dtype=torch.float16, device="cuda")
    q, s = B.ln_quant(dev(x), dev(g), dev(b), 1e-5, u_out=u)
    ug = host(u)
    f16_close(ug, O.layer_norm(x, g, b, 1e-5), rtol=2.0 ** -10, atol_frac=2.0 ** -11)
    qo, so = O.quantize_rows_q8(ug)
    assert np.array_equal(host(q), qo) and np.array_equal(host(s), so)
    q, s = B.quantize_rows_q8(dev(x))
    qo, so = O.quantize_rows_q8(x)
    assert np.array_equal(host(q), qo) and host(s).tobytes() == so.tobytes()


# Launches whose data (2 B read and 1 B written per element) exceed the 256 MB
# last-level cache take the non-temporal variants of the row kernels; the
# step's launches take the cached ones.  65536 rows of 1536 (302 MB):
# sampled rows against the oracle, every row of the two variants computed the
# same way, so the codes are bit-exact here as at the step's sizes.
def test_row_kernels_beyond_last_level_cache():
    M, H = 65536, 1536
    g = torch.Generator(device="cuda").manual_seed(11)
    xt = (torch.randn((M, H), generator=g, device="cuda") * 2 + 0.5).half()
    r = rng(12)
    gam = (1 + 0.02 * r.standard_normal(H)).astype(np.float32)
    bet = (0.02 * r.standard_normal(H)).astype(np.float32)
    rows = np.unique(np.concatenate([[0, 1, M // 2, M - 2, M - 1], r.integers(0, M, 59)]))
    idx = torch.from_numpy(rows).cuda()
    xs = host(xt.index_select(0, idx))
    q, s = B.quantize_rows_q8(xt)
    qo, so = O.quantize_rows_q8(xs)
    assert np.array_equal(host(q.index_select(0, idx)), qo)
    assert host(s.index_select(0, idx)).tobytes() == so.tobytes()
    del q, s
    u = torch.empty((M, H), dtype=torch.float16, device="cuda")
    q, s = B.ln_quant(xt, dev(gam), dev(bet), 1e-5, u_out=u)
    ug = host(u.index_select(0, idx))
    f16_close(ug, O.layer_norm(xs, gam, bet, 1e-5), rtol=2.0 ** -10, atol_frac=2.0 ** -11)
    qo, so = O.quantize_rows_q8(ug)
    assert np.array_equal(host(q.index_select(0, idx)), qo) and np.array_equal(host(s.index_select(0, idx)), so)
    del q, s
    y = B.ln_f16(xt, dev(gam), dev(bet), 1e-5)
    assert np.array_equal(host(y.index_select(0, idx)), ug)


# ------------------------------------------------------------- W8A8 GEMM

# small launches take 32 x 64 tiles whose K splits in two halves when the
# 128-byte stages are even in number and at least 4: (200, 1024, 257),
# (70, 512, 100) (two stages per half, fewer than the ring's lookahead) and
# (130, 6144, 96); (40, 384, 64) has an odd count and runs unsplit
W8A8_SHAPES = [(1, 16, 1), (3, 32, 7), (77, 272, 130), (128, 256, 768), (200, 1024, 257), (70, 512, 100),
               (40, 384, 64), (512, 1024, 3072), (130, 6144, 96)]


@pytest.mark.parametrize("M,K,N", W8A8_SHAPES)
def test_w8a8_linear(M, K, N):
    r = rng(M * 7 + K * 3 + N)
    x = r.standard_normal((M, K)).astype(np.float16)
    w = (0.02 * r.standard_normal((N, K))).astype(np.float16)
    b = (0.02 * r.standard_normal(N)).astype(np.float32)
    res = r.standard_normal((M, N)).astype(np.float16)
    wq, ws = O.quantize_rows_q8(w)
    acc = torch.empty((M, N), dtype=torch.int32, device="cuda")
    xq = torch.empty((M, K), dtype=torch.int8, device="cuda")
    xs = torch.empty(M, dtype=torch.float32, device="cuda")
    y = B.w8a8_linear(dev(x), dev(wq), dev(ws), bias=dev(b), residual=dev(res), xq=xq, x_scale=xs, acc=acc)
    ro = O.w8a8_linear(x, wq, ws, b, residual=res)
    assert np.array_equal(host(xq), ro.xq)
    assert np.array_equal(host(xs), ro.x_scale)
    assert np.array_equal(host(acc).astype(np.int64), ro.acc)
    f16_close(host(y), ro.y)


# Saturated codes: rows of +-1 and weights of +-0.01 quantize to +-127 everywhere,
# so at K = 6144 the int32 accumulators reach 127 * 127 * 6144 ~ 9.9e7 (all
# signs equal in some rows and columns); shapes of both large tiles and of the
# small ones
@pytest.mark.parametrize("M,K,N", [(512, 6144, 384), (8192, 1536, 1536), (96, 6144, 130)])
def test_w8a8_saturated_codes(M, K, N):
    r = rng(M + K + N)
    x = np.where(r.random((M, K)) < 0.5, -1.0, 1.0).astype(np.float16)
    x[0] = 1.0
    w = np.where(r.random((N, K)) < 0.5, -0.01, 0.01).astype(np.float16)
    w[0] = 0.01
    w[1] = -0.01
    wq, ws = O.quantize_rows_q8(w)
    assert np.abs(wq.astype(np.int64)).min() == 127
    acc = torch.empty((M, N), dtype=torch.int32, device="cuda")
    xq = torch.empty((M, K), dtype=torch.int8, device="cuda")
    xs = torch.empty(M, dtype=torch.float32, device="cuda")
    y = B.w8a8_linear(dev(x), dev(wq), dev(ws), xq=xq, x_scale=xs, acc=acc)
    ro = O.w8a8_linear(x, wq, ws, None)
    assert np.array_equal(host(xq), ro.xq) and np.array_equal(host(xs), ro.x_scale)
    a = host(acc).astype(np.int64)
    assert a[0, 0] == 127 * 127 * K and a[0, 1] == -127 * 127 * K
    assert np.array_equal(a, ro.acc)
    f16_close(host(y), ro.y)


def test_w8a8_gelu_inplace_residual_and_prequant():
    r = rng(9)
    M, K, N = 96, 512, 384
    x = r.standard_normal((M, K)).astype(np.float16)
    w = (0.05 * r.standard_normal((N, K))).astype(np.float16)
    wq, ws = O.quantize_rows_q8(w)
    # GELU epilogue
    y = B.w8a8_linear(dev(x), dev(wq), dev(ws), act=L.ALD_ACT_GELU)
    f16_close(host(y), O.w8a8_linear(x, wq, ws, None, act=1).y)
    # in-place residual (residual aliases y)
    h = r.standard_normal((M, N)).astype(np.float16)
    ht = dev(h)
    B.w8a8_linear(dev(x), dev(wq), dev(ws), residual=ht, y=ht)
    f16_close(host(ht), O.w8a8_linear(x, wq, ws, None, residual=h).y)
    # pre-quantized input
    xq, xs = O.quantize_rows_q8(x)
    y2 = B.w8a8_linear(None, dev(wq), dev(ws), xq=dev(xq), x_scale=dev(xs), prequant=True)
    assert np.array_equal(host(y2), host(B.w8a8_linear(dev(x), dev(wq), dev(ws))))


@pytest.mark.parametrize("M,K,N", [(8192, 1536, 4608), (8192, 6144, 1536)])
def test_w8a8_serve_shapes_sampled(M, K, N):
    """Full serving-batch shapes in the launch configuration of the step;
    accumulators checked on sampled rows against the exact integer GEMM."""
    g = torch.Generator(device="cuda").manual_seed(M + K + N)
    xq = torch.randint(-127, 128, (M, K), dtype=torch.int8, device="cuda", generator=g)
    wq = torch.randint(-127, 128, (N, K), dtype=torch.int8, device="cuda", generator=g)
    xs = torch.rand(M, device="cuda", generator=g) * 0.01
    ws = torch.rand(N, device="cuda", generator=g) * 0.001
    acc = torch.empty((M, N), dtype=torch.int32, device="cuda")
    y = B.w8a8_linear(None, wq, ws, xq=xq, x_scale=xs, acc=acc, prequant=True)
    rows = np.sort(rng(0).choice(M, 48, replace=False))
    rows = np.concatenate([rows, [0, M - 1]])
    a = host(xq)[rows]
    ref = O.int_gemm(a, host(wq))
    assert np.array_equal(host(acc)[rows].astype(np.int64), ref)
    yo = (ref * host(xs)[rows, None].astype(np.float64) * host(ws)[None, :].astype(np.float64)).astype(np.float16)
    f16_close(host(y)[rows], yo)


@pytest.mark.parametrize("M,K,N", [(8192, 1536, 4608), (8192, 1536, 1536), (8192, 6144, 1536), (8192, 1536, 6144)])
def test_w8a8_serve_shapes_every_tile(M, K, N):
    """The serving block's W8A8 launches (256 x 192 tiles with producer waves
    for qkv, o/q/ox and down, 256 x 256 for up; row-band tile order): the
    whole int32 accumulator against the exact integer GEMM, so every tile of
    the launch is checked, and the fp16 output on its first and last rows."""
    g = torch.Generator(device="cuda").manual_seed(3 * M + K + N)
    xq = torch.randint(-127, 128, (M, K), dtype=torch.int8, device="cuda", generator=g)
    wq = torch.randint(-127, 128, (N, K), dtype=torch.int8, device="cuda", generator=g)
    xs = torch.rand(M, device="cuda", generator=g) * 0.01
    ws = torch.rand(N, device="cuda", generator=g) * 0.001
    acc = torch.empty((M, N), dtype=torch.int32, device="cuda")
    y = B.w8a8_linear(None, wq, ws, xq=xq, x_scale=xs, acc=acc, prequant=True)
    a, w = host(xq), host(wq)
    ref = O.int_gemm(a, w)
    assert np.array_equal(host(acc).astype(np.int64), ref)
    rows = np.array([0, 1, M - 2, M - 1])
    yo = (ref[rows] * host(xs)[rows, None].astype(np.float64) * host(ws)[None, :].astype(np.float64)).astype(np.float16)
    f16_close(host(y)[rows], yo)


# the two large tiles of the launch, ragged in M and N, K an odd number of
# 128-byte stages: 256 x 192 (N = 1500 fills one round of 256 CUs with 256
# such tiles, where 256 x 256 tiles would leave 64 CUs idle) and 256 x 256
# (N = 6100: both need whole rounds of the same area, and the tie keeps
# 256 x 256); checked on sampled rows, the ragged last rows included
LARGE_TILE_SHAPES = [(8000, 640, 1500), (8000, 640, 6100)]


def _sample_rows(M, seed, n=40):
    return np.concatenate([np.sort(rng(seed).choice(M - 8, n, replace=False)), np.arange(M - 8, M)])


@pytest.mark.parametrize("M,K,N", LARGE_TILE_SHAPES)
def test_w8a8_large_tiles_ragged(M, K, N):
    r = rng(M + 3 * K + N)
    x = r.standard_normal((M, K)).astype(np.float16)
    w = (0.02 * r.standard_normal((N, K))).astype(np.float16)
    b = (0.02 * r.standard_normal(N)).astype(np.float32)
    res = r.standard_normal((M, N)).astype(np.float16)
    wq, ws = O.quantize_rows_q8(w)
    acc = torch.empty((M, N), dtype=torch.int32, device="cuda")
    xq = torch.empty((M, K), dtype=torch.int8, device="cuda")
    xs = torch.empty(M, dtype=torch.float32, device="cuda")
    y = B.w8a8_linear(dev(x), dev(wq), dev(ws), bias=dev(b), residual=dev(res), xq=xq, x_scale=xs, acc=acc)
    rows = _sample_rows(M, N)
    ro = O.w8a8_linear(x[rows], wq, ws, b, residual=res[rows])
    assert np.array_equal(host(xq)[rows], ro.xq)
    assert np.array_equal(host(xs)[rows], ro.x_scale)
    assert np.array_equal(host(acc)[rows].astype(np.int64), ro.acc)
    f16_close(host(y)[rows], ro.y)
    g = B.w8a8_linear(dev(x), dev(wq), dev(ws), bias=dev(b), act=L.ALD_ACT_GELU)
    f16_close(host(g)[rows], O.w8a8_linear(x[rows], wq, ws, b, act=1).y)


@pytest.mark.parametrize("M,K,N", LARGE_TILE_SHAPES)
def test_q8w_large_tiles_ragged(M, K, N):
    r = rng(M + 7 * K + N)
    x = r.standard_normal((M, K)).astype(np.float16)
    w = (0.02 * r.standard_normal((N, K))).astype(np.float16)
    b = (0.02 * r.standard_normal(N)).astype(np.float32)
    res = r.standard_normal((M, N)).astype(np.float16)
    q, s = O.quantize_rows_q8(w)
    rows = _sample_rows(M, N + 2)
    y = B.q8w_linear(dev(x), dev(q), dev(s), dev(b), residual=dev(res))
    f16_close(host(y)[rows], O.q8w_linear(x[rows], q, s, b, residual=res[rows]))


@pytest.mark.parametrize("M,K,N", LARGE_TILE_SHAPES)
def test_f16_large_tiles_ragged(M, K, N):
    r = rng(M + 5 * K + N)
    x = r.standard_normal((M, K)).astype(np.float16)
    w = (0.05 * r.standard_normal((N, K))).astype(np.float16)
    b = (0.02 * r.standard_normal(N)).astype(np.float32)
    res = r.standard_normal((M, N)).astype(np.float16)
    rows = _sample_rows(M, N + 1)
    y = B.f16_linear(dev(x), dev(w), dev(b), residual=dev(res))
    f16_close(host(y)[rows], O.f16_linear(x[rows], w, b, residual=res[rows]))
    y = B.f16_linear(dev(x), dev(w), dev(b), act=L.ALD_ACT_GELU)
    f16_close(host(y)[rows], O.f16_linear(x[rows], w, b, act=1))


# ------------------------------------------------------------- fp16 and q4 GEMMs

@pytest.mark.parametrize("M,K,N", [(1, 8, 1), (77, 264, 130), (256, 1024, 64), (300, 2048, 520)])
def test_f16_linear(M, K, N):
    r = rng(M + K + N)
    x = r.standard_normal((M, K)).astype(np.float16)
    w = (0.05 * r.standard_normal((N, K))).astype(np.float16)
    b = (0.02 * r.standard_normal(N)).astype(np.float32)
    res = r.standard_normal((M, N)).astype(np.float16)
    y = B.f16_linear(dev(x), dev(w), dev(b), residual=dev(res))
    f16_close(host(y), O.f16_linear(x, w, b, residual=res))
    y = B.f16_linear(dev(x), dev(w), dev(b), act=L.ALD_ACT_GELU)
    f16_close(host(y), O.f16_linear(x, w, b, act=1))


@pytest.mark.parametrize("M,K,N", [(1, 32, 1), (77, 96, 130), (256, 2048, 64), (300, 1024, 520), (200, 640, 203)])
def test_q4_linear(M, K, N):
    r = rng(M * 3 + K + N)
    x = r.standard_normal((M, K)).astype(np.float16)
    w = (0.02 * r.standard_normal((N, K))).astype(np.float16)
    b = (0.02 * r.standard_normal(N)).astype(np.float32)
    res = r.standard_normal((M, N)).astype(np.float16)
    p, s = O.quantize_q4(w)
    y = B.q4_linear(dev(x), dev(p), dev(s), dev(b), residual=dev(res))
    f16_close(host(y), O.q4_linear(x, p, s, b, residual=res))


@pytest.mark.parametrize("M,K,N", [(8192, 2048, 6144), (8192, 8192, 2048)])
def test_q4_full_shapes_sampled(M, K, N):
    """4-bit weight GEMMs at the full 4-request x 1024-token CFG batch (8192
    rows, hidden 2048, MLP 8192) in the step's launch configuration, checked
    on sampled rows against the oracle."""
    r = rng(M + K + N)
    g = torch.Generator(device="cuda").manual_seed(K + N)
    x = torch.randn((M, K), dtype=torch.float16, device="cuda", generator=g)
    w = (0.02 * r.standard_normal((N, K))).astype(np.float16)
    b = (0.02 * r.standard_normal(N)).astype(np.float32)
    p, s = O.quantize_q4(w)
    y = B.q4_linear(x, dev(p), dev(s), dev(b), act=L.ALD_ACT_GELU)
    rows = np.concatenate([np.sort(rng(1).choice(M, 40, replace=False)), [0, M - 1]])
    f16_close(host(y)[rows], O.q4_linear(host(x)[rows], p, s, b, act=1))


# ------------------------------------------------------------- 8-bit weight-only GEMM

# one shape per tile size of the launch (64x64, 128x64, 128x128 and the
# 8-wave 256x192, whose weight copies are padded to a multiple of the
# waves), ragged in M and N, K an odd number of 64-element slices
@pytest.mark.parametrize("M,K,N", [(1, 64, 1), (77, 192, 130), (200, 640, 203), (1100, 320, 1400),
                                   (1500, 576, 1900), (3000, 640, 3900)])
def test_q8w_linear(M, K, N):
    r = rng(M * 5 + K + N)
    x = r.standard_normal((M, K)).astype(np.float16)
    w = (0.02 * r.standard_normal((N, K))).astype(np.float16)
    b = (0.02 * r.standard_normal(N)).astype(np.float32)
    res = r.standard_normal((M, N)).astype(np.float16)
    q, s = O.quantize_rows_q8(w)
    y = B.q8w_linear(dev(x), dev(q), dev(s), dev(b), residual=dev(res))
    f16_close(host(y), O.q8w_linear(x, q, s, b, residual=res))


def test_q8w_gelu_inplace_residual_and_strided_input():
    r = rng(21)
    M, K, N = 160, 384, 272
    xw = r.standard_normal((M, K + 64)).astype(np.float16)
    w = (0.05 * r.standard_normal((N, K))).astype(np.float16)
    q, s = O.quantize_rows_q8(w)
    xd = dev(xw)[:, :K]  # row stride K + 64
    y = B.q8w_linear(xd, dev(q), dev(s), act=L.ALD_ACT_GELU)
    f16_close(host(y), O.q8w_linear(xw[:, :K], q, s, None, act=1))
    h = r.standard_normal((M, N)).astype(np.float16)
    ht = dev(h)
    B.q8w_linear(xd, dev(q), dev(s), residual=ht, y=ht)
    f16_close(host(ht), O.q8w_linear(xw[:, :K], q, s, None, residual=h))


@pytest.mark.parametrize("M,K,N", [(8192, 1536, 4608), (8192, 6144, 1536)])
def test_q8w_serve_shapes_sampled(M, K, N):
    """8-bit weight-only GEMMs at the serving CFG batch (8192 rows, hidden
    1536, MLP 6144) in the step's launch configuration, sampled rows."""
    r = rng(M + K + N + 1)
    g = torch.Generator(device="cuda").manual_seed(K + N + 1)
    x = torch.randn((M, K), dtype=torch.float16, device="cuda", generator=g)
    w = (0.02 * r.standard_normal((N, K))).astype(np.float16)
    b = (0.02 * r.standard_normal(N)).astype(np.float32)
    q, s = O.quantize_rows_q8(w)
    y = B.q8w_linear(x, dev(q), dev(s), dev(b), act=L.ALD_ACT_GELU)
    rows = np.concatenate([np.sort(rng(2).choice(M, 40, replace=False)), [0, M - 1]])
    f16_close(host(y)[rows], O.q8w_linear(host(x)[rows], q, s, b, act=1))


# ------------------------------------------------------------- attention

def _attn_ref(q, k, v, nh, cu_q, cu_k):
    return O.attention_varlen(q, k, v, cu_q, cu_k, nh, 0.125)


# the launch takes 2-wave workgroups of 32 queries on small grids, 4-wave
# ones of 64 queries from 256 such workgroups ((4, 200, 150, 16)) and 4-wave
# ones of 128 queries from 512 ((16, 400, 140, 8)); grids of 1024 or more
# workgroups run remapped to one range of (sequence, head) per XCD ((16, 500,
# ., 16)), and dense key sets of at most 128 keys issue the Q loads together
# with the first tile copies; ragged queries and keys
@pytest.mark.parametrize("B_,Sq,Sk,nh", [(1, 1, 1, 1), (2, 64, 32, 4), (2, 100, 77, 3), (1, 256, 256, 2),
                                          (3, 130, 200, 2), (2, 96, 150, 2), (1, 40, 300, 3), (16, 512, 128, 1),
                                          (4, 200, 150, 16), (16, 400, 140, 8), (16, 500, 140, 16),
                                          (16, 500, 100, 16)])
def test_attention_dense(B_, Sq, Sk, nh):
    r = rng(B_ * 100 + Sq + Sk)
    W = nh * 64
    q = r.standard_normal((B_ * Sq, W)).astype(np.float16)
    k = r.standard_normal((B_ * Sk, W)).astype(np.float16)
    v = r.standard_normal((B_ * Sk, W)).astype(np.float16)
    out = B.attn_fwd(dev(q), dev(k), dev(v), nh, B_, Sq, Sk)
    ref = _attn_ref(q, k, v, nh, np.arange(B_ + 1) * Sq, np.arange(B_ + 1) * Sk)
    f16_close(host(out), ref, rtol=2.0 ** -8, atol_frac=2.0 ** -8)


def test_attention_strided_qkv_views():
    r = rng(5)
    S, nh = 96, 3
    H = nh * 64
    qkv = r.standard_normal((2 * S, 3 * H)).astype(np.float16)
    t = dev(qkv)
    out = B.attn_fwd(t[:, :H], t[:, H:2 * H], t[:, 2 * H:], nh, 2, S, S)
    cu = np.arange(3) * S
    ref = _attn_ref(qkv[:, :H], qkv[:, H:2 * H], qkv[:, 2 * H:], nh, cu, cu)
    f16_close(host(out), ref, rtol=2.0 ** -8, atol_frac=2.0 ** -8)


def test_attention_varlen_and_empty():
    r = rng(6)
    lens_q = [128, 1, 0, 577, 64, 200]
    lens_k = [128, 1, 5, 577, 0, 33]
    nh = 2
    W = nh * 64
    cq = np.concatenate([[0], np.cumsum(lens_q)]).astype(np.int32)
    ck = np.concatenate([[0], np.cumsum(lens_k)]).astype(np.int32)
    q = r.standard_normal((cq[-1], W)).astype(np.float16)
    k = r.standard_normal((ck[-1], W)).astype(np.float16)
    v = r.standard_normal((ck[-1], W)).astype(np.float16)
    out = B.attn_fwd(dev(q), dev(k), dev(v), nh, len(lens_q), cu_seqlens_q=dev(cq), cu_seqlens_k=dev(ck),
                     max_sq=max(lens_q), max_sk=max(lens_k))
    ref = _attn_ref(q, k, v, nh, cq, ck)
    f16_close(host(out), ref, rtol=2.0 ** -8, atol_frac=2.0 ** -8)


def test_attention_single_key_and_uniform():
    r = rng(7)
    nh, S = 2, 70
    q = r.standard_normal((S, nh * 64)).astype(np.float16)
    k = r.standard_normal((1, nh * 64)).astype(np.float16)
    v = r.standard_normal((1, nh * 64)).astype(np.float16)
    out = host(B.attn_fwd(dev(q), dev(k), dev(v), nh, 1, S, 1))
    assert np.array_equal(out, np.broadcast_to(v, out.shape))        # one key: weight exactly 1
    kk = np.broadcast_to(k, (40, nh * 64)).copy()
    vv = r.standard_normal((40, nh * 64)).astype(np.float16)
    out = host(B.attn_fwd(dev(q), dev(kk), dev(vv), nh, 1, S, 40))
    f16_close(out, np.broadcast_to(vv.astype(np.float64).mean(axis=0), out.shape), rtol=2.0 ** -9,
              atol_frac=2.0 ** -9)


# Scores spread over hundreds of units.  The weights are 2^(c (s - m)) in
# fp16 against a row reference m, so a reference taken over only part of a
# query's keys (one of the 4 lanes that hold them) overflows the weights to
# inf and the row to NaN once the spread passes ~90; the unit-normal inputs
# above never reach that.  Grid shapes as in test_attention_dense, with
# ragged key counts.
@pytest.mark.parametrize("B_,Sq,Sk,nh,mult", [(2, 64, 32, 4, 3.0), (4, 200, 150, 16, 2.0), (16, 500, 140, 16, 2.0),
                                               (2, 256, 512, 8, 3.0), (16, 512, 128, 4, 4.0)])
def test_attention_wide_score_range(B_, Sq, Sk, nh, mult):
    r = rng(B_ * 7 + Sq + Sk)
    W = nh * 64
    q = (r.standard_normal((B_ * Sq, W)) * mult).astype(np.float16)
    k = (r.standard_normal((B_ * Sk, W)) * mult).astype(np.float16)
    v = r.standard_normal((B_ * Sk, W)).astype(np.float16)
    out = B.attn_fwd(dev(q), dev(k), dev(v), nh, B_, Sq, Sk)
    ref = _attn_ref(q, k, v, nh, np.arange(B_ + 1) * Sq, np.arange(B_ + 1) * Sk)
    f16_close(host(out), ref, rtol=2.0 ** -8, atol_frac=2.0 ** -8)


# Keys along one direction with scores rising (or falling) along the key
# order by 60 units per 64-key tile: rising, every tile's maximum passes the
# exponent reference and moves it (the rescale of the output and the row
# sums runs at every tile); falling, the first tile holds each row's maximum.
@pytest.mark.parametrize("order", ["rising", "falling"])
@pytest.mark.parametrize("Sk", [512, 333])
def test_attention_moving_reference(order, Sk):
    r = rng(11 if order == "rising" else 12)
    nh, Sq = 2, 96
    W = nh * 64
    u = np.full(64, 0.5)                                  # |u|^2 = 16
    steps = np.arange(Sk) / 64.0 * 3.75                   # 60 score units per tile
    if order == "falling":
        steps = steps[::-1]
    q = (np.tile(u, (Sq, nh)) + 0.05 * r.standard_normal((Sq, W))).astype(np.float16)
    k = (np.tile(steps[:, None] * u[None, :], (1, nh)) + 0.05 * r.standard_normal((Sk, W))).astype(np.float16)
    v = r.standard_normal((Sk, W)).astype(np.float16)
    out = B.attn_fwd(dev(q), dev(k), dev(v), nh, 1, Sq, Sk)
    ref = _attn_ref(q, k, v, nh, np.array([0, Sq]), np.array([0, Sk]))
    f16_close(host(out), ref, rtol=2.0 ** -8, atol_frac=2.0 ** -8)


# ------------------------------------------------------------- steering, CFG, sampler

def test_steer_add():
    r = rng(8)
    M, H, S, R = 4 * 96, 256, 96, 2
    h = r.standard_normal((M, H)).astype(np.float16)
    h[5, 3] = np.float16(-0.0)
    d = r.standard_normal(H)
    d = (d / np.linalg.norm(d)).astype(np.float32)
    alpha = np.array([0.5, 0.0], np.float32)
    ht = dev(h)
    B.steer_add(ht, dev(alpha), 3.25, dev(d), rows_per_req=S, R=R)
    got = host(ht)
    row_req = (np.arange(M) // S) % R
    ref = O.steer_add(h, alpha[row_req], 3.25, d)
    f16_close(got, ref, rtol=2.0 ** -10, atol_frac=2.0 ** -11)
    untouched = row_req == 1
    assert got[untouched].tobytes() == h[untouched].tobytes()
    # alpha = 0 everywhere: bit-identical
    ht = dev(h)
    B.steer_add(ht, dev(np.zeros(2, np.float32)), 3.25, dev(d), rows_per_req=S, R=R)
    assert host(ht).tobytes() == h.tobytes()


@pytest.mark.parametrize("H", [256, 1536, 2000])
def test_steer_project(H):
    """Projection steering, h += beta (h . d) d, on rows of nonzero beta; rows of
    beta = 0 untouched bit for bit (ragged H exercises the partial chunk)."""
    r = rng(9 + H)
    M, S, R = 4 * 96, 96, 2
    h = r.standard_normal((M, H)).astype(np.float16)
    d = r.standard_normal(H)
    d = (d / np.linalg.norm(d)).astype(np.float32)
    beta = np.array([0.0, 0.75], np.float32)
    ht = dev(h)
    B.steer_add(ht, dev(beta), 123.0, dev(d), rows_per_req=S, R=R, mode=L.ALD_STEER_PROJECT)
    got = host(ht)
    row_req = (np.arange(M) // S) % R
    ref = O.steer_project(h, beta[row_req], d)
    f16_close(got, ref, rtol=2.0 ** -10, atol_frac=2.0 ** -11)
    untouched = row_req == 0
    assert got[untouched].tobytes() == h[untouched].tobytes()


# The row kernels cap their grids (16384 four-row workgroups for the
# quantizers and LayerNorms, 4096 for the steering add, 1024 for the
# projection) and walk the remaining rows with the grid stride, the next
# row's loads in flight; these row counts make each wave take several rows,
# with a ragged last round.
def test_row_kernels_grid_stride():
    r = rng(77)
    M, K = 4 * 16384 * 2 + 37, 64
    x = (r.standard_normal((M, K)) * r.uniform(0.01, 30, (M, 1))).astype(np.float16)
    q, s = B.quantize_rows_q8(dev(x))
    qo, so = O.quantize_rows_q8(x)
    assert np.array_equal(host(q), qo)
    assert host(s).tobytes() == so.tobytes()
    g = (1 + 0.02 * r.standard_normal(K)).astype(np.float32)
    b = (0.02 * r.standard_normal(K)).astype(np.float32)
    u = torch.empty((M, K), dtype=torch.float16, device="cuda")
    q, s = B.ln_quant(dev(x), dev(g), dev(b), 1e-5, u_out=u)
    ug = host(u)
    f16_close(ug, O.layer_norm(x, g, b, 1e-5), rtol=2.0 ** -10, atol_frac=2.0 ** -11)
    qo, so = O.quantize_rows_q8(ug)
    assert np.array_equal(host(q), qo)
    assert np.array_equal(host(s), so)


@pytest.mark.parametrize("mode", [L.ALD_STEER_ADD, L.ALD_STEER_PROJECT])
def test_steer_grid_stride(mode):
    r = rng(78 + mode)
    M, H, S, R = 4 * 4096 * 3 + 96, 128, 96, 2
    h = r.standard_normal((M, H)).astype(np.float16)
    d = r.standard_normal(H)
    d = (d / np.linalg.norm(d)).astype(np.float32)
    a = np.array([0.5, 0.0], np.float32)
    ht = dev(h)
    B.steer_add(ht, dev(a), 2.5, dev(d), rows_per_req=S, R=R, mode=mode)
    got = host(ht)
    row_req = (np.arange(M) // S) % R
    ref = O.steer_add(h, a[row_req], 2.5, d) if mode == L.ALD_STEER_ADD else O.steer_project(h, a[row_req], d)
    f16_close(got, ref, rtol=2.0 ** -10, atol_frac=2.0 ** -11)
    untouched = row_req == 1
    assert got[untouched].tobytes() == h[untouched].tobytes()


# C / 4 dividing 64 takes the one-vector-per-thread kernel (C = 8, 64, 256),
# the others the wave-per-token kernel (C = 200, 512)
@pytest.mark.parametrize("C,mode", [(64, L.ALD_STEER_ADD), (64, L.ALD_STEER_PROJECT), (8, L.ALD_STEER_PROJECT),
                                    (256, L.ALD_STEER_PROJECT), (200, L.ALD_STEER_ADD), (512, L.ALD_STEER_PROJECT)])
def test_steer_latent(C, mode):
    """Latent-site steering: a steered fp32 copy of the latent; tokens of a
    zero-strength request are copied bit for bit, the others agree with the
    oracle after the fp16 rounding the model input gets (one fp32 FMA per
    value before it, so at most one fp16 step apart)."""
    r = rng(10 + C)
    lens = np.array([37, 0, 300, 129])
    n, R = int(lens.sum()), len(lens)
    x = r.standard_normal((n, C)).astype(np.float32)
    d = r.standard_normal(C)
    d = (d / np.linalg.norm(d)).astype(np.float32)
    alpha = np.array([0.5, 0.25, 0.0, -1.5], np.float32)
    row_req = np.repeat(np.arange(R), lens).astype(np.int32)
    got = host(B.steer_latent(dev(x), dev(alpha), 7.5, dev(d), row_req=dev(row_req), mode=mode))
    mname = "project" if mode == L.ALD_STEER_PROJECT else "add"
    ref = O.steer_latent(x, alpha[row_req], 7.5, d, mode=mname)
    zero = alpha[row_req] == 0
    assert got[zero].tobytes() == x[zero].tobytes()
    g16 = got.astype(np.float16).astype(np.float64)
    r16 = ref.astype(np.float64)
    ulp = np.spacing(np.abs(ref)).astype(np.float64)
    assert np.all(np.abs(g16 - r16) <= ulp * 1.0001 + 2.0 ** -24)
    # dense mapping (rows_per_req) gives the same result as the explicit map
    dense = host(B.steer_latent(dev(x[:300]), dev(alpha[:3]), 7.5, dev(d), rows_per_req=100, R=3, mode=mode))
    assert dense.tobytes() == host(B.steer_latent(dev(x[:300]), dev(alpha[:3]), 7.5, dev(d),
                                                  row_req=dev((np.arange(300) // 100).astype(np.int32)),
                                                  mode=mode)).tobytes()


@pytest.mark.parametrize("a,an", [(0.3, 0.55), (4.04e-5, 5.2e-5), (0.9999, 1.0)])
def test_ddim_sampler_ops(a, an):
    """DDIM update and its warm-start re-noise against the oracle (fp64), per
    request alpha_bar; an inactive request keeps its latent bit for bit.  The
    fp32 update divides by sqrt(a): the bar scales with 1 / sqrt(a)."""
    r = rng(31)
    R, S, C = 3, 70, 64
    n = R * S
    x = r.standard_normal((n, C)).astype(np.float32)
    e = r.standard_normal((n, C)).astype(np.float32)
    x0 = r.standard_normal((n, C)).astype(np.float32)
    ab = np.array([a, a, 0.5], np.float32)
    abn = np.array([an, an, 0.7], np.float32)
    active = np.array([1, 1, 0], np.uint8)
    req = np.arange(n) // S
    xd = dev(x)
    B.sampler_update(L.ALD_DDIM, xd, dev(ab), dev(abn), v_hat=dev(e), rows_per_req=S, active=dev(active))
    got = host(xd)
    on = req < 2
    ref = O.ddim_update(x[on], e[on], ab[req[on]][:, None], abn[req[on]][:, None])
    err = np.max(np.abs(got[on].astype(np.float64) - ref)) / np.max(np.abs(ref))
    assert err < 2e-6 / np.sqrt(a), err
    assert got[~on].tobytes() == x[~on].tobytes()
    xd = dev(x)
    B.sampler_update(L.ALD_RENOISE_VP, xd, dev(ab), x0=dev(x0), eps=dev(e), rows_per_req=S, active=dev(active))
    got = host(xd)
    ref = O.renoise_vp(x0[on], e[on], ab[req[on]][:, None])
    assert np.max(np.abs(got[on].astype(np.float64) - ref)) < 1e-6
    assert got[~on].tobytes() == x[~on].tobytes()


def test_cfg_merge_and_sampler():
    r = rng(9)
    R, S, C = 3, 50, 64
    n = R * S
    v = r.standard_normal((2 * n, C)).astype(np.float16)
    w = np.array([3.0, 1.0, 0.0], np.float32)
    vh = host(B.cfg_merge(dev(v), dev(w), rows_per_req=S))
    req = np.arange(n) // S
    ref = O.cfg_merge(v[:n], v[n:], w[req][:, None])
    assert np.allclose(vh, ref, rtol=1e-6, atol=1e-6)
    assert np.array_equal(vh[req == 1], v[:n][req == 1].astype(np.float32))   # w = 1: cond branch
    assert np.array_equal(vh[req == 2], v[n:][req == 2].astype(np.float32))   # w = 0: uncond branch
    x = r.standard_normal((n, C)).astype(np.float32)
    tc = np.array([1.0, 0.5, 0.25], np.float32)
    tn = np.array([0.875, 0.375, 0.0], np.float32)
    act = np.array([1, 0, 1], np.uint8)
    xt = dev(x)
    B.sampler_update(L.ALD_EULER, xt, dev(tc), dev(tn), v_hat=dev(ref), rows_per_req=S, active=dev(act))
    xe = O.euler_update(x, ref, tc[req][:, None], tn[req][:, None])
    xe[req == 1] = x[req == 1]
    assert np.allclose(host(xt), xe, rtol=1e-6, atol=1e-6)
    x0 = r.standard_normal((n, C)).astype(np.float32)
    eps = r.standard_normal((n, C)).astype(np.float32)
    tt = np.array([0.0, 1.0, 0.4375], np.float32)
    xt = dev(x)
    B.sampler_update(L.ALD_RENOISE, xt, dev(tt), x0=dev(x0), eps=dev(eps), rows_per_req=S)
    got = host(xt)
    assert np.array_equal(got[req == 0], x0[req == 0])      # t = 0: the cached latent
    assert np.array_equal(got[req == 1], eps[req == 1])     # t = 1: pure noise
    assert np.allclose(got, O.renoise(x0, eps, tt[req][:, None]), rtol=1e-6, atol=1e-6)
