"""Pins of the oracle's quantizers and integer GEMM (CPU only).

The pages give 8-bit weights, W8A8 arithmetic and 4-bit storage (aria,
Section III-A) but no quantizer formula and no worked values; the pins are
hand-derived closed forms (tests/golden), brute force, and error bounds that
hold for any correct symmetric round-to-nearest quantizer.
"""
import json
import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import ald_oracle as O

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


def test_q8_hand_cases():
    for case in _load("q8_ties.json")["cases"]:
        u = np.array([case["u"]], dtype=np.float16)
        q, s = O.quantize_rows_q8(u)
        assert q.dtype == np.int8
        assert q[0].tolist() == case["codes"], case["why"]
        assert float(s[0]) == pytest.approx(case["scale"], rel=0, abs=0), case["why"]


def test_q8_scale_is_fp32_quotient():
    # s must be the correctly rounded fp32 value of amax / 127 (exact rational check)
    rng = np.random.default_rng(5)
    u = rng.standard_normal((64, 96)).astype(np.float16)
    _, s = O.quantize_rows_q8(u)
    for i in range(u.shape[0]):
        amax = Fraction(float(np.max(np.abs(u[i].astype(np.float64)))))
        exact = amax / 127
        got = Fraction(float(s[i]))
        # nearest fp32: neighbours are further away
        up = Fraction(float(np.nextafter(np.float32(s[i]), np.float32(np.inf))))
        dn = Fraction(float(np.nextafter(np.float32(s[i]), np.float32(-np.inf))))
        assert abs(got - exact) <= abs(up - exact) and abs(got - exact) <= abs(dn - exact)


def test_q8_round_to_nearest_bound_and_range():
    rng = np.random.default_rng(1)
    u = (rng.standard_normal((200, 257)) * rng.uniform(0.01, 50, size=(200, 1))).astype(np.float16)
    u[3] = 0
    u[7, :] = np.float16(-3.0)
    q, s = O.quantize_rows_q8(u)
    uf = u.astype(np.float64)
    amax = np.max(np.abs(uf), axis=1)
    for i in range(u.shape[0]):
        if amax[i] == 0:
            assert s[i] == 0 and not q[i].any()
            continue
        # codes are the nearest integers to 127 u / amax (up to fp32 rounding of the product)
        ideal = 127.0 * uf[i] / amax[i]
        assert np.all(np.abs(q[i] - ideal) <= 0.5 + 1e-4)
        assert np.max(np.abs(q[i])) == 127          # the amax element saturates exactly
        assert np.all(np.abs(q[i]) <= 127)
        assert np.all(np.sign(q[i]) * np.sign(uf[i]) >= 0)
        # monotone in u
        order = np.argsort(uf[i], kind="stable")
        assert np.all(np.diff(q[i][order].astype(np.int64)) >= 0)
        # |u - q s| <= s / 2 (plus fp32 slack)
        err = np.abs(uf[i] - q[i] * float(s[i]))
        assert np.all(err <= 0.5 * float(s[i]) * (1 + 1e-5) + 1e-12)


def test_int_gemm_brute_force():
    rng = np.random.default_rng(2)
    for (M, N, K) in [(1, 1, 1), (3, 5, 7), (17, 9, 64), (5, 33, 130)]:
        a = rng.integers(-127, 128, size=(M, K)).astype(np.int8)
        b = rng.integers(-127, 128, size=(N, K)).astype(np.int8)
        acc = O.int_gemm(a, b)
        for m in range(M):
            for n in range(N):
                ref = 0
                for k in range(K):
                    ref += int(a[m, k]) * int(b[n, k])
                assert acc[m, n] == ref


def test_int_gemm_extremes_exact():
    K = 8192
    a = np.full((2, K), 127, np.int8)
    a[1] = -127
    b = np.full((3, K), 127, np.int8)
    b[1] = -127
    b[2, ::2] = -127
    acc = O.int_gemm(a, b)
    assert acc[0, 0] == K * 127 * 127
    assert acc[1, 0] == -K * 127 * 127
    assert acc[0, 1] == -K * 127 * 127
    assert acc[0, 2] == 0


def test_w8a8_error_bound_and_orientation():
    rng = np.random.default_rng(3)
    M, K, N = 24, 192, 40
    x = rng.standard_normal((M, K)).astype(np.float16)
    w = (0.02 * rng.standard_normal((N, K))).astype(np.float16)
    b = (0.02 * rng.standard_normal(N)).astype(np.float32)
    wq, ws = O.quantize_rows_q8(w)
    r = O.w8a8_linear(x, wq, ws, b)
    xf, wf = x.astype(np.float64), w.astype(np.float64)
    exact = xf @ wf.T + b
    bound = (np.abs(xf) @ (np.ones_like(wf) * ws[:, None] / 2).T
             + (np.ones_like(xf) * r.x_scale[:, None] / 2) @ np.abs(wf).T
             + K * (r.x_scale[:, None] * ws[None, :]) / 4)
    fp16_round = np.abs(exact) * 2.0 ** -11 + 2.0 ** -24
    assert np.all(np.abs(r.y.astype(np.float64) - exact) <= bound * 1.0001 + fp16_round * 1.01)
    # the raw accumulators are the integer products of the codes
    assert np.array_equal(r.acc, O.int_gemm(r.xq, wq))


def test_w8a8_residual_and_gelu():
    rng = np.random.default_rng(4)
    x = rng.standard_normal((8, 64)).astype(np.float16)
    w = (0.05 * rng.standard_normal((16, 64))).astype(np.float16)
    res = rng.standard_normal((8, 16)).astype(np.float16)
    wq, ws = O.quantize_rows_q8(w)
    base = O.w8a8_linear(x, wq, ws, None)
    deq = base.acc * base.x_scale[:, None].astype(np.float64) * ws[None, :].astype(np.float64)
    withres = O.w8a8_linear(x, wq, ws, None, residual=res).y.astype(np.float64)
    assert np.allclose(withres, deq + res.astype(np.float64), atol=2e-3, rtol=2e-3)
    gl = O.w8a8_linear(x, wq, ws, None, act=1).y.astype(np.float64)
    from math import erf, sqrt
    ref = np.vectorize(lambda v: 0.5 * v * (1 + erf(v / sqrt(2))))(deq)
    assert np.allclose(gl, ref, atol=1e-3, rtol=1e-3)


def test_q4_pack_fixture():
    g = _load("q4_pack.json")
    for case in g["pack_cases"]:
        codes = np.array(case["codes"], dtype=np.int64)
        # build a row whose quantization yields exactly these codes: s = 1 needs amax 7
        row = codes.astype(np.float16)
        row = np.concatenate([row, np.zeros(32 - len(row), np.float16)])
        row[-1] = np.float16(7.0)  # amax 7 -> s = 1
        packed, s = O.quantize_q4(row[None, :])
        assert float(s[0, 0]) == 1.0
        assert packed[0, :len(case["bytes"])].tolist() == case["bytes"], case["why"]
        assert O.unpack_q4(packed)[0, :len(codes)].tolist() == codes.tolist()
    rc = g["reconstruct_case"]
    w = (np.array(rc["codes"], np.float64) * rc["s"]).astype(np.float16)[None, :]
    packed, s = O.quantize_q4(w)
    assert float(s[0, 0]) == rc["s"]
    assert O.unpack_q4(packed)[0].tolist() == rc["codes"]
    assert np.array_equal(O.dequantize_q4(packed, s), w)


def test_q4_error_bound():
    rng = np.random.default_rng(6)
    N, K = 48, 256
    w = (0.02 * rng.standard_normal((N, K))).astype(np.float16)
    w[5, 32:64] = 0
    packed, s = O.quantize_q4(w)
    codes = O.unpack_q4(packed).astype(np.int64)
    assert codes.min() >= -7 and codes.max() <= 7
    deq = O.dequantize_q4(packed, s).astype(np.float64)
    wf = w.astype(np.float64)
    s_el = np.repeat(s.astype(np.float64), 32, axis=1)
    # fp16 ulp of the largest dequantized magnitude in the group (7 s)
    ulp = np.repeat(np.array([[np.spacing(np.float16(7 * v)) for v in row] for row in s.astype(np.float32)],
                             dtype=np.float64), 32, axis=1)
    assert np.all(np.abs(wf - deq) <= s_el / 2 * (1 + 1e-6) + ulp / 2 + 1e-12)
    assert not codes[5, 32:64].any() and s[5, 1] == 0
    # the group's extreme saturates at +-7 and amax/7 is the (fp16-rounded) scale
    amax = np.max(np.abs(wf.reshape(N, K // 32, 32)), axis=2)
    assert np.allclose(s.astype(np.float64), amax / 7, rtol=2 ** -10)


def test_planted_rounding_mistake_is_caught(monkeypatch):
    """A quantizer that truncates instead of rounding half-even must fail the tie pin."""
    real = O.quantize_rows_q8

    def trunc(u16):
        u = np.asarray(u16, np.float16).astype(np.float32)
        amax = np.max(np.abs(u), axis=1).astype(np.float32)
        inv = np.where(amax > 0, np.float32(127) / np.where(amax > 0, amax, 1), 0).astype(np.float32)
        return np.clip(np.trunc(u * inv[:, None]), -127, 127).astype(np.int8), (amax / np.float32(127)).astype(np.float32)

    monkeypatch.setattr(O, "quantize_rows_q8", trunc)
    with pytest.raises(AssertionError):
        test_q8_hand_cases()
    monkeypatch.setattr(O, "quantize_rows_q8", real)
    test_q8_hand_cases()


def test_q8w_brute_force_exact():
    """8-bit weight-only linear against a plain triple loop; operands chosen so
    every product and sum is exact in fp64 and the fp16 result is exact too,
    with a distinct power-of-two scale per output channel (a scale applied
    along the wrong axis, or a transposed weight, changes the result)."""
    rng = np.random.default_rng(11)
    M, K, N = 5, 64, 7
    x = (rng.integers(-8, 9, size=(M, K)) / 4).astype(np.float16)
    q = rng.integers(-127, 128, size=(N, K)).astype(np.int8)
    s = (2.0 ** -rng.integers(4, 9, size=N)).astype(np.float32)
    b = (rng.integers(-4, 5, size=N) / 8).astype(np.float32)
    y = O.q8w_linear(x, q, s, b)
    for m in range(M):
        for n in range(N):
            acc = Fraction(0)
            for k in range(K):
                acc += Fraction(float(x[m, k])) * int(q[n, k]) * Fraction(float(s[n]))
            acc += Fraction(float(b[n]))
            assert float(y[m, n]) == float(np.float16(float(acc))), (m, n)


def test_q8w_error_bound_vs_unquantized_weight():
    """With the weight's own per-channel q8 quantization, the result stays
    within the quantizer's half-step bound of the fp16-weight product."""
    rng = np.random.default_rng(12)
    M, K, N = 16, 256, 48
    x = rng.standard_normal((M, K)).astype(np.float16)
    w = (0.02 * rng.standard_normal((N, K))).astype(np.float16)
    q, s = O.quantize_rows_q8(w)
    y = O.q8w_linear(x, q, s).astype(np.float64)
    exact = x.astype(np.float64) @ w.astype(np.float64).T
    bound = np.abs(x.astype(np.float64)).sum(axis=1)[:, None] * s.astype(np.float64)[None, :] / 2
    fp16_round = np.abs(exact) * 2.0 ** -11 + 2.0 ** -24
    assert np.all(np.abs(y - exact) <= bound * 1.0001 + fp16_round * 1.01)
    # the weight-only arm is strictly closer than W8A8, which also rounds x
    w8 = O.w8a8_linear(x, q, s).y.astype(np.float64)
    assert np.abs(y - exact).mean() < np.abs(w8 - exact).mean()


def test_q8w_residual_and_gelu():
    rng = np.random.default_rng(13)
    x = rng.standard_normal((6, 64)).astype(np.float16)
    q = rng.integers(-127, 128, size=(10, 64)).astype(np.int8)
    s = (0.001 * (1 + rng.random(10))).astype(np.float32)
    res = rng.standard_normal((6, 10)).astype(np.float16)
    lin = x.astype(np.float64) @ (q.astype(np.float64) * s.astype(np.float64)[:, None]).T
    got = O.q8w_linear(x, q, s, residual=res).astype(np.float64)
    assert np.allclose(got, lin + res.astype(np.float64), atol=2e-3, rtol=2e-3)
    from math import erf, sqrt
    ref = np.vectorize(lambda v: 0.5 * v * (1 + erf(v / sqrt(2))))(lin)
    assert np.allclose(O.q8w_linear(x, q, s, act=1).astype(np.float64), ref, atol=1e-3, rtol=1e-3)


def _exact_linear(x, w, b=None, res=None):
    """fp16(sum_k x[m, k] w[n, k] + b[n] + res[m, n]) from exact rational
    arithmetic on the given operand values (a plain triple loop)."""
    M, K = x.shape
    N = w.shape[0]
    out = np.empty((M, N), np.float16)
    for m in range(M):
        for n in range(N):
            acc = Fraction(0)
            for k in range(K):
                acc += Fraction(float(x[m, k])) * Fraction(float(w[n, k]))
            if b is not None:
                acc += Fraction(float(b[n]))
            if res is not None:
                acc += Fraction(float(res[m, n]))
            out[m, n] = np.float16(float(acc))  # acc is a short dyadic rational: float() is exact
    return out


@pytest.mark.parametrize("N", [48, 5])
def test_f16_linear_brute_force_exact(N):
    """fp16-weight linear against a plain triple loop, on a square (N = K) and
    a non-square weight.  Dyadic operands keep every product and sum exact, so
    the result must equal the exact value rounded once to fp16; the square
    weight is far from symmetric, so x . W (no transpose) fails."""
    rng = np.random.default_rng(21)
    M, K = 6, 48
    x = (rng.integers(-16, 17, size=(M, K)) / 8).astype(np.float16)
    w = (rng.integers(-64, 65, size=(N, K)) / 256).astype(np.float16)
    b = (rng.integers(-8, 9, size=N) / 16).astype(np.float32)
    res = (rng.integers(-8, 9, size=(M, N)) / 4).astype(np.float16)
    if N == K:
        assert np.abs(w.astype(np.float64) - w.astype(np.float64).T).max() > 0.1
        assert not np.array_equal(O.f16_linear(x, w), O.f16_linear(x, w.T.copy()))
    assert np.array_equal(O.f16_linear(x, w, b), _exact_linear(x, w, b))
    assert np.array_equal(O.f16_linear(x, w, b, residual=res), _exact_linear(x, w, b, res))
    assert np.array_equal(O.f16_linear(x, w), _exact_linear(x, w))


def _pack_nibbles(codes):
    """Two's-complement nibbles by hand: byte j holds k = 2j low, 2j + 1 high."""
    c = np.asarray(codes, np.int64) & 0xF
    return (c[:, 0::2] | (c[:, 1::2] << 4)).astype(np.uint8)


@pytest.mark.parametrize("N", [64, 9])
def test_q4_linear_brute_force_exact(N):
    """4-bit-weight linear against a plain triple loop over the weight each
    code and its group's scale stand for (q * s, exact here: powers of two),
    on a square (N = K) and a non-square weight.  Every group of 32 along K has
    its own scale, so a scale read from the wrong group or channel, a nibble
    order swap or a transposed weight changes the result."""
    rng = np.random.default_rng(22)
    M, K = 5, 64
    codes = rng.integers(-7, 8, size=(N, K))
    scales = (2.0 ** -rng.integers(3, 9, size=(N, K // 32))).astype(np.float16)
    assert (scales[:, 0] != scales[:, 1]).any()
    packed = _pack_nibbles(codes)
    w_eff = (codes * np.repeat(scales.astype(np.float64), 32, axis=1)).astype(np.float16)
    x = (rng.integers(-16, 17, size=(M, K)) / 8).astype(np.float16)
    b = (rng.integers(-8, 9, size=N) / 16).astype(np.float32)
    assert np.array_equal(O.q4_linear(x, packed, scales, b), _exact_linear(x, w_eff, b))
    # swapped nibbles (k = 2j in the high half) would give another result
    swapped = ((packed >> 4) | (packed << 4)).astype(np.uint8)
    assert not np.array_equal(O.q4_linear(x, swapped, scales, b), _exact_linear(x, w_eff, b))


def test_prepared_linear_modes_route_to_their_own_linear():
    """Each weight mode of a prepared linear computes its own arithmetic:
    W8A8 = exact product of both operands' q8 values; W8A16 = fp16 x times
    the weight's q8 values; q4 = fp16 x times the 4-bit values; f16 = the
    plain fp16 product (each against the brute-force loop), and the four
    results differ pairwise, so a mode routed to another's linear fails."""
    rng = np.random.default_rng(23)
    M, K, N = 4, 64, 6
    x = rng.standard_normal((M, K)).astype(np.float16)
    w = (0.05 * rng.standard_normal((N, K))).astype(np.float16)
    b = (0.02 * rng.standard_normal(N)).astype(np.float32)
    xq, xs = O.quantize_rows_q8(x)
    wq, ws = O.quantize_rows_q8(w)
    q4p, q4s = O.quantize_q4(w)

    def deq(q, s):
        return (q.astype(np.float64) * s.astype(np.float64)[:, None])

    def exact(xv, wv):  # exact sum, then one rounding; operands as fp64 values
        out = np.empty((M, N), np.float16)
        for m in range(M):
            for n in range(N):
                acc = sum((Fraction(float(xv[m, k])) * Fraction(float(wv[n, k])) for k in range(K)), Fraction(0))
                acc += Fraction(float(b[n]))
                out[m, n] = np.float16(float(acc))
        return out

    want = {"f16": exact(x.astype(np.float64), w.astype(np.float64)),
            "w8a16": exact(x.astype(np.float64), deq(wq, ws)),
            "q4": exact(x.astype(np.float64), O.dequantize_q4(q4p, q4s).astype(np.float64)),
            "w8a8": exact(deq(xq, xs), deq(wq, ws))}
    got = {mode: O.prepare_linear(w, b, mode)(x) for mode in want}
    for mode in want:
        # fp64 evaluation of the exact sum may differ from it in the last bits,
        # so allow one fp16 ulp where rounding sits on a tie
        d = np.abs(got[mode].astype(np.float64) - want[mode].astype(np.float64))
        assert np.all(d <= np.spacing(np.abs(want[mode])).astype(np.float64)), mode
    modes = list(want)
    for i in range(len(modes)):
        for j in range(i + 1, len(modes)):
            assert not np.array_equal(got[modes[i]], got[modes[j]]), (modes[i], modes[j])


def test_prepared_linear_dispatch_calls(monkeypatch):
    """The mode dispatch itself: each mode calls its own linear with that
    mode's packed operands (and the residual and activation passed through)."""
    calls = []
    for name in ("w8a8_linear", "q4_linear", "q8w_linear", "f16_linear"):
        def rec(*a, _n=name, **k):
            calls.append((_n, a, k))
            return O.W8A8Result(np.zeros(1), None, None, None) if _n == "w8a8_linear" else np.zeros(1)
        monkeypatch.setattr(O, name, rec)
    rng = np.random.default_rng(24)
    w = (0.05 * rng.standard_normal((4, 64))).astype(np.float16)
    b = np.zeros(4, np.float32)
    x = rng.standard_normal((2, 64)).astype(np.float16)
    r = rng.standard_normal((2, 4)).astype(np.float16)
    expect = {"w8a8": "w8a8_linear", "w8a16": "q8w_linear", "q4": "q4_linear", "f16": "f16_linear"}
    for mode, fn in expect.items():
        p = O.prepare_linear(w, b, mode)
        calls.clear()
        p(x, residual=r, act=1)
        assert len(calls) == 1 and calls[0][0] == fn, (mode, calls)
        args = calls[0][1]
        if mode in ("w8a8", "w8a16"):
            assert args[1] is p.wq and args[2] is p.ws
        elif mode == "q4":
            assert args[1] is p.q4 and args[2] is p.q4s
        else:
            assert args[1] is p.w16
        assert args[-2] is r and args[-1] == 1


def test_planted_linear_mistakes_are_caught(monkeypatch):
    """An f16 linear without the transpose, and a q4 mode that computes the
    fp16 weights instead of the 4-bit ones, must each fail a pin above."""
    real_f16 = O.f16_linear

    def no_transpose(x16, w16, bias=None, residual=None, act=0):
        y64 = np.asarray(x16, np.float16).astype(np.float64) @ np.asarray(w16, np.float16).astype(np.float64)
        return O._epilogue(y64, bias, residual, act)

    monkeypatch.setattr(O, "f16_linear", no_transpose)
    with pytest.raises(AssertionError):
        test_f16_linear_brute_force_exact(48)
    monkeypatch.setattr(O, "f16_linear", real_f16)

    def q4_as_f16(self, x16, residual=None, act=0):
        if self.mode == "q4":
            return real_f16(x16, self.w16, self.bias, residual, act)
        return real_call(self, x16, residual, act)

    real_call = O.PreparedLinear.__call__
    monkeypatch.setattr(O.PreparedLinear, "__call__", q4_as_f16)
    with pytest.raises(AssertionError):
        test_prepared_linear_modes_route_to_their_own_linear()
