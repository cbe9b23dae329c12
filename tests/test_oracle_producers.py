"""Pins of the producer oracle (RMSNorm / SwiGLU + int8 plane) against facts
that do not come from the oracle itself: exact invariances, closed forms,
values of the logistic function, and an exact rational evaluation of the sum
of squares."""
from fractions import Fraction
import math

import numpy as np
import pytest

import oracle
from oracle import producers


def _rows(seed, M, K, scale=1.0):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((M, K)) * scale).astype(np.float32)


# ---------------------------------------------------------------- RMSNorm

def test_rmsnorm_power_of_two_scaling_is_exact():
    """With eps = 0, multiplying a row by 2^k multiplies ss by 4^k, sqrt by
    2^k and r by 2^-k, all exactly: y does not change by a single bit."""
    x = _rows(1, 6, 512)
    w = _rows(2, 1, 512)[0]
    y0, r0 = producers.rmsnorm(x, w, 0.0)
    for k in (-20, -3, 7, 30):
        yk, rk = producers.rmsnorm(x * np.float32(2.0 ** k), w, 0.0)
        assert np.array_equal(yk, y0)
        assert np.array_equal(rk, r0 * np.float32(2.0 ** -k))


def test_rmsnorm_unit_rms_and_closed_form():
    """w = 1, eps = 0: every output row has root-mean-square 1 (to f32
    rounding); a constant row c maps to sign(c)."""
    x = _rows(3, 5, 1024, scale=3.0)
    y, _ = producers.rmsnorm(x, np.ones(1024, np.float32), 0.0)
    rms = np.sqrt((y.astype(np.float64) ** 2).mean(axis=1))
    assert np.all(np.abs(rms - 1.0) < 2e-7)
    for c in (0.37, -5.5, 1e-20, 3e19):
        yc, _ = producers.rmsnorm(np.full((1, 256), c, np.float32), np.ones(256, np.float32), 0.0)
        assert np.all(np.abs(yc - np.sign(c)) <= 2.0 ** -23)


def test_rmsnorm_eps_and_zero_row():
    """An all-zero row gives y = 0 and r = 1/sqrt(eps); a row far below
    sqrt(eps) is scaled by about 1/sqrt(eps)."""
    w = _rows(4, 1, 256)[0]
    y, r = producers.rmsnorm(np.zeros((1, 256), np.float32), w, 1e-6)
    assert not y.any()
    assert r[0] == np.float32(1.0 / math.sqrt(float(np.float32(1e-6))))
    x = _rows(5, 1, 256, scale=1e-9)
    y, r = producers.rmsnorm(x, np.ones(256, np.float32), 1e-6)
    assert abs(float(r[0]) * math.sqrt(1e-6) - 1.0) < 1e-6


def test_rmsnorm_weight_scales_exactly():
    x = _rows(6, 3, 512)
    w = _rows(7, 1, 512)[0]
    y1, _ = producers.rmsnorm(x, w, 1e-5)
    y2, _ = producers.rmsnorm(x, w * np.float32(8.0), 1e-5)
    assert np.array_equal(y2, y1 * np.float32(8.0))


def test_rmsnorm_sum_is_exact():
    """The scale comes from the exact sum of squares: the same r as an exact
    rational evaluation rounded once, including rows where a plain f64
    running sum drops the small terms."""
    K = 1024
    x = _rows(8, 4, K)
    x[3] = np.float32(2.0 ** -27)
    x[3, 0] = np.float32(1.0)                      # 1 + 1023 * 2^-54: lost by a running f64 sum
    eps = 1e-6
    _, r = producers.rmsnorm(x, np.ones(K, np.float32), eps)
    for t in range(x.shape[0]):
        exact = sum((Fraction(float(v)) ** 2 for v in x[t]), Fraction(0))
        r_exact = np.float32(1.0 / math.sqrt(float(exact) / K + float(np.float32(eps))))
        assert r[t] == r_exact
    running = 0.0
    for v in x[3].astype(np.float64):
        running += v * v
    assert running == 1.0 and float(sum((Fraction(float(v)) ** 2 for v in x[3]), Fraction(0))) > 1.0


def test_rmsnorm_matches_f64_definition():
    """Against the definition evaluated directly in f64: within 2 f32 ulps."""
    x = _rows(9, 7, 768, scale=2.0)
    w = _rows(10, 1, 768)[0]
    y, _ = producers.rmsnorm(x, w, 1e-6)
    x64 = x.astype(np.float64)
    ref = x64 / np.sqrt((x64 ** 2).mean(axis=1, keepdims=True) + 1e-6) * w.astype(np.float64)
    assert np.all(np.abs(y - ref) <= 2.5 * np.spacing(np.abs(ref).astype(np.float32)))


# ---------------------------------------------------------------- SwiGLU

def test_silu_known_values():
    """SiLU(0) = 0; SiLU(1) is the logistic function at 1, 1/(1 + 1/e)."""
    y = producers.swiglu(np.array([0.0, 1.0, -1.0], np.float32), np.ones(3, np.float32))
    assert y[0] == 0.0
    assert y[1] == np.float32(0.7310585786300049)
    assert y[2] == np.float32(-0.2689414213699951)


def test_silu_odd_part_identity():
    """SiLU(g) - SiLU(-g) = g (since sigma(g) + sigma(-g) = 1)."""
    g = np.random.default_rng(11).standard_normal(4096).astype(np.float32) * np.float32(6.0)
    one = np.ones_like(g)
    diff = producers.swiglu(g, one).astype(np.float64) - producers.swiglu(-g, one).astype(np.float64)
    assert np.all(np.abs(diff - g) <= 2.0 * np.spacing(np.abs(g)) + 1e-30)


def test_silu_tails_and_sign():
    one = np.ones(4, np.float32)
    big = producers.swiglu(np.array([30.0, 60.0, 100.0, 1e30], np.float32), one)
    assert np.array_equal(big, np.array([30.0, 60.0, 100.0, 1e30], np.float32))
    neg = producers.swiglu(np.array([-30.0, -60.0, -100.0, -1e30], np.float32), one)
    assert np.all(neg <= 0.0) and np.all(np.abs(neg) < 3e-12)
    # minimum of SiLU is about -0.278 at g about -1.278
    g = np.linspace(-6, 6, 20001, dtype=np.float32)
    s = producers.swiglu(g, np.ones_like(g))
    assert abs(float(s.min()) + 0.27846454) < 1e-6


def test_swiglu_scales_with_up_exactly():
    rng = np.random.default_rng(12)
    g = rng.standard_normal(2048).astype(np.float32)
    u = rng.standard_normal(2048).astype(np.float32)
    assert np.array_equal(producers.swiglu(g, u * np.float32(4.0)), producers.swiglu(g, u) * np.float32(4.0))


def test_silu_matches_math_exp():
    """Element by element against Python's math.exp (a different exp): the
    f32 results agree bit for bit on a spread of inputs."""
    g = np.random.default_rng(13).standard_normal(3000).astype(np.float32) * np.float32(5.0)
    s = producers.swiglu(g, np.ones_like(g))
    ref = np.array([np.float32(float(v) / (1.0 + math.exp(-float(v)))) for v in g], np.float32)
    assert np.array_equal(s, ref)


# ---------------------------------------------------------------- planes

@pytest.mark.parametrize("which", ["rmsnorm", "swiglu"])
def test_plane_is_quantizer_of_producer_output(which):
    rng = np.random.default_rng(14)
    if which == "rmsnorm":
        x = rng.standard_normal((9, 512)).astype(np.float32)
        w = rng.standard_normal(512).astype(np.float32)
        q, d, s, y = producers.rmsnorm_quantize(x, w, 1e-6)
    else:
        g = rng.standard_normal((9, 512)).astype(np.float32)
        u = rng.standard_normal((9, 512)).astype(np.float32)
        q, d, s, y = producers.swiglu_quantize(g, u)
    q2, d2, s2 = oracle.quantize_act(y)
    assert np.array_equal(q, q2) and np.array_equal(d, d2) and np.array_equal(s, s2)
    # |y - d*q| <= d/2 (plus the division's rounding) in every block
    dq = (q.astype(np.float64).reshape(9, -1, 32) * d.astype(np.float64)[:, :, None]).reshape(9, 512)
    assert np.all(np.abs(y - dq) <= np.repeat(d, 32, axis=1) * (0.5 + 2 ** -16))


# ---------------------------------------------------------------- fused FFN composition

def _const_q4k_rows(N, K, value):
    """N rows of K Q4_K weights that all dequantize to the integer `value`
    exactly: value >= 0 through d = 1, sc = value, q4 = 1, dmin = 0;
    value < 0 through the min term alone (q4 = 0, dmin = 1, m = -value)."""
    from blocks import q4k_pack
    if value >= 0:
        blk = q4k_pack(1.0, 0.0, [value] * 8, [0] * 8, np.ones(256, np.int64))
    else:
        blk = q4k_pack(1.0, 1.0, [1] * 8, [-value] * 8, np.zeros(256, np.int64))
    return np.tile(blk, (N, K // 256)).reshape(N, (K // 256) * 144)


@pytest.mark.parametrize("gate,up", [(-30, 1), (2, -3), (5, 7)])
def test_ffn_applies_silu_to_the_gate_matrix(gate, up):
    """FusedFFN is SwiGLU(gate, up) = SiLU(x Wg^T) * (x Wu^T) (minfer Compute
    Graph Design, "The Op vocabulary"). Token 0's plane is q = (127, -126, 0,
    ...) with d = 1 (so its activation sum is 1) and token 1 is all zero:
    with Wg and Wu dequantizing to the constants `gate` and `up`, g = gate and
    u = up exactly, so y = SiLU(gate) * up from the logistic function alone.
    SiLU is not symmetric in its arguments, so a composition that swaps the
    two matrices gives SiLU(up) * gate, far from it (gate = -30, up = 1:
    -2.8e-12 against -21.9)."""
    N, K = 256, 512                    # N is the down projection's K: whole 32-blocks
    Wg, Wu = _const_q4k_rows(N, K, gate), _const_q4k_rows(N, K, up)
    x = np.zeros((2, K), np.float32)
    x[0, 0], x[0, 1] = 127.0, -126.0
    q, d, _ = oracle.quantize_act(x)
    assert q[0, 0] == 127 and q[0, 1] == -126 and d[0, 0] == 1.0 and not q[1].any()
    qo, do, so, y = producers.ffn_q4k(Wg, Wu, q, d, N, K)
    silu = lambda v: v / (1.0 + math.exp(-v))
    want = silu(gate) * up
    swapped = silu(up) * gate
    assert np.allclose(y[0], want, rtol=1e-6, atol=0.0), (y[0], want)
    assert abs(want - swapped) > 1e-3 * max(abs(want), abs(swapped))
    assert not np.allclose(y[0], swapped, rtol=1e-3, atol=0.0)
    assert np.all(y[1] == 0.0)
    # the plane of a constant row: every q is +-127 and d = |y| / 127
    assert np.all(qo[0] == (127 if want > 0 else -127)) and not qo[1].any()
    assert np.array_equal(do[0], np.full(N // 32, np.float32(abs(y[0, 0])) / np.float32(127)))
    assert not do[1].any() and not so[1].any()
