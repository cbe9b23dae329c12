"""Oracle of the producer-fused activation quantizers: RMSNorm and SwiGLU
followed by the per-32 int8 activation quantizer.

TEST INFRASTRUCTURE ONLY: the tests, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` use it. The product library and its binding
never import it.

What is computed. The pages have the producers of the matmul inputs, the
RMS normalisation and the SwiGLU epilogue, write the int8 activation plane
directly instead of an f32 tensor (minfer Features, "GPU — CUDA"). The two
producers are the graph ops RmsNorm{eps} and SwiGLU = Silu(gate) * up (minfer
Compute Graph Design, "The Op vocabulary"). The pages give no arithmetic for
either; the readings taken here, written out step by step, are:

  RMSNorm of a row x[0..K) with weight w and eps:
    ss = sum_k x_k^2, the exact real sum rounded once to f64 (each x_k^2 is
         exact in f64; math.fsum returns the correctly rounded sum);
    r  = 1 / sqrt(ss / K + eps), three correctly rounded f64 operations,
         then rounded to f32;
    y_k = (x_k * r) * w_k, two f32 products.
  SwiGLU of gate g and up u:
    s_k = g_k / (1 + exp(-g_k)) evaluated in f64, rounded to f32;
    y_k = s_k * u_k, one f32 product.

The plane is then ``oracle.quantize_act(y)``: the quantizer whose rules are
pinned on their own. The f64 steps make the f32 result depend on nothing but
the definition (the sum is exact; SiLU's f64 exp is within an f64 ulp on any
libm, so its f32 rounding agrees except within 2^-29 of a rounding boundary).
"""
from __future__ import annotations

import math

import numpy as np

from . import quantize_act


def rmsnorm(x: np.ndarray, w: np.ndarray, eps: float) -> tuple[np.ndarray, np.ndarray]:
    """RMSNorm of every row of x [M, K] (f32) with weight w [K] (f32).

    Returns (y [M, K] f32, r [M] f32), r being each row's f32 scale."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    w = np.ascontiguousarray(w, dtype=np.float32)
    M, K = x.shape
    assert w.shape == (K,)
    eps64 = float(np.float32(eps))
    y = np.empty_like(x)
    r = np.empty(M, dtype=np.float32)
    for t in range(M):
        sq = x[t].astype(np.float64) ** 2            # exact squares
        ss = math.fsum(sq.tolist())                  # exact sum, rounded once
        r[t] = np.float32(1.0 / math.sqrt(ss / K + eps64))
        y[t] = (x[t] * r[t]) * w
    return y, r


def swiglu(g: np.ndarray, u: np.ndarray) -> np.ndarray:
    """SiLU(g) * u elementwise for f32 arrays of one shape."""
    g = np.asarray(g, dtype=np.float32)
    u = np.asarray(u, dtype=np.float32)
    assert g.shape == u.shape
    g64 = g.astype(np.float64)
    with np.errstate(over="ignore"):
        s = (g64 / (1.0 + np.exp(-g64))).astype(np.float32)
    return (s * u).astype(np.float32)


def rmsnorm_quantize(x, w, eps):
    """(q, d, s, y): the int8 plane of RMSNorm(x) and the f32 values it quantizes."""
    y, _ = rmsnorm(x, w, eps)
    q, d, s = quantize_act(y)
    return q, d, s, y


def swiglu_quantize(g, u):
    """(q, d, s, y): the int8 plane of SiLU(g) * u and the f32 values it quantizes."""
    y = swiglu(g, u)
    q, d, s = quantize_act(y)
    return q, d, s, y


def ffn_q4k(Wg, Wu, q, d, N, K, tokens=None):
    """Fused FFN up half: (q, d, s, y) with y = SwiGLU(g, u), g and u the
    oracle's f32 Q4_K matmuls of the plane (q, d) with Wg and Wu (minfer
    Compute Graph Design, "The Op vocabulary": FusedFFN, a gate|up matmul with
    an in-place SwiGLU). Only composes the pinned pieces. With `tokens`, only
    those rows of the plane are computed (each row is independent)."""
    from . import matmul_q4k
    g = matmul_q4k(Wg, q, d, N, K, tokens=tokens)
    u = matmul_q4k(Wu, q, d, N, K, tokens=tokens)
    return swiglu_quantize(g, u)

