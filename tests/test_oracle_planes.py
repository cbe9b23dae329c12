"""Pins of the oracle's registration-time planes: the Q6_K expansion (int8
limb planes of sc*(q - 32) plus d) and the Q4_K decoded-scale planes (d*sc,
dmin*m per sub-block). Each is checked against the independent numpy
decoders of tests/blocks.py, element by element, and through a matmul
evaluated from the planes against the separately pinned raw-block matmuls."""
import numpy as np
import pytest

import oracle
from blocks import q4k_fields, q6k_fields, q6k_pack
from quant_gemm_amd import synth


def _qplane(rng, M, K):
    q = rng.integers(-127, 128, size=(M, K), dtype=np.int8)
    d = rng.uniform(0.001, 0.05, size=(M, K // 32)).astype(np.float32)
    return q, d


@pytest.mark.parametrize("N,K", [(3, 256), (7, 768), (33, 512)])
def test_expand_q6k_matches_numpy_decoder(N, K):
    rng = np.random.default_rng(N + K)
    W = synth.q6k_weights(rng, N, K)
    lo, hi, dw = oracle.expand_q6k(W, N, K)
    d, scales, q = q6k_fields(W, N, K)                 # [N, nb], [N, nb, 16], [N, nb, 256]
    p = (scales[:, :, np.arange(256) // 16] * (q - 32)).reshape(N, K)
    assert lo.min() >= 0 and lo.max() <= 63 and hi.min() >= -64 and hi.max() <= 64
    assert np.array_equal(64 * hi.astype(np.int64) + lo, p)
    assert np.array_equal(dw.astype(np.float64), d)


def test_expand_q6k_extremes():
    """sc = -128 with q = 0 gives p = 4096 = 64*64 + 0; sc = 127 with q = 0
    gives p = -4064 = 64*(-64) + 32; q = 32 gives p = 0 for any scale."""
    sc = np.array([-128, 127, -1, 1] + [5] * 12)
    qv = np.full(256, 32)
    qv[0:16] = 0
    qv[16:32] = 0
    qv[32] = 63
    qv[48] = 1
    blk = q6k_pack(0.5, sc, qv)
    lo, hi, dw = oracle.expand_q6k(blk.reshape(1, -1), 1, 256)
    assert (hi[0, 0], lo[0, 0]) == (64, 0)
    assert (hi[0, 16], lo[0, 16]) == (-64, 32)
    assert (hi[0, 32], lo[0, 32]) == (-1, 33)          # -1 * 31 = -31 = 64*(-1) + 33
    assert (hi[0, 48], lo[0, 48]) == (-1, 33)          # 1 * (1 - 32) = -31
    assert not hi[0, 64:].any() and not lo[0, 64:].any()
    assert dw[0, 0] == 0.5


def test_expand_q6k_planes_reproduce_the_matmul():
    """out = sum over 32-blocks of d_w * d_x * sum((64 hi + lo) * q): the
    raw-block matmul, to 1e-12 relative."""
    rng = np.random.default_rng(71)
    M, N, K = 5, 9, 768
    W = synth.q6k_weights(rng, N, K)
    q, dx = _qplane(rng, M, K)
    lo, hi, dw = oracle.expand_q6k(W, N, K)
    p = 64 * hi.astype(np.int64) + lo                  # [N, K]
    J = (q.astype(np.int64).reshape(M, 1, K // 32, 32) * p.reshape(1, N, K // 32, 32)).sum(axis=3)
    wscale = np.repeat(dw.astype(np.float64), 8, axis=1)          # d per 32-block
    out = (J * dx.astype(np.float64)[:, None, :] * wscale[None, :, :]).sum(axis=2)
    ref = oracle.matmul_q6k(W, q, dx, N, K, f64=True)
    assert np.abs(out - ref).max() <= 1e-12 * np.abs(ref).max()


@pytest.mark.parametrize("N,K", [(3, 256), (12, 1024)])
def test_dsc_q4k_matches_numpy_decoder(N, K):
    rng = np.random.default_rng(N * 3 + K)
    W = synth.q4k_weights(rng, N, K)
    fw, fm = oracle.dsc_q4k(W, N, K)
    d, dmin, sc, m, _ = q4k_fields(W, N, K)
    assert np.array_equal(fw.astype(np.float64), (d[:, :, None] * sc).reshape(N, K // 32))
    assert np.array_equal(fm.astype(np.float64), (dmin[:, :, None] * m).reshape(N, K // 32))


def test_dsc_q4k_planes_reproduce_the_matmul():
    rng = np.random.default_rng(72)
    M, N, K = 4, 7, 512
    W = synth.q4k_weights(rng, N, K)
    q, dx = _qplane(rng, M, K)
    fw, fm = oracle.dsc_q4k(W, N, K)
    _, _, _, _, qw = q4k_fields(W, N, K)
    qw = qw.reshape(N, K)
    I = (q.astype(np.int64).reshape(M, 1, K // 32, 32) * qw.reshape(1, N, K // 32, 32)).sum(axis=3)
    S = q.astype(np.int64).reshape(M, K // 32, 32).sum(axis=2)
    out = ((I * fw[None].astype(np.float64) - S[:, None, :] * fm[None].astype(np.float64))
           * dx.astype(np.float64)[:, None, :]).sum(axis=2)
    ref = oracle.matmul_q4k(W, q, dx, N, K, f64=True)
    assert np.abs(out - ref).max() <= 1e-12 * np.abs(ref).max()
