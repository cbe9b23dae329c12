"""Test-only helpers: block encoders and a brute-force float64 reference.

Nothing here is used by the product library or by the oracle. The decoders in
this file are a second, vectorized numpy coding of the GGML Q4_K / Q5_K /
Q6_K super-block layouts (minfer Architecture, §6 Quantization & Tensor Layout),
written independently of the loop-by-loop C decoders of the oracle, so that the
brute-force pin compares two separate readings of the same layout.

Layouts (little-endian):
  Q4_K (144 B): f16 d @0, f16 dmin @2, 12-byte scale/min field @4, 128 B of
    4-bit quants @16. Weight w = 64c + 32h + i -> (qs[32c+i] >> 4h) & 15, in
    sub-block j = w // 32. Codes: for j < 4, sc_j = B[j] & 63 and
    m_j = B[j+4] & 63; for j >= 4, sc_j = (B[j+4] & 15) | (B[j-4] >> 6) << 4
    and m_j = (B[j+4] >> 4) | (B[j] >> 6) << 4.
  Q5_K (176 B): f16 d @0, f16 dmin @2, the Q4_K scale/min field @4, qh[32]
    @16, qs[128] @48. Weight w = 64c + 32h + i -> (qs[32c+i] >> 4h) & 15 |
    ((qh[i] >> (2c + h)) & 1) << 4, in sub-block j = w // 32 = 2c + h.
  Q6_K (210 B): ql[128] @0, qh[64] @128, int8 scales[16] @192, f16 d @208.
    Weight w = 128g + 32r + i -> low4 = (ql[64g + 32(r%2) + i] >> 4(r//2)) & 15,
    high2 = (qh[32g + i] >> 2r) & 3, value d*scales[w//16]*(low4|high2<<4 - 32).
"""
from __future__ import annotations

import numpy as np


# ---------------------------------------------------------------------------
# Encoders (build blocks with chosen fields)
# ---------------------------------------------------------------------------

def q4k_pack(d: float, dmin: float, sc, m, q) -> np.ndarray:
    """Pack one Q4_K block. sc, m: 8 codes in 0..63; q: 256 quants in 0..15."""
    sc = [int(v) for v in sc]
    m = [int(v) for v in m]
    q = np.asarray(q, dtype=np.int64)
    assert len(sc) == 8 and len(m) == 8 and q.shape == (256,)
    assert all(0 <= v < 64 for v in sc + m) and q.min() >= 0 and q.max() < 16
    blk = np.zeros(144, np.uint8)
    blk[0:2] = np.array([d], np.float16).view(np.uint8)
    blk[2:4] = np.array([dmin], np.float16).view(np.uint8)
    B = [0] * 12
    for j in range(4):
        B[j] = (sc[j] & 63) | ((sc[j + 4] >> 4) << 6)
        B[j + 4] = (m[j] & 63) | ((m[j + 4] >> 4) << 6)
        B[j + 8] = (sc[j + 4] & 15) | ((m[j + 4] & 15) << 4)
    blk[4:16] = np.array(B, np.uint8)
    qs = np.zeros(128, np.int64)
    for w in range(256):
        c, h, i = w // 64, (w // 32) % 2, w % 32
        qs[32 * c + i] |= int(q[w]) << (4 * h)
    blk[16:144] = qs.astype(np.uint8)
    return blk


def q5k_pack(d: float, dmin: float, sc, m, q) -> np.ndarray:
    """Pack one Q5_K block. sc, m: 8 codes in 0..63; q: 256 quants in 0..31."""
    q = np.asarray(q, dtype=np.int64)
    assert q.shape == (256,) and q.min() >= 0 and q.max() < 32
    low = q4k_pack(d, dmin, sc, m, q & 15)          # d, dmin, codes and low nibbles
    blk = np.zeros(176, np.uint8)
    blk[0:16] = low[0:16]
    blk[48:176] = low[16:144]
    qh = np.zeros(32, np.int64)
    for w in range(256):
        j, i = w // 32, w % 32
        qh[i] |= (int(q[w]) >> 4) << j
    blk[16:48] = qh.astype(np.uint8)
    return blk


def q6k_pack(d: float, scales, q) -> np.ndarray:
    """Pack one Q6_K block. scales: 16 ints in -128..127; q: 256 stored quants in 0..63."""
    scales = np.asarray(scales, dtype=np.int64)
    q = np.asarray(q, dtype=np.int64)
    assert scales.shape == (16,) and q.shape == (256,)
    assert q.min() >= 0 and q.max() < 64
    blk = np.zeros(210, np.uint8)
    ql = np.zeros(128, np.int64)
    qh = np.zeros(64, np.int64)
    for w in range(256):
        g, r, i = w // 128, (w // 32) % 4, w % 32
        ql[64 * g + 32 * (r % 2) + i] |= (int(q[w]) & 15) << (4 * (r // 2))
        qh[32 * g + i] |= (int(q[w]) >> 4) << (2 * r)
    blk[0:128] = ql.astype(np.uint8)
    blk[128:192] = qh.astype(np.uint8)
    blk[192:208] = scales.astype(np.int8).view(np.uint8)
    blk[208:210] = np.array([d], np.float16).view(np.uint8)
    return blk


# ---------------------------------------------------------------------------
# Vectorized decoders and brute force
# ---------------------------------------------------------------------------

def q4k_fields(W: np.ndarray, N: int, K: int):
    """Decode all Q4_K blocks -> (d, dmin [N, nb] f64, sc, m [N, nb, 8], q [N, nb, 256])."""
    nb = K // 256
    blk = np.ascontiguousarray(W, dtype=np.uint8).reshape(N, nb, 144)
    d = blk[:, :, 0:2].copy().view(np.float16)[:, :, 0].astype(np.float64)
    dmin = blk[:, :, 2:4].copy().view(np.float16)[:, :, 0].astype(np.float64)
    B = blk[:, :, 4:16].astype(np.int64)
    sc = np.empty((N, nb, 8), np.int64)
    m = np.empty((N, nb, 8), np.int64)
    sc[:, :, 0:4] = B[:, :, 0:4] & 63
    m[:, :, 0:4] = B[:, :, 4:8] & 63
    sc[:, :, 4:8] = (B[:, :, 8:12] & 15) | ((B[:, :, 0:4] >> 6) << 4)
    m[:, :, 4:8] = (B[:, :, 8:12] >> 4) | ((B[:, :, 4:8] >> 6) << 4)
    qs = blk[:, :, 16:144].astype(np.int64).reshape(N, nb, 4, 1, 32)
    q = np.concatenate([qs & 15, qs >> 4], axis=3).reshape(N, nb, 256)
    return d, dmin, sc, m, q


def q5k_fields(W: np.ndarray, N: int, K: int):
    """Decode all Q5_K blocks -> (d, dmin [N, nb] f64, sc, m [N, nb, 8], q [N, nb, 256] in 0..31)."""
    nb = K // 256
    blk = np.ascontiguousarray(W, dtype=np.uint8).reshape(N, nb, 176)
    as_q4 = np.concatenate([blk[:, :, 0:16], blk[:, :, 48:176]], axis=2)
    d, dmin, sc, m, low = q4k_fields(as_q4.reshape(N, nb * 144), N, K)
    qh = blk[:, :, 16:48].astype(np.int64)                          # [N, nb, 32]
    high = np.stack([(qh >> j) & 1 for j in range(8)], axis=2)      # [N, nb, 8 sub-blocks, 32]
    return d, dmin, sc, m, low | (high.reshape(N, nb, 256) << 4)


def q6k_fields(W: np.ndarray, N: int, K: int):
    """Decode all Q6_K blocks -> (d [N, nb] f64, scales [N, nb, 16], q [N, nb, 256] stored)."""
    nb = K // 256
    blk = np.ascontiguousarray(W, dtype=np.uint8).reshape(N, nb, 210)
    ql = blk[:, :, 0:128].astype(np.int64).reshape(N, nb, 2, 2, 32)  # g, r%2, i
    qh = blk[:, :, 128:192].astype(np.int64).reshape(N, nb, 2, 1, 32)  # g, -, i
    low = np.concatenate([ql & 15, ql >> 4], axis=3)   # g, (r%2) + 2*(r//2), i
    high = np.concatenate([(qh >> (2 * r)) & 3 for r in range(4)], axis=3)
    q = (low | (high << 4)).reshape(N, nb, 256)
    scales = blk[:, :, 192:208].copy().view(np.int8).astype(np.int64)
    d = blk[:, :, 208:210].copy().view(np.float16)[:, :, 0].astype(np.float64)
    return d, scales, q


def dequant_f64(fmt: str, W: np.ndarray, N: int, K: int) -> np.ndarray:
    """Every weight value in float64, [N, K]. Exact: all products fit in 53 bits."""
    nb = K // 256
    if fmt in ("q4k", "q5k"):
        d, dmin, sc, m, q = (q4k_fields if fmt == "q4k" else q5k_fields)(W, N, K)
        j = np.arange(256) // 32
        w = d[:, :, None] * sc[:, :, j] * q - dmin[:, :, None] * m[:, :, j]
    else:
        d, scales, q = q6k_fields(W, N, K)
        j = np.arange(256) // 16
        w = d[:, :, None] * scales[:, :, j] * (q - 32)
    return w.reshape(N, nb * 256)


def bruteforce_f64(fmt: str, W: np.ndarray, q: np.ndarray, dx: np.ndarray,
                   N: int, K: int) -> np.ndarray:
    """out[t, n] = sum_k w[n, k] * (dx[t, k//32] * q[t, k]), all in float64."""
    w = dequant_f64(fmt, W, N, K)
    xhat = np.repeat(dx.astype(np.float64), 32, axis=1) * q.astype(np.float64)
    return xhat @ w.T
