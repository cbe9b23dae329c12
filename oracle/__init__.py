"""Python face of the CPU oracle (``oracle.c``).

TEST INFRASTRUCTURE ONLY: the tests, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` use it. The product library and its binding
never import it.

Functions take and return numpy arrays. See ``oracle.c`` for what is computed
and which passage of the pages each step follows.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
LIB_PATH = os.path.join(_HERE, "liboracle.so")

# -ffp-contract=off: no fused multiply-add may change a rounding of the
# activation quantizer; no -ffast-math, so division, roundf and subnormals
# keep IEEE semantics.
CFLAGS = ["-O2", "-std=c99", "-fopenmp", "-fPIC", "-shared",
          "-ffp-contract=off", "-fno-fast-math"]


def build(force: bool = True) -> str:
    """Compile ``oracle.c`` into ``liboracle.so`` with gcc."""
    if force or not os.path.exists(LIB_PATH):
        tmp = LIB_PATH + ".tmp"
        subprocess.check_call(["gcc", *CFLAGS, _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, LIB_PATH)
    return LIB_PATH


_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            build(force=False)
        L = ctypes.CDLL(LIB_PATH)
        P = ctypes.c_void_p
        I64 = ctypes.c_int64
        L.oracle_quantize_act.argtypes = [P, I64, I64, I64, P, P, P]
        L.oracle_quantize_act.restype = None
        for name in ("oracle_matmul_q4k", "oracle_matmul_q5k", "oracle_matmul_q6k"):
            f = getattr(L, name)
            f.argtypes = [P, P, P, I64, I64, I64, P, I64, P, P]
            f.restype = None
        for name in ("oracle_q4k_block_decode", "oracle_q5k_block_decode"):
            f = getattr(L, name)
            f.argtypes = [P, P, P, P, P, P]
            f.restype = None
        L.oracle_expand_q6k.argtypes = [P, I64, I64, P, P, P]
        L.oracle_expand_q6k.restype = None
        L.oracle_dsc_q4k.argtypes = [P, I64, I64, P, P]
        L.oracle_dsc_q4k.restype = None
        L.oracle_q6k_block_decode.argtypes = [P, P, P, P]
        L.oracle_q6k_block_decode.restype = None
        L.oracle_max_threads.argtypes = []
        L.oracle_max_threads.restype = ctypes.c_int
        L.oracle_set_threads.argtypes = [ctypes.c_int]
        L.oracle_set_threads.restype = None
        _lib = L
    return _lib


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def quantize_act(x: np.ndarray):
    """f32 [M, K] -> (q int8 [M, K], d f32 [M, K/32], s f32 [M, K/32])."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    M, K = x.shape
    assert K % 32 == 0
    q = np.empty((M, K), np.int8)
    d = np.empty((M, K // 32), np.float32)
    s = np.empty((M, K // 32), np.float32)
    lib().oracle_quantize_act(_ptr(x), M, K, K, _ptr(q), _ptr(d), _ptr(s))
    return q, d, s


def _matmul(name, W, q, d, N, K, tokens, f64):
    q = np.ascontiguousarray(q, dtype=np.int8)
    d = np.ascontiguousarray(d, dtype=np.float32)
    W = np.ascontiguousarray(W, dtype=np.uint8)
    M = q.shape[0]
    assert q.shape == (M, K) and d.shape == (M, K // 32)
    if tokens is None:
        toks_p, ntok = None, M
    else:
        toks = np.ascontiguousarray(tokens, dtype=np.int64)
        assert toks.ndim == 1 and (toks.size == 0 or (toks.min() >= 0 and toks.max() < M))
        toks_p, ntok = _ptr(toks), toks.size
    out = np.empty((ntok, N), np.float64 if f64 else np.float32)
    getattr(lib(), name)(_ptr(W), _ptr(q), _ptr(d), M, N, K, toks_p, ntok,
                         _ptr(out) if f64 else None, None if f64 else _ptr(out))
    return out


def matmul_q4k(W, q, d, N, K, tokens=None, f64=False):
    """Q4_K weights [N rows, K/256 blocks] x activation plane -> out [M or len(tokens), N]."""
    assert W.size == N * (K // 256) * 144
    return _matmul("oracle_matmul_q4k", W, q, d, N, K, tokens, f64)


def matmul_q5k(W, q, d, N, K, tokens=None, f64=False):
    """Q5_K weights [N rows, K/256 blocks] x activation plane -> out [M or len(tokens), N]."""
    assert W.size == N * (K // 256) * 176
    return _matmul("oracle_matmul_q5k", W, q, d, N, K, tokens, f64)


def matmul_q6k(W, q, d, N, K, tokens=None, f64=False):
    """Q6_K weights [N rows, K/256 blocks] x activation plane -> out [M or len(tokens), N]."""
    assert W.size == N * (K // 256) * 210
    return _matmul("oracle_matmul_q6k", W, q, d, N, K, tokens, f64)


def q4k_block_decode(blk: np.ndarray):
    """One 144-byte Q4_K block -> dict(d, dmin, sc[8], m[8], q[256])."""
    blk = np.ascontiguousarray(blk, dtype=np.uint8)
    assert blk.size == 144
    d = np.zeros(1, np.float64)
    dmin = np.zeros(1, np.float64)
    sc = np.zeros(8, np.int32)
    m = np.zeros(8, np.int32)
    q4 = np.zeros(256, np.uint8)
    lib().oracle_q4k_block_decode(_ptr(blk), _ptr(d), _ptr(dmin), _ptr(sc),
                                  _ptr(m), _ptr(q4))
    return dict(d=float(d[0]), dmin=float(dmin[0]), sc=sc, m=m, q=q4)


def q5k_block_decode(blk: np.ndarray):
    """One 176-byte Q5_K block -> dict(d, dmin, sc[8], m[8], q[256] in 0..31)."""
    blk = np.ascontiguousarray(blk, dtype=np.uint8)
    assert blk.size == 176
    d = np.zeros(1, np.float64)
    dmin = np.zeros(1, np.float64)
    sc = np.zeros(8, np.int32)
    m = np.zeros(8, np.int32)
    q5 = np.zeros(256, np.uint8)
    lib().oracle_q5k_block_decode(_ptr(blk), _ptr(d), _ptr(dmin), _ptr(sc),
                                  _ptr(m), _ptr(q5))
    return dict(d=float(d[0]), dmin=float(dmin[0]), sc=sc, m=m, q=q5)


def q6k_block_decode(blk: np.ndarray):
    """One 210-byte Q6_K block -> dict(d, sc[16], q[256] stored 0..63)."""
    blk = np.ascontiguousarray(blk, dtype=np.uint8)
    assert blk.size == 210
    d = np.zeros(1, np.float64)
    sc = np.zeros(16, np.int32)
    q6 = np.zeros(256, np.uint8)
    lib().oracle_q6k_block_decode(_ptr(blk), _ptr(d), _ptr(sc), _ptr(q6))
    return dict(d=float(d[0]), sc=sc, q=q6)


def expand_q6k(W, N, K):
    """Q6_K expansion planes of W [N rows of K]: (lo int8 [N, K] in 0..63,
    hi int8 [N, K] in -64..64, dw f32 [N, K/256]) with 64*hi + lo = sc*(q - 32)."""
    W = np.ascontiguousarray(W, dtype=np.uint8)
    assert W.size == N * (K // 256) * 210
    lo = np.empty((N, K), np.int8)
    hi = np.empty((N, K), np.int8)
    dw = np.empty((N, K // 256), np.float32)
    lib().oracle_expand_q6k(_ptr(W), N, K, _ptr(lo), _ptr(hi), _ptr(dw))
    return lo, hi, dw


def dsc_q4k(W, N, K):
    """Q4_K decoded-scale planes of W [N rows of K]: (fw, fm) f32 [N, K/32],
    fw = d*sc_j and fm = dmin*m_j per 32-value sub-block."""
    W = np.ascontiguousarray(W, dtype=np.uint8)
    assert W.size == N * (K // 256) * 144
    fw = np.empty((N, K // 32), np.float32)
    fm = np.empty((N, K // 32), np.float32)
    lib().oracle_dsc_q4k(_ptr(W), N, K, _ptr(fw), _ptr(fm))
    return fw, fm


def max_threads() -> int:
    return lib().oracle_max_threads()


def set_threads(n: int) -> None:
    lib().oracle_set_threads(n)
