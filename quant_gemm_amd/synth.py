"""Seeded synthetic inputs for the k-quant weight matmul.

This module is shared by the CPU oracle tests and by the HIP tests and bench.
It only draws random bytes and floats: it holds none of the method's
arithmetic (no block decoding, no activation quantization, no dot products).

What it does know is where the two f16 fields sit inside a super-block, so
that it can overwrite the random bytes there with drawn scales. The blocks are
GGML's 256-value super-blocks (minfer Architecture, §6 Quantization & Tensor
Layout): a Q4_K block is 144 bytes and a Q5_K block 176 bytes, both with f16
``d`` at byte 0 and f16 ``dmin`` at byte 2; a Q6_K block is 210 bytes with f16
``d`` at byte 208.

Because every bit of a block outside those f16 fields belongs to exactly one
quant or one scale/min code, uniform random bytes give independent uniform
quants (0..15, 0..31 or 0..63), uniform 6-bit scale/min codes (0..63) and
uniform int8 Q6_K scales (-128..127), whatever the packing.

Draw order for one matrix: weight bytes, then ``d`` (then ``dmin`` for Q4_K
and Q5_K),
from the weight stream; activations, then the outlier columns, from the
activation stream. Scales are drawn in float64 and rounded to f16 by numpy
(round to nearest even); the stored f16 is authoritative.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

QK_K = 256
Q4K_BLOCK_BYTES = 144
Q5K_BLOCK_BYTES = 176
Q6K_BLOCK_BYTES = 210
QK8 = 32  # activation quantization block

BLOCK_BYTES = {"q4k": Q4K_BLOCK_BYTES, "q5k": Q5K_BLOCK_BYTES, "q6k": Q6K_BLOCK_BYTES}


def row_bytes(fmt: str, K: int) -> int:
    """Bytes in one weight row of K values (K a multiple of 256)."""
    return (K // QK_K) * BLOCK_BYTES[fmt]


def q4k_weights(rng: np.random.Generator, N: int, K: int,
                d_range=(1e-3, 1e-2), dmin_range=(0.0, 5e-3)) -> np.ndarray:
    """N rows of K/256 Q4_K blocks as a uint8 array [N, (K/256)*144]."""
    assert K % QK_K == 0
    nb = K // QK_K
    raw = rng.integers(0, 256, size=(N, nb, Q4K_BLOCK_BYTES), dtype=np.uint8)
    d = rng.uniform(d_range[0], d_range[1], size=(N, nb)).astype(np.float16)
    dmin = rng.uniform(dmin_range[0], dmin_range[1], size=(N, nb)).astype(np.float16)
    raw[:, :, 0:2] = d.view(np.uint8).reshape(N, nb, 2)
    raw[:, :, 2:4] = dmin.view(np.uint8).reshape(N, nb, 2)
    return raw.reshape(N, nb * Q4K_BLOCK_BYTES)


def q5k_weights(rng: np.random.Generator, N: int, K: int,
                d_range=(5e-4, 5e-3), dmin_range=(0.0, 5e-3)) -> np.ndarray:
    """N rows of K/256 Q5_K blocks as a uint8 array [N, (K/256)*176]."""
    assert K % QK_K == 0
    nb = K // QK_K
    raw = rng.integers(0, 256, size=(N, nb, Q5K_BLOCK_BYTES), dtype=np.uint8)
    d = rng.uniform(d_range[0], d_range[1], size=(N, nb)).astype(np.float16)
    dmin = rng.uniform(dmin_range[0], dmin_range[1], size=(N, nb)).astype(np.float16)
    raw[:, :, 0:2] = d.view(np.uint8).reshape(N, nb, 2)
    raw[:, :, 2:4] = dmin.view(np.uint8).reshape(N, nb, 2)
    return raw.reshape(N, nb * Q5K_BLOCK_BYTES)


def q6k_weights(rng: np.random.Generator, N: int, K: int,
                d_range=(1e-4, 1e-3)) -> np.ndarray:
    """N rows of K/256 Q6_K blocks as a uint8 array [N, (K/256)*210]."""
    assert K % QK_K == 0
    nb = K // QK_K
    raw = rng.integers(0, 256, size=(N, nb, Q6K_BLOCK_BYTES), dtype=np.uint8)
    d = rng.uniform(d_range[0], d_range[1], size=(N, nb)).astype(np.float16)
    raw[:, :, 208:210] = d.view(np.uint8).reshape(N, nb, 2)
    return raw.reshape(N, nb * Q6K_BLOCK_BYTES)


def weights(fmt: str, rng: np.random.Generator, N: int, K: int) -> np.ndarray:
    gen = {"q4k": q4k_weights, "q5k": q5k_weights, "q6k": q6k_weights}[fmt]
    return gen(rng, N, K)


def activations(rng: np.random.Generator, M: int, K: int,
                outliers: bool = False) -> np.ndarray:
    """f32 activations [M, K] ~ N(0, 1).

    With ``outliers``, round(0.01*K) distinct columns, drawn without
    replacement and shared by all rows, are multiplied by 20.
    """
    x = rng.standard_normal((M, K), dtype=np.float32)
    if outliers:
        n_out = int(round(0.01 * K))
        cols = rng.choice(K, size=n_out, replace=False)
        x[:, cols] *= np.float32(20.0)
    return x


@dataclass(frozen=True)
class Case:
    """One matrix of a workload: weights [N rows of K] times activations [M, K]."""
    name: str
    fmt: str          # "q4k", "q5k" or "q6k"
    M: int
    N: int
    K: int
    outliers: bool
    seed: int
    w_key: int        # weight stream key
    x_key: int        # activation stream key (cases sharing it share x)

    @property
    def ops(self) -> int:
        """Algorithmic int8 operations, 2*M*N*K."""
        return 2 * self.M * self.N * self.K

    @property
    def weight_bytes(self) -> int:
        return self.N * row_bytes(self.fmt, self.K)

    def make_weights(self) -> np.ndarray:
        rng = np.random.default_rng([self.seed, 0, self.w_key])
        return weights(self.fmt, rng, self.N, self.K)

    def make_activations(self) -> np.ndarray:
        rng = np.random.default_rng([self.seed, 1, self.x_key])
        return activations(rng, self.M, self.K, self.outliers)


def _c(name, fmt, M, N, K, outliers, seed, w_key, x_key):
    return Case(name, fmt, M, N, K, outliers, seed, w_key, x_key)


# The workloads: 7B-class shapes (hidden 3584, FFN 18944, fused QKV 4608,
# vocabulary rows 152064, prompt of 3314 tokens).
WORKLOAD_GROUPS = {
    0: [_c("tiny_q4k", "q4k", 8, 256, 1024, False, 1000, 0, 0)],
    1: [_c("q4k_decode_ffn_up", "q4k", 1, 18944, 3584, False, 1001, 0, 0)],
    2: [_c("q6k_ffn_down_m1", "q6k", 1, 3584, 18944, False, 1002, 0, 0),
        _c("q6k_ffn_down_m512", "q6k", 512, 3584, 18944, False, 1002, 0, 1)],
    3: [_c("q4k_prefill_ffn_up", "q4k", 3314, 18944, 3584, True, 1003, 0, 0),
        _c("q4k_prefill_attn_o", "q4k", 3314, 3584, 3584, True, 1003, 1, 0)],
    4: [_c("layer_qkv", "q4k", 3314, 4608, 3584, True, 1004, 0, 0),
        _c("layer_o", "q4k", 3314, 3584, 3584, True, 1004, 1, 1),
        _c("layer_gate", "q4k", 3314, 18944, 3584, True, 1004, 2, 2),
        _c("layer_up", "q4k", 3314, 18944, 3584, True, 1004, 3, 2),
        _c("layer_down", "q6k", 3314, 3584, 18944, True, 1004, 4, 3),
        _c("output_head", "q6k", 1, 152064, 3584, True, 1004, 5, 4)],
    # One GPU's share of the ffn_up matrix when its rows are split over 8
    # GPUs (N / 8 = 2368 rows each), decode and prefill
    "shard8": [_c("q4k_decode_ffn_up_n2368", "q4k", 1, 2368, 3584, False, 1006, 0, 0),
               _c("q4k_prefill_ffn_up_n2368", "q4k", 3314, 2368, 3584, True, 1006, 1, 1)],
    # Q5_K at the ffn_up shape, decode and prefill
    "q5k": [_c("q5k_decode_ffn_up", "q5k", 1, 18944, 3584, False, 1005, 0, 0),
            _c("q5k_prefill_ffn_up", "q5k", 3314, 18944, 3584, True, 1005, 0, 1)],
}


def all_cases():
    for grp, cases in WORKLOAD_GROUPS.items():
        for c in cases:
            yield grp, c


def case_by_name(name: str) -> Case:
    for _, c in all_cases():
        if c.name == name:
            return c
    raise KeyError(name)
