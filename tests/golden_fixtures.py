"""Builders for the hand-derived fixtures under tests/golden/.

Each fixture gives block bytes (or the rule that makes them), an activation
plane row, and an expected value derived by hand in its "derivation" field.
"""
import json
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _plane(fx):
    K = fx["K"]
    q = np.zeros((1, K), np.int8)
    for k, v in fx["act_q"].items():
        q[0, int(k)] = v
    d = np.full((1, K // 32), fx["act_d_default"], np.float32)
    for b, v in fx["act_d"].items():
        d[0, int(b)] = v
    return q, d


def q4k_case():
    fx = load("q4k_hand_block.json")
    blk = np.zeros(144, np.uint8)
    blk[0:2] = np.frombuffer(bytes.fromhex(fx["d_f16_hex"])[::-1], np.uint8)
    blk[2:4] = np.frombuffer(bytes.fromhex(fx["dmin_f16_hex"])[::-1], np.uint8)
    blk[4:16] = np.frombuffer(bytes.fromhex(fx["scales_hex"]), np.uint8)
    i = np.arange(128)
    blk[16:144] = ((i + 1) % 16) | (((i + 7) % 16) << 4)
    q, d = _plane(fx)
    return fx, blk, q, d


def q5k_case():
    fx = load("q5k_hand_block.json")
    blk = np.zeros(176, np.uint8)
    blk[0:2] = np.frombuffer(bytes.fromhex(fx["d_f16_hex"])[::-1], np.uint8)
    blk[2:4] = np.frombuffer(bytes.fromhex(fx["dmin_f16_hex"])[::-1], np.uint8)
    blk[4:16] = np.frombuffer(bytes.fromhex(fx["scales_hex"]), np.uint8)
    blk[16:48] = (9 * np.arange(32)) % 256
    i = np.arange(128)
    blk[48:176] = ((i + 1) % 16) | (((i + 7) % 16) << 4)
    q, d = _plane(fx)
    return fx, blk, q, d


def q6k_case():
    fx = load("q6k_hand_block.json")
    blk = np.zeros(210, np.uint8)
    i = np.arange(128)
    blk[0:128] = (i % 16) | ((i // 16) << 4)
    blk[128:192] = np.arange(64)
    blk[192:208] = (np.arange(16) - 8).astype(np.int8).view(np.uint8)
    blk[208:210] = np.frombuffer(bytes.fromhex(fx["d_f16_hex"])[::-1], np.uint8)
    q, d = _plane(fx)
    return fx, blk, q, d


def quantizer_rows():
    fx = load("quantizer_hand_rows.json")
    rows = fx["rows"]
    x = np.zeros((len(rows), 32), np.float32)
    q = np.zeros((len(rows), 32), np.int8)
    d = np.zeros((len(rows), 1), np.float32)
    s = np.zeros((len(rows), 1), np.float32)
    for r, row in enumerate(rows):
        for k, v in row["x"].items():
            x[r, int(k)] = v
        for k, v in row["q"].items():
            q[r, int(k)] = v
        d[r, 0] = row["d"]
        s[r, 0] = row["s"]
    return x, q, d, s
