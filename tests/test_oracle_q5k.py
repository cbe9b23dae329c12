"""Pins of the oracle's Q5_K matmul (GGML's 176-byte block: the Q4_K fields
plus one high bit per quant) to things other than itself.

  * the numpy decoder of tests/blocks.py and a float64 dequantize-then-multiply
    agree with the oracle (run with the other formats in test_oracle_pins);
  * with every high bit clear a Q5_K block is the Q4_K block of the same
    fields, and with every high bit set it adds exactly 16 d sc_j per value:
    both compared with the separately pinned Q4_K matmul;
  * integer GEMM with unit scales and zero mins over all 32 quant values;
  * one-hot probes of every position, on the low nibble and on the high bit;
  * the min term's closed form, zero invariants, encoder round trips;
  * a hand-derived block (tests/golden/q5k_hand_block.json).
"""
import numpy as np

import oracle
import golden_fixtures as gf
from blocks import bruteforce_f64, q4k_pack, q5k_fields, q5k_pack
from quant_gemm_amd import synth


def _qplane(rng, M, K):
    q = rng.integers(-127, 128, size=(M, K), dtype=np.int8)
    d = rng.uniform(0.001, 0.05, size=(M, K // 32)).astype(np.float32)
    return q, d


def _rows(blocks_per_row):
    return np.stack([np.concatenate(r) for r in blocks_per_row])


def _unit_diag():
    """x = 127 e_k for k = 0..255: plane q = x, d = 1 on the block holding k."""
    x = np.zeros((256, 256), np.float32)
    x[np.arange(256), np.arange(256)] = 127.0
    q, d, _ = oracle.quantize_act(x)
    assert np.array_equal(q.astype(np.float32), x)
    assert np.array_equal(d[np.arange(256), np.arange(256) // 32], np.ones(256, np.float32))
    return q, d


def test_high_bits_clear_is_q4k():
    rng = np.random.default_rng(61)
    M, N, K = 4, 6, 512
    W5 = synth.q5k_weights(rng, N, K).reshape(N, K // 256, 176)
    W5[:, :, 16:48] = 0                                   # every high bit 0
    W4 = np.concatenate([W5[:, :, 0:16], W5[:, :, 48:176]], axis=2).reshape(N, -1)
    q, d = _qplane(rng, M, K)
    got = oracle.matmul_q5k(W5.reshape(N, -1), q, d, N, K, f64=True)
    assert np.array_equal(got, oracle.matmul_q4k(W4, q, d, N, K, f64=True))


def test_high_bits_set_adds_sixteen_d_sc():
    """Every high bit 1: out = Q4_K(same fields) + sum_b 16 d sc_b dx_b sum(q in b)."""
    rng = np.random.default_rng(62)
    M, N, K = 3, 5, 768
    nb = K // 256
    W5 = synth.q5k_weights(rng, N, K).reshape(N, nb, 176)
    W5[:, :, 16:48] = 0xFF
    W4 = np.concatenate([W5[:, :, 0:16], W5[:, :, 48:176]], axis=2).reshape(N, -1)
    q, d = _qplane(rng, M, K)
    got = oracle.matmul_q5k(W5.reshape(N, -1), q, d, N, K, f64=True)
    base = oracle.matmul_q4k(W4, q, d, N, K, f64=True)
    dd = np.zeros((N, K // 32))
    for n in range(N):
        for s in range(nb):
            f = oracle.q4k_block_decode(W4[n, 144 * s:144 * s + 144])
            dd[n, 8 * s:8 * s + 8] = f["d"] * f["sc"]
    qsum = q.astype(np.int64).reshape(M, K // 32, 32).sum(axis=2)
    extra = (16.0 * d.astype(np.float64) * qsum) @ dd.T
    assert np.abs(got - (base + extra)).max() <= 1e-12 * np.abs(got).max()


def test_q5k_reduces_to_integer_gemm():
    rng = np.random.default_rng(63)
    M, N, K = 5, 6, 512
    qw = rng.integers(0, 32, size=(N, K))
    qw[0, :32] = np.arange(32)                            # every quant value appears
    W = _rows([[q5k_pack(1.0, 0.0, [1] * 8, [0] * 8, qw[n, 256 * s:256 * s + 256])
                for s in range(K // 256)] for n in range(N)])
    x = rng.integers(-127, 128, size=(M, K)).astype(np.float32)
    for t in range(M):
        for b in range(K // 32):
            x[t, 32 * b + (t + b) % 32] = 127.0           # |max| = 127 -> d = 1, q = x
    q, d, _ = oracle.quantize_act(x)
    assert np.all(d == 1.0) and np.array_equal(q.astype(np.float32), x)
    got = oracle.matmul_q5k(W, q, d, N, K)
    exact = x.astype(np.int64) @ qw.T.astype(np.int64)
    assert np.array_equal(got, exact.astype(np.float32))


def test_q5k_one_hot_positions():
    """One nonzero quant at position p: out != 0 only for input column p. The
    value 16 probes the high bit alone, 1 + p % 15 the low nibble alone."""
    q, d = _unit_diag()
    for p in range(256):
        for val in (16, 1 + p % 15, 31):
            qw = np.zeros(256, int)
            qw[p] = val
            W = q5k_pack(1.0, 0.0, [1] * 8, [0] * 8, qw).reshape(1, -1)
            out = oracle.matmul_q5k(W, q, d, 1, 256)[:, 0]
            assert list(np.flatnonzero(out)) == [p] and out[p] == 127.0 * val


def test_q5k_scale_and_min_groups():
    """Each scale code multiplies, and each min code subtracts from, exactly
    its own 32-column group."""
    q, d = _unit_diag()
    sc = [1, 2, 3, 5, 7, 11, 13, 17]
    W = q5k_pack(1.0, 0.0, sc, [0] * 8, np.full(256, 17)).reshape(1, -1)
    out = oracle.matmul_q5k(W, q, d, 1, 256)[:, 0]
    assert np.array_equal(out, 127.0 * 17 * np.repeat(sc, 32))
    m = [63, 1, 2, 4, 8, 16, 32, 9]
    W = q5k_pack(1.0, 1.0, [0] * 8, m, np.full(256, 31)).reshape(1, -1)
    out = oracle.matmul_q5k(W, q, d, 1, 256)[:, 0]
    assert np.array_equal(out, -127.0 * np.repeat(m, 32))


def test_q5k_min_term_closed_form():
    """All quants zero: out[t, n] = -sum_b dmin m_b dx[t, b] sum(q[t, block b])."""
    rng = np.random.default_rng(64)
    M, N, K = 3, 4, 512
    nb = K // 256
    dmins = rng.uniform(0.0, 0.01, size=(N, nb)).astype(np.float16).astype(np.float64)
    ms = rng.integers(0, 64, size=(N, nb, 8))
    scs = rng.integers(0, 64, size=(N, nb, 8))
    W = _rows([[q5k_pack(0.5, dmins[n, s], scs[n, s], ms[n, s], np.zeros(256, int))
                for s in range(nb)] for n in range(N)])
    q, d = _qplane(rng, M, K)
    got = oracle.matmul_q5k(W, q, d, N, K, f64=True)
    qsum = q.astype(np.int64).reshape(M, K // 32, 32).sum(axis=2)
    mins = (dmins[:, :, None] * ms).reshape(N, K // 32)
    expect = -(d.astype(np.float64) * qsum) @ mins.T
    assert np.abs(got - expect).max() <= 1e-12 * np.abs(expect).max()


def test_q5k_zero_quants_zero_dmin_give_zero():
    rng = np.random.default_rng(65)
    N, K, M = 5, 512, 3
    W = synth.q5k_weights(rng, N, K).reshape(N, K // 256, 176)
    W[:, :, 16:] = 0                                      # high bits and low nibbles
    W[:, :, 2:4] = np.array([0.0], np.float16).view(np.uint8)
    q, d, _ = oracle.quantize_act(rng.standard_normal((M, K), dtype=np.float32))
    assert np.all(oracle.matmul_q5k(W.reshape(N, -1), q, d, N, K) == 0.0)


def test_q5k_decode_inverts_pack():
    rng = np.random.default_rng(66)
    for _ in range(20):
        sc = rng.integers(0, 64, 8)
        m = rng.integers(0, 64, 8)
        qv = rng.integers(0, 32, 256)
        blk = q5k_pack(0.25, 0.125, sc, m, qv)
        f = oracle.q5k_block_decode(blk)
        assert f["d"] == 0.25 and f["dmin"] == 0.125
        assert list(f["sc"]) == list(sc) and list(f["m"]) == list(m)
        assert np.array_equal(f["q"], qv)
        # the packed low half is the Q4_K packing of the low nibbles
        assert np.array_equal(blk[48:], q4k_pack(0.25, 0.125, sc, m, qv & 15)[16:])


def test_q5k_numpy_decoder_matches_oracle_decode():
    rng = np.random.default_rng(67)
    N, K = 3, 512
    W = synth.q5k_weights(rng, N, K)
    d, dmin, sc, m, qv = q5k_fields(W, N, K)
    for n in range(N):
        for s in range(K // 256):
            f = oracle.q5k_block_decode(W[n, 176 * s:176 * s + 176])
            assert f["d"] == d[n, s] and f["dmin"] == dmin[n, s]
            assert np.array_equal(f["sc"], sc[n, s]) and np.array_equal(f["m"], m[n, s])
            assert np.array_equal(f["q"], qv[n, s])


def test_q5k_generator_codes_are_uniform():
    rng = np.random.default_rng(68)
    N, K = 64, 2048
    W = synth.q5k_weights(rng, N, K)
    _, _, sc, m, qv = q5k_fields(W, N, K)
    counts = np.bincount(qv.reshape(-1), minlength=32)
    assert counts.size == 32 and counts.min() > 0.9 * qv.size / 32
    assert sc.max() == 63 and m.max() == 63 and sc.min() == 0


def test_q5k_hand_block():
    fx, blk, q, d = gf.q5k_case()
    f = oracle.q5k_block_decode(blk)
    assert f["d"] == 0.5 and f["dmin"] == 0.25
    assert list(f["sc"]) == fx["expected_codes"]["sc"]
    assert list(f["m"]) == fx["expected_codes"]["m"]
    for k, v in fx["expected_quants"].items():
        assert f["q"][int(k)] == v, k
    out = oracle.matmul_q5k(blk.reshape(1, -1), q, d, 1, fx["K"], f64=True)
    assert out[0, 0] == fx["expected_out"]
    assert bruteforce_f64("q5k", blk.reshape(1, -1), q, d, 1, fx["K"])[0, 0] == fx["expected_out"]
