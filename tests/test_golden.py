"""The oracle against hand-derived examples (tests/golden/*.json)."""
import numpy as np

import oracle
import golden_fixtures as gf


def test_q4k_hand_block_codes_and_output():
    fx, blk, q, d = gf.q4k_case()
    f = oracle.q4k_block_decode(blk)
    assert f["d"] == 0.5 and f["dmin"] == 0.25
    assert list(f["sc"]) == fx["expected_codes"]["sc"]
    assert list(f["m"]) == fx["expected_codes"]["m"]
    for k, v in fx["expected_quants"].items():
        assert f["q"][int(k)] == v
    out = oracle.matmul_q4k(blk.reshape(1, -1), q, d, 1, fx["K"], f64=True)
    assert out[0, 0] == fx["expected_out"]


def test_q6k_hand_block_output():
    fx, blk, q, d = gf.q6k_case()
    f = oracle.q6k_block_decode(blk)
    assert f["d"] == 0.125
    assert list(f["sc"]) == list(range(-8, 8))
    for k, v in fx["expected_quants"].items():
        assert f["q"][int(k)] == v
    out = oracle.matmul_q6k(blk.reshape(1, -1), q, d, 1, fx["K"], f64=True)
    assert out[0, 0] == fx["expected_out"]


def test_quantizer_hand_rows():
    x, q, d, s = gf.quantizer_rows()
    gq, gd, gs = oracle.quantize_act(x)
    assert np.array_equal(gq, q) and np.array_equal(gd, d) and np.array_equal(gs, s)
