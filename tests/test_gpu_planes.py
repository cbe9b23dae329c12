"""GPU parity of the registration-time planes and the GEMMs that read them,
through the C ABI.

  * mq_expand_q6k and mq_dsc_q4k write exactly the oracle's planes (integer
    limbs and exact f32 products: compared bit for bit);
  * mq_matmul_q6k_x and mq_matmul_q4k_dsc meet the matmul bar against the
    raw-block oracle (max|d| <= 1e-4 max|oracle|), for small shapes, split-K
    shapes and the full-size workloads (sampled token rows), and agree
    bitwise with the raw-block GEMM where the arithmetic is the same;
  * a Q6_K matmul of at least 512 tokens given its full workspace expands
    W there and runs the expansion-plane GEMM: bitwise the raw-block GEMM's
    result with the split-K workspace alone.
"""
import numpy as np
import pytest

import oracle
import quant_gemm_amd as mq
from quant_gemm_amd import synth

pytestmark = pytest.mark.gpu

TOL = 1e-4


def to_dev(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda")


def host(t):
    import torch
    torch.cuda.synchronize()
    return t.cpu().numpy()


def check_close(got, ref, what):
    ref = np.asarray(ref, dtype=np.float64)
    got = np.asarray(got, dtype=np.float64)
    assert got.shape == ref.shape and np.all(np.isfinite(got)), what
    err = np.abs(got - ref).max()
    assert err <= TOL * np.abs(ref).max(), f"{what}: max|d|={err:.3e}"
    return err / np.abs(ref).max()


@pytest.mark.parametrize("N,K", [(1, 256), (37, 768), (3584, 18944)])
def test_expand_q6k_bit_exact(dev, N, K):
    rng = np.random.default_rng(N + K)
    W = synth.q6k_weights(rng, N, K)
    print(f"[planes] expand_q6k N={N} K={K}", flush=True)
    lo, hi, dw = mq.expand_q6k(to_dev(W.reshape(-1)), N, K)
    rlo, rhi, rdw = oracle.expand_q6k(W, N, K)
    assert np.array_equal(host(lo), rlo) and np.array_equal(host(hi), rhi) and np.array_equal(host(dw), rdw)


@pytest.mark.parametrize("off", [4, 8, 12])
def test_q6k_expansion_from_4_byte_aligned_weights(dev, off):
    """Q6_K weights need only 4-byte alignment: here W starts `off` bytes
    into a 256-aligned buffer, so the expansion kernel stages its 16-block
    groups with dword loads instead of 16-byte ones (45 rows of 19 blocks:
    53 full groups and an odd tail of 7). Its planes equal the oracle's,
    and a 512-token GEMM given its full workspace (the expansion plan)
    equals the raw-block plan bit for bit."""
    import torch
    rng = np.random.default_rng(off)
    N, K, M = 45, 4864, 512
    W = synth.q6k_weights(rng, N, K)
    buf = torch.zeros(W.size + off, dtype=torch.uint8, device="cuda")
    Wd = buf[off:]
    Wd.copy_(torch.from_numpy(W.reshape(-1)).to("cuda"))
    assert Wd.data_ptr() % 16 == off
    print(f"[planes] expand_q6k from W at +{off} bytes, N={N} K={K}", flush=True)
    lo, hi, dw = mq.expand_q6k(Wd, N, K)
    rlo, rhi, rdw = oracle.expand_q6k(W, N, K)
    assert np.array_equal(host(lo), rlo) and np.array_equal(host(hi), rhi) and np.array_equal(host(dw), rdw)
    x = synth.activations(rng, M, K, outliers=True)
    q, d, s = _plane(x)
    full = mq.matmul_workspace(mq.MQ_FMT_Q6K, M, N, K, mq.MQ_PATH_GEMM)
    split = mq.matmul_split_workspace(mq.MQ_FMT_Q6K, M, N, K, mq.MQ_PATH_GEMM)
    assert full == split + mq.q6k_expansion_bytes(N, K) and split > 0
    got = host(mq.matmul_q6k(Wd, q, d, None, N, K, path=mq.MQ_PATH_GEMM,
                             workspace=torch.empty(full, dtype=torch.uint8, device="cuda")))
    raw = host(mq.matmul_q6k(Wd, q, d, None, N, K, path=mq.MQ_PATH_GEMM,
                             workspace=torch.empty(split, dtype=torch.uint8, device="cuda")))
    assert np.array_equal(got, raw), "expansion plan and raw blocks: the same result bit for bit"
    toks = np.array([0, 1, 127, 128, 300, 511])
    rq, rd, _ = oracle.quantize_act(x)
    check_close(got[toks], oracle.matmul_q6k(W, rq, rd, N, K, tokens=toks), f"q6k expansion plan, W at +{off}")


@pytest.mark.parametrize("N,K", [(1, 256), (45, 1280), (18944, 3584)])
def test_dsc_q4k_bit_exact(dev, N, K):
    rng = np.random.default_rng(N * 7 + K)
    W = synth.q4k_weights(rng, N, K)
    print(f"[planes] dsc_q4k N={N} K={K}", flush=True)
    fw, fm = mq.dsc_q4k(to_dev(W.reshape(-1)), N, K)
    rfw, rfm = oracle.dsc_q4k(W, N, K)
    assert np.array_equal(host(fw), rfw) and np.array_equal(host(fm), rfm)


SHAPES = [(1, 1, 256), (5, 129, 768), (31, 100, 512), (33, 64, 1024), (129, 300, 1280), (200, 64, 2048),
          (300, 700, 4608), (17, 257, 2560)]


def _plane(x):
    return mq.quantize_act(to_dev(x))


@pytest.mark.parametrize("M,N,K", SHAPES)
def test_matmul_q6k_x(dev, M, N, K):
    rng = np.random.default_rng(M * 31 + N * 7 + K)
    W = synth.q6k_weights(rng, N, K)
    x = synth.activations(rng, M, K, outliers=True)
    q, d, s = _plane(x)
    Wd = to_dev(W.reshape(-1))
    lo, hi, dw = mq.expand_q6k(Wd, N, K)
    got = host(mq.matmul_q6k_x(lo, hi, dw, q, d, N, K))
    rq, rd, _ = oracle.quantize_act(x)
    check_close(got, oracle.matmul_q6k(W, rq, rd, N, K), f"q6k_x M={M} N={N} K={K}")
    raw = host(mq.matmul_q6k(Wd, q, d, None, N, K, path=mq.MQ_PATH_GEMM))
    assert np.array_equal(got, raw), "same limbs, same order: the raw-block GEMM's result bit for bit"


@pytest.mark.parametrize("M,N,K", SHAPES)
def test_matmul_q4k_dsc(dev, M, N, K):
    rng = np.random.default_rng(M * 37 + N * 5 + K)
    W = synth.q4k_weights(rng, N, K)
    x = synth.activations(rng, M, K, outliers=True)
    q, d, s = _plane(x)
    Wd = to_dev(W.reshape(-1))
    fw, fm = mq.dsc_q4k(Wd, N, K)
    got = host(mq.matmul_q4k_dsc(Wd, fw, fm, q, d, s, N, K))
    rq, rd, _ = oracle.quantize_act(x)
    check_close(got, oracle.matmul_q4k(W, rq, rd, N, K), f"q4k_dsc M={M} N={N} K={K}")
    raw = host(mq.matmul_q4k(Wd, q, d, s, N, K, path=mq.MQ_PATH_GEMM))
    assert np.array_equal(got, raw), "same factors, same order: the raw-block GEMM's result bit for bit"


_SAMPLE = [0, 1, 63, 64, 127, 128, 129, 511, 1000, 2047, 2048, 3199, 3200, 3250, 3312, 3313]


@pytest.mark.parametrize("name", ["layer_down", "q6k_ffn_down_m512", "q4k_prefill_ffn_up", "layer_qkv"])
def test_full_size_planes(dev, name):
    case = synth.case_by_name(name)
    print(f"[planes] {name} {case.fmt} M={case.M} N={case.N} K={case.K}", flush=True)
    W = case.make_weights()
    x = case.make_activations()
    q, d, s = _plane(x)
    Wd = to_dev(W.reshape(-1))
    if case.fmt == "q6k":
        lo, hi, dw = mq.expand_q6k(Wd, case.N, case.K)
        out = host(mq.matmul_q6k_x(lo, hi, dw, q, d, case.N, case.K))
        mm = oracle.matmul_q6k
    else:
        fw, fm = mq.dsc_q4k(Wd, case.N, case.K)
        out = host(mq.matmul_q4k_dsc(Wd, fw, fm, q, d, s, case.N, case.K))
        mm = oracle.matmul_q4k
    toks = np.array(sorted({t for t in _SAMPLE if t < case.M} | {case.M - 1}))
    rq, rd, _ = oracle.quantize_act(x)
    rel = check_close(out[toks], mm(W, rq, rd, case.N, case.K, tokens=toks), name)
    print(f"[planes] {name}: max|d|/max|ref| = {rel:.2e}", flush=True)


@pytest.mark.parametrize("M", [512, 1100])
def test_q6k_matmul_expansion_plan(dev, M):
    """mq_matmul_q6k_ws at M >= 512 with the full workspace (the query's
    bytes) expands W into it and runs the expansion-plane GEMM; with only
    the split-K part it runs the raw-block GEMM. Same splits, same limbs,
    same order: the same bits, and the oracle's result within the bar. The
    weights carry super-blocks with d = +0 and -0 (zeroed limbs) and with a
    negative d (the accumulators' rescale by a signed factor)."""
    import torch
    rng = np.random.default_rng(M)
    N, K = 300, 4608
    W = synth.q6k_weights(rng, N, K).reshape(N, K // 256, 210)
    zero = rng.random((N, K // 256)) < 0.1
    zero[0, :] = True
    W[:, :, 208][zero] = 0
    W[:, :, 209][zero] = np.where(rng.random(zero.sum()) < 0.5, 0x80, 0x00)
    neg = (rng.random((N, K // 256)) < 0.3) & ~zero
    W[:, :, 209][neg] ^= 0x80
    W = W.reshape(N, -1)
    x = synth.activations(rng, M, K, outliers=True)
    q, d, s = _plane(x)
    Wd = to_dev(W.reshape(-1))
    full = mq.matmul_workspace(mq.MQ_FMT_Q6K, M, N, K, mq.MQ_PATH_GEMM)
    split = mq.matmul_split_workspace(mq.MQ_FMT_Q6K, M, N, K, mq.MQ_PATH_GEMM)
    assert full == split + mq.q6k_expansion_bytes(N, K)
    assert split > 0, "this shape splits K"
    print(f"[planes] expansion plan M={M} N={N} K={K}: workspace {full} bytes, split part {split}", flush=True)
    ws_full = torch.empty(full, dtype=torch.uint8, device="cuda")
    ws_split = torch.empty(split, dtype=torch.uint8, device="cuda")
    got = host(mq.matmul_q6k(Wd, q, d, None, N, K, path=mq.MQ_PATH_GEMM, workspace=ws_full))
    raw = host(mq.matmul_q6k(Wd, q, d, None, N, K, path=mq.MQ_PATH_GEMM, workspace=ws_split))
    assert np.array_equal(got, raw), "expansion plan and raw blocks: the same result bit for bit"
    assert np.all(got[:, 0] == 0.0)
    toks = np.array(sorted({t for t in (0, 1, 127, 128, 511, 512, 1023, 1024, M - 1) if t < M}))
    rq, rd, _ = oracle.quantize_act(x)
    check_close(got[toks], oracle.matmul_q6k(W, rq, rd, N, K, tokens=toks), "q6k expansion plan")
    with pytest.raises(mq.MQError) as e:
        mq.matmul_q6k(Wd, q, d, None, N, K, path=mq.MQ_PATH_GEMM,
                      workspace=torch.empty(split - 256, dtype=torch.uint8, device="cuda"))
    assert e.value.status == 7
