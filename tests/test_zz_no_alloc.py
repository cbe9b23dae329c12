"""The allocation-free Q6_K entry point (mq_matmul_q6k_static): its split-K
partial sums live in the library's static device array. Checked through the
C ABI against mq_matmul_q6k_ws (same kernels and split, caller workspace) on
two calls in a row, the second with a smaller input, and against the oracle.
"""
import numpy as np
import pytest

import oracle
import quant_gemm_amd as mq
from quant_gemm_amd import synth

pytestmark = pytest.mark.gpu

TOL = 1e-4


def _case(seed, M, N, K):
    import torch
    rng = np.random.default_rng(seed)
    W = synth.q6k_weights(rng, N, K)
    x = synth.activations(rng, M, K, outliers=True)
    rq, rd, _ = oracle.quantize_act(x)
    q, d, _ = mq.quantize_act(torch.from_numpy(x).to("cuda"))
    return W, torch.from_numpy(W.reshape(-1)).to("cuda"), rq, rd, q, d


def _host(t):
    import torch
    torch.cuda.synchronize()
    return t.cpu().numpy()


def test_static_scratch_matches_caller_workspace(dev):
    import torch
    # the full Q6_K M=512 down projection (split 4 ways: 29.4 MB of the
    # 32 MiB array), then a smaller split-K shape in the same array
    for seed, M, N, K in ((1002, 512, 3584, 18944), (77, 300, 700, 4608)):
        # the static array holds the split-K part only (never expansion planes)
        need = mq.matmul_split_workspace(mq.MQ_FMT_Q6K, M, N, K)
        assert 0 < need <= mq.STATIC_SCRATCH_BYTES, (M, N, K, need)
        print(f"[no-alloc] M={M} N={N} K={K} scratch {need} bytes", flush=True)
        W, Wd, rq, rd, q, d = _case(seed, M, N, K)
        got = _host(mq.matmul_q6k_static(Wd, q, d, N, K))
        ws = torch.empty(need, dtype=torch.uint8, device="cuda")   # caller workspace, same plan
        ref = _host(mq.matmul_q6k(Wd, q, d, None, N, K, workspace=ws))
        assert np.array_equal(got, ref), "static scratch and caller workspace: the same bits"
        toks = np.arange(0, M, 37) if M > 64 else None
        orc = oracle.matmul_q6k(W, rq, rd, N, K, tokens=toks)
        g = got if toks is None else got[toks]
        err = np.abs(g.astype(np.float64) - orc).max()
        assert err <= TOL * np.abs(orc).max(), err


def test_static_scratch_rejects_plans_beyond_it(dev):
    import torch
    M, N, K = 3314, 3584, 18944
    # the static array never holds expansion planes: the call needs the
    # split-K part of the query's figure
    need = mq.matmul_split_workspace(mq.MQ_FMT_Q6K, M, N, K)
    assert need > mq.STATIC_SCRATCH_BYTES
    Wd = torch.zeros(N * (K // 256) * 210, dtype=torch.uint8, device="cuda")
    q = torch.zeros((M, K), dtype=torch.int8, device="cuda")
    d = torch.zeros((M, K // 32), dtype=torch.float32, device="cuda")
    with pytest.raises(mq.MQError) as e:
        mq.matmul_q6k_static(Wd, q, d, N, K)
    assert e.value.status == 7 and str(need) in str(e.value)
