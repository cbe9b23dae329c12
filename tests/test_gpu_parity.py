"""GPU parity: libmq (HIP, gfx950) against the CPU oracle, through the C ABI.

Bars:
  * the int8 activation plane (q, d, s) is bit-identical to the oracle's;
  * every matmul output matrix satisfies max|gpu - oracle| <= 1e-4 * max|oracle|
    over the compared elements (the oracle is the exact result rounded once
    to f32; the GPU accumulates in f32 in its own order).
Full-size workloads compare sampled token rows (all N outputs of each
sampled token, tile edges and the ragged tail included); small shapes compare
everything.
"""
import numpy as np
import pytest

import oracle
import quant_gemm_amd as mq
from blocks import q4k_pack, q5k_pack, q6k_pack
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


def gpu_plane(x_np):
    q, d, s = mq.quantize_act(to_dev(x_np))
    return q, d, s


def check_close(got, ref, what):
    ref = np.asarray(ref, dtype=np.float64)
    got = np.asarray(got, dtype=np.float64)
    assert got.shape == ref.shape, what
    assert np.all(np.isfinite(got)), what
    scale = np.abs(ref).max()
    err = np.abs(got - ref).max()
    assert err <= TOL * scale, f"{what}: max|d|={err:.3e} > {TOL}*{scale:.3e}"
    return err / max(scale, 1e-300)


GPU_MM = {"q4k": mq.matmul_q4k, "q5k": mq.matmul_q5k, "q6k": mq.matmul_q6k}
ORACLE_MM = {"q4k": oracle.matmul_q4k, "q5k": oracle.matmul_q5k, "q6k": oracle.matmul_q6k}


def run_matmul(fmt, W_np, q, d, s, N, K, path=mq.MQ_PATH_AUTO):
    W = to_dev(W_np.reshape(-1))
    return GPU_MM[fmt](W, q, d, None if fmt == "q6k" else s, N, K, path=path)


def oracle_mm(fmt, W_np, q_np, d_np, N, K, tokens=None):
    return ORACLE_MM[fmt](W_np, q_np, d_np, N, K, tokens=tokens)


FMT_SEED = {"q4k": 0, "q6k": 1, "q5k": 2}


# ---------------------------------------------------------------- quantizer

_QSHAPES = [(8, 1024), (1, 3584), (3314, 3584), (1, 18944), (512, 18944), (3314, 18944), (7, 256)]


@pytest.mark.parametrize("M,K", _QSHAPES)
def test_quantizer_bit_exact(dev, M, K):
    rng = np.random.default_rng(M * 7 + K)
    x = synth.activations(rng, M, K, outliers=K >= 3584)
    q, d, s = gpu_plane(x)
    rq, rd, rs = oracle.quantize_act(x)
    assert np.array_equal(host(q), rq)
    assert np.array_equal(host(d).view(np.uint32), rd.view(np.uint32))
    assert np.array_equal(host(s).view(np.uint32), rs.view(np.uint32))


def test_quantizer_edge_values(dev):
    rng = np.random.default_rng(5)
    K = 512
    x = rng.standard_normal((12, K)).astype(np.float32)
    x[0] = 0.0                                          # all-zero rows
    x[1, :32] = np.float32(127.0)
    x[1, 32:64] = np.array([127.0] + [2.5, -2.5, 0.5, -0.5, 1.5, -1.5] * 5 + [126.5], np.float32)
    x[2] *= np.float32(1e-30)                           # tiny amax
    x[3] *= np.float32(1e-39)                           # subnormal inputs
    x[4] *= np.float32(3e37)                            # near the top of the f32 range
    x[5] = -x[6]                                        # sign symmetry
    x[7] = 0.0
    x[7, ::32] = np.float32(1e-45)                      # amax/127 underflows to 0
    x[7, 64] = np.float32(2e-43)                        # amax/127 is a subnormal
    x[8] = np.round(x[8] * 10) / 10                     # many ties after scaling
    x[9, 5] = np.float32(-1000.0)                       # one outlier
    q, d, s = gpu_plane(x)
    rq, rd, rs = oracle.quantize_act(x)
    assert np.array_equal(host(q), rq)
    assert np.array_equal(host(d).view(np.uint32), rd.view(np.uint32))
    assert np.array_equal(host(s).view(np.uint32), rs.view(np.uint32))


def test_quantizer_strided_rows(dev):
    """ldx > K, including a row stride that is not a multiple of 4 (scalar path)."""
    import torch
    rng = np.random.default_rng(6)
    for ldx in (1024 + 4, 1024 + 3):
        xw = rng.standard_normal((5, ldx)).astype(np.float32)
        xt = to_dev(xw)[:, :1024]
        assert xt.stride(0) == ldx
        q, d, s = mq.quantize_act(xt)
        rq, rd, rs = oracle.quantize_act(np.ascontiguousarray(xw[:, :1024]))
        assert np.array_equal(host(q), rq)
        assert np.array_equal(host(d), rd) and np.array_equal(host(s), rs)
    del torch


# ---------------------------------------------------------------- small shapes, full compare

SMALL = [(1, 1, 256), (2, 7, 512), (3, 33, 256), (5, 129, 768), (8, 256, 1024),
         (9, 31, 256), (31, 100, 512), (127, 129, 256), (129, 300, 1280), (200, 64, 2048)]


@pytest.mark.parametrize("fmt", ["q4k", "q5k", "q6k"])
@pytest.mark.parametrize("M,N,K", SMALL)
def test_small_shapes_all_paths(dev, fmt, M, N, K):
    rng = np.random.default_rng(M * 10007 + N * 101 + K + FMT_SEED[fmt])
    W = synth.weights(fmt, rng, N, K)
    x = synth.activations(rng, M, K, outliers=True)
    q, d, s = gpu_plane(x)
    rq, rd, _ = oracle.quantize_act(x)
    ref = oracle_mm(fmt, W, rq, rd, N, K)
    paths = [mq.MQ_PATH_AUTO, mq.MQ_PATH_GEMM]
    if M <= mq.gemv_max_m():
        paths.append(mq.MQ_PATH_GEMV)
    for p in paths:
        out = host(run_matmul(fmt, W, q, d, s, N, K, path=p))
        check_close(out, ref, f"{fmt} M={M} N={N} K={K} path={p}")



# Shapes whose tile count is small against the chip, so the GEMM cuts K into
# several ranges (uneven ones included) and sums the partial planes.
@pytest.mark.parametrize("fmt,M,N,K", [("q4k", 64, 2000, 3584), ("q4k", 40, 130, 6912),
                                       ("q6k", 300, 700, 4608), ("q6k", 17, 257, 2560),
                                       ("q5k", 200, 900, 4608), ("q5k", 24, 300, 5120)])
def test_split_k_shapes(dev, fmt, M, N, K):
    rng = np.random.default_rng(M * 7919 + N + K)
    W = synth.weights(fmt, rng, N, K)
    x = synth.activations(rng, M, K, outliers=True)
    rq, rd, _ = oracle.quantize_act(x)
    q, d, s = gpu_plane(x)
    ref = oracle_mm(fmt, W, rq, rd, N, K)
    got = host(run_matmul(fmt, W, q, d, s, N, K, path=mq.MQ_PATH_GEMM))
    check_close(got, ref, f"{fmt} M={M} N={N} K={K}")
    again = host(run_matmul(fmt, W, q, d, s, N, K, path=mq.MQ_PATH_GEMM))
    assert np.array_equal(got, again), "split-K result must not depend on scheduling"


def test_workspace_reuse_across_streams(dev):
    """Split-K GEMMs keep their partial sums in the workspace the caller
    gives each call (here torch's allocator on the call's stream): calls
    queued back to back on two streams (no host synchronization in
    between), small, large and small again, give the bits the same calls
    give one at a time."""
    import torch
    cases = []
    for fmt, M, N, K in [("q4k", 40, 130, 6912), ("q6k", 300, 700, 4608), ("q4k", 64, 2000, 3584),
                         ("q6k", 17, 257, 2560)]:
        rng = np.random.default_rng(M * 7919 + N + K)
        W = synth.weights(fmt, rng, N, K)
        q, d, s = gpu_plane(synth.activations(rng, M, K, outliers=True))
        cases.append((fmt, to_dev(W.reshape(-1)), q, d, s, N, K))
    fmt_code = {"q4k": mq.MQ_FMT_Q4K, "q6k": mq.MQ_FMT_Q6K}
    for c in cases:
        assert mq.matmul_workspace(fmt_code[c[0]], c[2].shape[0], c[5], c[6], mq.MQ_PATH_GEMM) > 0, c[0]
    mm = {"q4k": lambda W, q, d, s, N, K, st: mq.matmul_q4k(W, q, d, s, N, K, stream=st, path=mq.MQ_PATH_GEMM),
          "q6k": lambda W, q, d, s, N, K, st: mq.matmul_q6k(W, q, d, s, N, K, stream=st, path=mq.MQ_PATH_GEMM)}
    ref = [host(mm[c[0]](*c[1:], None)) for c in cases]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    outs = []
    for rep in range(3):
        for i, c in enumerate(cases):
            if (rep + i) % 2:
                with torch.cuda.stream(side):
                    outs.append((i, mm[c[0]](*c[1:], side)))
            else:
                outs.append((i, mm[c[0]](*c[1:], None)))
    torch.cuda.synchronize()
    for i, o in outs:
        assert np.array_equal(o.cpu().numpy(), ref[i]), f"case {i}: queued result differs"


def test_workspace_free_plan_matches(dev):
    """Without a workspace the GEMMs do not split K and the FFN runs its
    one-launch GEMM; both meet the bar against the oracle, and the split
    plan's result against the unsplit one."""
    rng = np.random.default_rng(91)
    for fmt, M, N, K in [("q4k", 40, 130, 6912), ("q6k", 300, 700, 4608), ("q5k", 24, 300, 5120)]:
        W = synth.weights(fmt, rng, N, K)
        x = synth.activations(rng, M, K, outliers=True)
        rq, rd, _ = oracle.quantize_act(x)
        q, d, s = gpu_plane(x)
        Wd = to_dev(W.reshape(-1))
        sp = None if fmt == "q6k" else s
        ref = oracle_mm(fmt, W, rq, rd, N, K)
        free = host(GPU_MM[fmt](Wd, q, d, sp, N, K, path=mq.MQ_PATH_GEMM, workspace=False))
        split = host(GPU_MM[fmt](Wd, q, d, sp, N, K, path=mq.MQ_PATH_GEMM))
        check_close(free, ref, f"{fmt} M={M} workspace-free")
        check_close(split, ref, f"{fmt} M={M} split")
    from oracle import producers
    M, N, K = 5, 512, 1024
    Wg, Wu = synth.q4k_weights(rng, N, K), synth.q4k_weights(rng, N, K)
    x = synth.activations(rng, M, K, outliers=True)
    rq, rd, _ = oracle.quantize_act(x)
    q, d, s = gpu_plane(x)
    _, _, _, ry = producers.ffn_q4k(Wg, Wu, rq, rd, N, K)
    import torch
    y = torch.empty((M, N), dtype=torch.float32, device="cuda")
    fq, fd, _, y = mq.ffn_q4k(to_dev(Wg.reshape(-1)), to_dev(Wu.reshape(-1)), q, d, s, N, K, y=y, workspace=False)
    check_close(host(y), ry, "ffn workspace-free")
    cq, cd, _ = oracle.quantize_act(host(y))
    assert np.array_equal(host(fq), cq) and np.array_equal(host(fd), cd)


def test_graph_capture_on_fresh_stream(dev):
    """A split-K GEMM and the two-pass FFN captured into a HIP graph on a
    stream no call has used before (their workspaces come from the graph's
    own memory pool during capture). Each of three replays runs on the
    capture stream with eager split-K GEMMs queued right behind it on the
    same stream, with no host synchronization in between; the replay's
    outputs and the eager ones each equal their one-at-a-time results bit
    for bit. Eager work and synchronizations separate the replays."""
    import torch
    rng = np.random.default_rng(77)
    M, N, K = 40, 130, 6912                       # split-K shape
    W = synth.q4k_weights(rng, N, K)
    q, d, s = gpu_plane(synth.activations(rng, M, K, outliers=True))
    Wd = to_dev(W.reshape(-1))
    Mf, Nf, Kf = 12, 512, 1024                    # two-pass FFN (GEMMs)
    Wg, Wu = to_dev(synth.q4k_weights(rng, Nf, Kf).reshape(-1)), to_dev(synth.q4k_weights(rng, Nf, Kf).reshape(-1))
    qf, df, sf = gpu_plane(synth.activations(rng, Mf, Kf, outliers=True))
    big_M, big_N, big_K = 300, 700, 4608          # eager split-K work on the capture stream
    Wb = to_dev(synth.q6k_weights(rng, big_N, big_K).reshape(-1))
    qb, db, sb = gpu_plane(synth.activations(rng, big_M, big_K, outliers=True))
    assert mq.matmul_workspace(mq.MQ_FMT_Q4K, M, N, K, mq.MQ_PATH_GEMM) > 0
    assert mq.matmul_workspace(mq.MQ_FMT_Q6K, big_M, big_N, big_K, mq.MQ_PATH_GEMM) > 0
    assert mq.ffn_q4k_workspace(Mf, Nf, Kf, mq.MQ_PATH_GEMM) > 2 * Mf * Nf * 4

    out = torch.empty((M, N), dtype=torch.float32, device="cuda")
    ffn_out = [torch.empty((Mf, Nf), dtype=torch.int8, device="cuda"),
               torch.empty((Mf, Nf // 32), dtype=torch.float32, device="cuda"),
               torch.empty((Mf, Nf // 32), dtype=torch.float32, device="cuda")]
    ref = host(mq.matmul_q4k(Wd, q, d, s, N, K, path=mq.MQ_PATH_GEMM))
    rq, rdd, rss = (host(t) for t in mq.ffn_q4k(Wg, Wu, qf, df, sf, Nf, Kf, path=mq.MQ_PATH_GEMM))
    big_ref = host(mq.matmul_q6k(Wb, qb, db, sb, big_N, big_K, path=mq.MQ_PATH_GEMM))

    side = torch.cuda.Stream()                    # never used before the capture
    side.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        mq.matmul_q4k(Wd, q, d, s, N, K, out=out, path=mq.MQ_PATH_GEMM)
        mq.ffn_q4k(Wg, Wu, qf, df, sf, Nf, Kf, qo=ffn_out[0], do=ffn_out[1], so=ffn_out[2], path=mq.MQ_PATH_GEMM)
    for rep in range(3):
        out.zero_()
        for t in ffn_out:
            t.zero_()
        torch.cuda.synchronize()
        eager = []
        with torch.cuda.stream(side):
            g.replay()
            for _ in range(2):                    # queued behind the replay, no sync
                eager.append(mq.matmul_q6k(Wb, qb, db, sb, big_N, big_K, stream=side, path=mq.MQ_PATH_GEMM))
        torch.cuda.synchronize()
        assert np.array_equal(host(out), ref), f"replay {rep}: split-K GEMM differs"
        assert np.array_equal(host(ffn_out[0]), rq) and np.array_equal(host(ffn_out[1]), rdd) \
            and np.array_equal(host(ffn_out[2]), rss), f"replay {rep}: FFN plane differs"
        for e in eager:
            assert np.array_equal(host(e), big_ref), f"replay {rep}: eager split-K GEMM differs"


# The small-M band: token counts around the switches between the GEMV, the
# GEMM's 32-token tiles and its 128-token tiles, for every path.
@pytest.mark.parametrize("fmt", ["q4k", "q5k", "q6k"])
@pytest.mark.parametrize("M", [3, 5, 9, 16, 24, 32, 33, 64, 65, 96, 97])
def test_small_m_band(dev, fmt, M):
    N, K = 700, 2560
    rng = np.random.default_rng(M * 17 + FMT_SEED[fmt])
    W = synth.weights(fmt, rng, N, K)
    x = synth.activations(rng, M, K, outliers=True)
    rq, rd, _ = oracle.quantize_act(x)
    q, d, s = gpu_plane(x)
    ref = oracle_mm(fmt, W, rq, rd, N, K)
    paths = [mq.MQ_PATH_AUTO, mq.MQ_PATH_GEMM] + ([mq.MQ_PATH_GEMV] if M <= mq.gemv_max_m() else [])
    for path in paths:
        check_close(host(run_matmul(fmt, W, q, d, s, N, K, path=path)), ref, f"{fmt} M={M} path {path}")

def test_tiny_q4k_workload_exact(dev):
    case = synth.case_by_name("tiny_q4k")
    W = case.make_weights()
    x = case.make_activations()
    q, d, s = gpu_plane(x)
    rq, rd, _ = oracle.quantize_act(x)
    ref = oracle.matmul_q4k(W, rq, rd, case.N, case.K)
    for p in (mq.MQ_PATH_GEMV, mq.MQ_PATH_GEMM, mq.MQ_PATH_AUTO):
        check_close(host(run_matmul("q4k", W, q, d, s, case.N, case.K, path=p)), ref, f"tiny_q4k path={p}")


# ---------------------------------------------------------------- position probes

def _one_hot_rows(fmt):
    """256 weight rows; row p has a single nonzero weight, at position p,
    of value val[p] (Q5_K alternates values with and without the fifth bit)."""
    rows, val = [], np.zeros(256)
    for p in range(256):
        if fmt == "q4k":
            qv = np.zeros(256, int)
            qv[p] = val[p] = 1 + p % 15
            rows.append(q4k_pack(1.0, 0.0, [1] * 8, [0] * 8, qv))
        elif fmt == "q5k":
            qv = np.zeros(256, int)
            qv[p] = val[p] = (16, 31, 1 + p % 15, 17 + p % 15)[p % 4]
            rows.append(q5k_pack(1.0, 0.0, [1] * 8, [0] * 8, qv))
        else:
            qv = np.full(256, 32)
            qv[p] = 33 + p % 30
            val[p] = 1 + p % 30
            rows.append(q6k_pack(1.0, [1] * 16, qv))
    return np.stack(rows), val


@pytest.mark.parametrize("fmt", ["q4k", "q5k", "q6k"])
def test_one_hot_positions_gemm(dev, fmt):
    """Row n holds one nonzero quant at position n; token t is 127 e_t.
    out[t, n] != 0 exactly when t == n, for all 256 positions of a block."""
    K = N = M = 256
    W, val = _one_hot_rows(fmt)
    x = np.zeros((M, K), np.float32)
    x[np.arange(256), np.arange(256)] = 127.0
    q, d, s = gpu_plane(x)
    out = host(run_matmul(fmt, W, q, d, s, N, K, path=mq.MQ_PATH_GEMM))
    diag = np.diag(out).copy()
    assert np.array_equal(diag, 127.0 * val)
    off = out - np.diag(diag)
    assert not off.any()


@pytest.mark.parametrize("fmt", ["q4k", "q5k", "q6k"])
def test_one_hot_positions_gemv(dev, fmt):
    K, N = 256, 256
    W, val = _one_hot_rows(fmt)
    for t0 in range(0, 256, 8):
        x = np.zeros((8, K), np.float32)
        x[np.arange(8), t0 + np.arange(8)] = 127.0
        q, d, s = gpu_plane(x)
        out = host(run_matmul(fmt, W, q, d, s, N, K, path=mq.MQ_PATH_GEMV))
        nz = np.argwhere(out != 0)
        assert nz.tolist() == [[i, t0 + i] for i in range(8)]
        assert np.array_equal(out[np.arange(8), t0 + np.arange(8)], 127.0 * val[t0:t0 + 8])


# ---------------------------------------------------------------- invariants

@pytest.mark.parametrize("fmt", ["q4k", "q5k"])
def test_zero_quants_zero_dmin_give_zero(dev, fmt):
    rng = np.random.default_rng(9)
    N, K, M = 130, 512, 70
    W = synth.weights(fmt, rng, N, K).reshape(N, K // 256, -1)
    W[:, :, 16:] = 0                      # quants (and Q5_K's high bits)
    W[:, :, 2:4] = np.array([0.0], np.float16).view(np.uint8)
    x = rng.standard_normal((M, K)).astype(np.float32)
    q, d, s = gpu_plane(x)
    for p in (mq.MQ_PATH_GEMM, mq.MQ_PATH_AUTO):
        assert not host(run_matmul(fmt, W.reshape(N, -1), q, d, s, N, K, path=p)).any()
    q8, d8, s8 = gpu_plane(x[:8])
    assert not host(run_matmul(fmt, W.reshape(N, -1), q8, d8, s8, N, K, path=mq.MQ_PATH_GEMV)).any()


def test_determinism_and_streams(dev):
    import torch
    rng = np.random.default_rng(10)
    N, K, M = 300, 1024, 200
    W = synth.q4k_weights(rng, N, K)
    x = synth.activations(rng, M, K, outliers=True)
    q, d, s = gpu_plane(x)
    Wd = to_dev(W.reshape(-1))
    a = host(mq.matmul_q4k(Wd, q, d, s, N, K))
    b = host(mq.matmul_q4k(Wd, q, d, s, N, K))
    assert np.array_equal(a, b)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        c = mq.matmul_q4k(Wd, q, d, s, N, K, stream=side)
    side.synchronize()
    assert np.array_equal(a, c.cpu().numpy())


def test_cross_path_rows(dev):
    """Token rows computed alone (GEMV, M=1) agree with the same rows inside a large GEMM."""
    rng = np.random.default_rng(11)
    N, K, M = 500, 3584, 300
    for fmt in ("q4k", "q5k", "q6k"):
        W = synth.weights(fmt, rng, N, K)
        x = synth.activations(rng, M, K, outliers=True)
        q, d, s = gpu_plane(x)
        big = host(run_matmul(fmt, W, q, d, s, N, K))
        rq, rd, _ = oracle.quantize_act(x)
        for t in (0, 137, 299):
            q1, d1, s1 = gpu_plane(x[t:t + 1])
            one = host(run_matmul(fmt, W, q1, d1, s1, N, K))
            ref = oracle_mm(fmt, W, rq, rd, N, K, tokens=np.array([t]))
            check_close(one, ref, f"{fmt} single row {t}")
            check_close(big[t:t + 1], ref, f"{fmt} row {t} of M={M}")



def _both_paths(fmt, W, x, N, K, what):
    """GEMM on all rows and GEMV on the first 8, each against the oracle."""
    rq, rd, _ = oracle.quantize_act(x)
    q, d, s = gpu_plane(x)
    ref = oracle_mm(fmt, W, rq, rd, N, K)
    check_close(host(run_matmul(fmt, W, q, d, s, N, K, path=mq.MQ_PATH_GEMM)), ref, what + " GEMM")
    q8, d8, s8 = gpu_plane(x[:8])
    check_close(host(run_matmul(fmt, W, q8, d8, s8, N, K, path=mq.MQ_PATH_GEMV)), ref[:8], what + " GEMV")


@pytest.mark.parametrize("fmt", ["q4k", "q5k"])
def test_min_term_dominated(dev, fmt):
    """Outputs made mostly of the min term: large dmin, small d, and
    activations with a common offset so that the block sums are large."""
    rng = np.random.default_rng(12)
    N, K, M = 200, 2048, 150
    gen = synth.q4k_weights if fmt == "q4k" else synth.q5k_weights
    W = gen(rng, N, K, d_range=(1e-5, 2e-5), dmin_range=(5e-3, 1e-2))
    x = (rng.standard_normal((M, K)) + 3.0).astype(np.float32)
    _both_paths(fmt, W, x, N, K, "min-dominated")


def _log_uniform_f16(rng, shape, lo, hi):
    return np.exp(rng.uniform(np.log(lo), np.log(hi), size=shape)).astype(np.float16)


@pytest.mark.parametrize("fmt", ["q4k", "q5k", "q6k"])
def test_wide_scale_range(dev, fmt):
    """Block scales spread over the whole f16 range (subnormal to 6e4) and
    activation rows whose magnitudes differ by 2^+-40."""
    rng = np.random.default_rng(13)
    N, K, M = 96, 1536, 130
    W = synth.weights(fmt, rng, N, K).reshape(N, K // 256, -1)
    if fmt in ("q4k", "q5k"):
        W[:, :, 0:2] = _log_uniform_f16(rng, (N, K // 256), 1e-7, 6e4).view(np.uint8).reshape(N, K // 256, 2)
        W[:, :, 2:4] = _log_uniform_f16(rng, (N, K // 256), 1e-7, 6e4).view(np.uint8).reshape(N, K // 256, 2)
    else:
        W[:, :, 208:210] = _log_uniform_f16(rng, (N, K // 256), 1e-7, 6e4).view(np.uint8).reshape(N, K // 256, 2)
    x = rng.standard_normal((M, K)).astype(np.float32)
    x *= np.exp2(rng.integers(-40, 41, size=(M, 1))).astype(np.float32)
    W = W.reshape(N, -1)
    rq, rd, _ = oracle.quantize_act(x)
    q, d, s = gpu_plane(x)
    ref = oracle_mm(fmt, W, rq, rd, N, K)
    for path in (mq.MQ_PATH_GEMM, mq.MQ_PATH_GEMV):
        rows = slice(None) if path == mq.MQ_PATH_GEMM else slice(0, 8)
        if path == mq.MQ_PATH_GEMV:
            q, d, s = gpu_plane(x[:8])
        got = host(run_matmul(fmt, W, q, d, s, N, K, path=path))
        # one bar per token row: rows differ in scale by up to 2^80
        for t in range(got.shape[0]):
            check_close(got[t], ref[rows][t], f"{fmt} path {path} row {t}")

def test_q6k_zero_d_superblocks(dev):
    """Q6_K super-blocks with d = +0 or -0 among nonzero ones: they add
    nothing, whatever their quants and scales (the GEMMs keep their
    accumulators in units of the row's current d and zero such blocks'
    limbs). Covers a row whose first super-blocks are zero, one whose last
    ones are, one that is zero throughout, and the expansion planes."""
    rng = np.random.default_rng(14)
    N, K, M = 70, 2048, 130
    W = synth.q6k_weights(rng, N, K).reshape(N, K // 256, 210)
    zero = rng.random((N, K // 256)) < 0.3
    zero[0, :3] = True
    zero[1, -2:] = True
    zero[2, :] = True
    zero[3, :] = False
    neg = rng.random((N, K // 256)) < 0.5
    W[:, :, 208][zero] = 0
    W[:, :, 209][zero] = np.where(neg[zero], 0x80, 0x00)
    W = W.reshape(N, -1)
    x = synth.activations(rng, M, K, outliers=True)
    rq, rd, _ = oracle.quantize_act(x)
    ref = oracle_mm("q6k", W, rq, rd, N, K)
    assert np.all(ref[:, 2] == 0.0)
    q, d, s = gpu_plane(x)
    got = host(run_matmul("q6k", W, q, d, s, N, K, path=mq.MQ_PATH_GEMM))
    check_close(got, ref, "q6k GEMM, zero-d super-blocks")
    assert np.all(got[:, 2] == 0.0)
    Wd = to_dev(W.reshape(-1))
    lo, hi, dw = mq.expand_q6k(Wd, N, K)
    gx = host(mq.matmul_q6k_x(lo, hi, dw, q, d, N, K))
    assert np.array_equal(gx, got), "planes and raw blocks: the same result bit for bit"
    q8, d8, s8 = gpu_plane(x[:8])
    gv = host(run_matmul("q6k", W, q8, d8, s8, N, K, path=mq.MQ_PATH_GEMV))
    check_close(gv, ref[:8], "q6k GEMV, zero-d super-blocks")


# ---------------------------------------------------------------- signed block scales

def _negate_scales(fmt, W, rng, frac=0.5):
    """Flip the f16 sign bit of d (and dmin for Q4_K / Q5_K) in a random half
    of the blocks, independently: GGML's quantizers may store a negative d,
    and the kernels rescale by it."""
    W = W.copy()
    blk = {"q4k": 144, "q5k": 176, "q6k": 210}[fmt]
    b = W.reshape(-1, blk)
    n = b.shape[0]
    if fmt == "q6k":
        b[rng.random(n) < frac, 209] ^= 0x80
    else:
        b[rng.random(n) < frac, 1] ^= 0x80
        b[rng.random(n) < frac, 3] ^= 0x80
    return W


@pytest.mark.parametrize("fmt", ["q4k", "q5k", "q6k"])
@pytest.mark.parametrize("M", [1, 4, 40, 200])
def test_signed_block_scales(dev, fmt, M):
    """Mixed-sign nonzero d and dmin: every path against the oracle."""
    N, K = 300, 2560
    rng = np.random.default_rng(4242 + M + FMT_SEED[fmt])
    W = _negate_scales(fmt, synth.weights(fmt, rng, N, K), rng)
    hdr = W.reshape(-1, {"q4k": 144, "q5k": 176, "q6k": 210}[fmt])
    sign = hdr[:, 209] if fmt == "q6k" else hdr[:, 1]
    assert (sign & 0x80).any() and not (sign & 0x80).all()
    x = synth.activations(rng, M, K, outliers=True)
    rq, rd, _ = oracle.quantize_act(x)
    q, d, s = gpu_plane(x)
    ref = oracle_mm(fmt, W, rq, rd, N, K)
    paths = [mq.MQ_PATH_AUTO, mq.MQ_PATH_GEMM] + ([mq.MQ_PATH_GEMV] if M <= mq.gemv_max_m() else [])
    for p in paths:
        check_close(host(run_matmul(fmt, W, q, d, s, N, K, path=p)), ref, f"{fmt} M={M} signed d, path {p}")


# ---------------------------------------------------------------- Q6_K rows at 4-byte alignment

@pytest.mark.parametrize("M", [1, 2, 8, 40, 300])
def test_q6k_weights_at_4_byte_offsets(dev, M):
    """A Q6_K matrix that starts one row into a larger one: rows of K = 3584
    are 2940 bytes, so row r starts 12, 8, 4, 0 bytes past a 16-byte
    boundary for r = 1, 2, 3, 4. Every path (the LDS-ring GEMV, the register
    GEMV, both GEMM tiles) and the expansion planes of the slice against the
    oracle on the same rows."""
    import torch
    N, K = 131, 3584
    rng = np.random.default_rng(515 + M)
    Wfull = synth.q6k_weights(rng, N + 4, K)
    x = synth.activations(rng, M, K, outliers=True)
    rq, rd, _ = oracle.quantize_act(x)
    q, d, s = gpu_plane(x)
    Wd = to_dev(Wfull.reshape(-1))
    rowb = Wfull.shape[1]
    for r0 in (1, 2, 3):
        Wsl = Wd[r0 * rowb:(r0 + N) * rowb]
        assert Wsl.data_ptr() % 16 == 16 - 4 * r0 and Wsl.data_ptr() % 4 == 0
        ref = oracle_mm("q6k", np.ascontiguousarray(Wfull[r0:r0 + N]), rq, rd, N, K)
        paths = [mq.MQ_PATH_AUTO, mq.MQ_PATH_GEMM] + ([mq.MQ_PATH_GEMV] if M <= mq.gemv_max_m() else [])
        for p in paths:
            got = host(mq.matmul_q6k(Wsl, q, d, None, N, K, path=p))
            check_close(got, ref, f"q6k slice at row {r0} M={M} path {p}")
        lo, hi, dw = mq.expand_q6k(Wsl, N, K)
        check_close(host(mq.matmul_q6k_x(lo, hi, dw, q, d, N, K)), ref, f"q6k_x slice at row {r0} M={M}")
    del torch


# ---------------------------------------------------------------- full-size workloads

_SAMPLE_TOKENS = [0, 1, 2, 63, 64, 127, 128, 129, 511, 1000, 2047, 2048, 3199, 3200, 3201, 3250, 3312, 3313]


def _tokens_for(M):
    t = sorted({x for x in _SAMPLE_TOKENS if x < M} | {M - 1})
    return np.array(t, dtype=np.int64)


# Workloads compared over every output (the oracle takes a few seconds for
# each on the host cores); the others on the sampled token rows.
_FULL_COMPARE = {"q4k_prefill_ffn_up", "layer_down", "q4k_prefill_ffn_up_n2368"}


@pytest.mark.parametrize("name", [c.name for _, c in synth.all_cases()])
def test_full_size_workloads(dev, name):
    case = synth.case_by_name(name)
    print(f"[parity] {case.name} {case.fmt} M={case.M} N={case.N} K={case.K}", flush=True)
    W = case.make_weights()
    x = case.make_activations()
    q, d, s = gpu_plane(x)
    rq, rd, rs = oracle.quantize_act(x)
    assert np.array_equal(host(q), rq) and np.array_equal(host(d), rd) and np.array_equal(host(s), rs)
    out_t = run_matmul(case.fmt, W, q, d, s, case.N, case.K)
    toks = None if case.M <= 8 or name in _FULL_COMPARE else _tokens_for(case.M)
    ref = oracle_mm(case.fmt, W, rq, rd, case.N, case.K, tokens=toks)
    out = host(out_t)
    got = out if toks is None else out[toks]
    rel = check_close(got, ref, case.name)
    print(f"[parity] {case.name}: max|d|/max|ref| = {rel:.2e}", flush=True)


# Long rows (K >= 8192): the GEMVs give each wavefront one row and stream it
# in double-buffered batches; ragged N and several token counts.
@pytest.mark.parametrize("fmt", ["q4k", "q5k", "q6k"])
@pytest.mark.parametrize("M,N,K", [(1, 300, 18944), (2, 300, 18944), (3, 77, 8192), (8, 129, 18944),
                                   (16, 40, 10240)])
def test_long_rows_gemv(dev, fmt, M, N, K):
    rng = np.random.default_rng(M * 131 + N + K + FMT_SEED[fmt])
    W = synth.weights(fmt, rng, N, K)
    x = synth.activations(rng, M, K, outliers=True)
    rq, rd, _ = oracle.quantize_act(x)
    q, d, s = gpu_plane(x)
    ref = oracle_mm(fmt, W, rq, rd, N, K)
    for path in (mq.MQ_PATH_GEMV, mq.MQ_PATH_AUTO):
        check_close(host(run_matmul(fmt, W, q, d, s, N, K, path=path)), ref, f"{fmt} M={M} N={N} K={K} path {path}")


def test_time_next_kernel(dev):
    """The timing hook records the kernel's own start and end: a positive
    duration, the same result as an untimed call, and the request is used
    once (a later call leaves the events untouched)."""
    import ctypes
    import os
    import torch
    lib = ctypes.CDLL(os.path.join(os.path.dirname(torch.__file__), "lib", "libamdhip64.so"))
    lib.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
    lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
    lib.hipEventDestroy.argtypes = [ctypes.c_void_p]
    ev = [ctypes.c_void_p(), ctypes.c_void_p()]
    for e in ev:
        assert lib.hipEventCreateWithFlags(ctypes.byref(e), 0) == 0
    rng = np.random.default_rng(21)
    N, K, M = 4096, 3584, 1
    W = synth.q4k_weights(rng, N, K)
    q, d, s = gpu_plane(synth.activations(rng, M, K))
    ref = host(run_matmul("q4k", W, q, d, s, N, K))
    Wd = to_dev(W.reshape(-1))
    for path in (mq.MQ_PATH_GEMV, mq.MQ_PATH_GEMM):
        mq.time_next_kernel(ev[0].value, ev[1].value)
        got = host(mq.matmul_q4k(Wd, q, d, s, N, K, path=path))
        ms = ctypes.c_float()
        assert lib.hipEventElapsedTime(ctypes.byref(ms), ev[0], ev[1]) == 0
        assert 0.0 < ms.value < 100.0, ms.value
        check_close(got, ref.astype(np.float64), f"timed path {path}")
        # the request was consumed: a second call does not touch the events
        host(mq.matmul_q4k(Wd, q, d, s, N, K, path=path))
        ms2 = ctypes.c_float()
        assert lib.hipEventElapsedTime(ctypes.byref(ms2), ev[0], ev[1]) == 0
        assert ms2.value == ms.value
    # the quantizer is covered too, also with events that skip the
    # system-scope fence (hipEventDisableSystemFence, as bench.py uses)
    evf = [ctypes.c_void_p(), ctypes.c_void_p()]
    for e in evf:
        assert lib.hipEventCreateWithFlags(ctypes.byref(e), 0x20000000) == 0
    x = synth.activations(rng, 300, K, outliers=True)
    q0, d0, s0 = (host(t) for t in gpu_plane(x))
    for pair in (ev, evf):
        mq.time_next_kernel(pair[0].value, pair[1].value)
        q1, d1, s1 = (host(t) for t in gpu_plane(x))
        ms = ctypes.c_float()
        assert lib.hipEventElapsedTime(ctypes.byref(ms), pair[0], pair[1]) == 0
        assert 0.0 < ms.value < 100.0, ms.value
        assert np.array_equal(q1, q0) and np.array_equal(d1, d0) and np.array_equal(s1, s0)
    for e in ev + evf:
        lib.hipEventDestroy(e)


# Row lengths served by the persistent stream kernels with 2, 3 and 6 passes
# per row (Q4_K up to K = 10752, Q5_K up to 6144), ragged N. Both stream up
# to 8 tokens while the plane fits their LDS copy (M = 4 at K <= 6144, M = 7
# at K = 4096); the other cases run the row-grid kernels.
@pytest.mark.parametrize("fmt,K", [("q4k", 4096), ("q4k", 5120), ("q4k", 8192), ("q4k", 10752),
                                   ("q5k", 4096), ("q5k", 5120), ("q5k", 6144)])
@pytest.mark.parametrize("M", [1, 2, 4, 7])
def test_stream_pass_counts(dev, fmt, K, M):
    N = 1000 + 7 * (K // 256)
    rng = np.random.default_rng(K + M + FMT_SEED[fmt])
    W = synth.weights(fmt, rng, N, K)
    x = synth.activations(rng, M, K, outliers=True)
    rq, rd, _ = oracle.quantize_act(x)
    q, d, s = gpu_plane(x)
    ref = oracle_mm(fmt, W, rq, rd, N, K)
    check_close(host(run_matmul(fmt, W, q, d, s, N, K, path=mq.MQ_PATH_GEMV)), ref, f"{fmt} M={M} K={K}")


# One token on long Q6_K rows (K >= 8192: the LDS ring kernel where its
# plane fits, the row kernel beyond), ragged row counts, one row, rows of
# 36 blocks (not a whole number of the ring's 16-block segments), and
# super-blocks with d = +0, -0 and negative d.
@pytest.mark.parametrize("N,K", [(1, 8192), (37, 9216), (333, 12800), (1000, 18944), (70, 65536)])
def test_q6k_gemv_long_rows(dev, N, K):
    rng = np.random.default_rng(N * 13 + K)
    W = synth.q6k_weights(rng, N, K).reshape(N, K // 256, 210)
    zero = rng.random((N, K // 256)) < 0.1
    W[:, :, 208][zero] = 0
    W[:, :, 209][zero] = np.where(rng.random(zero.sum()) < 0.5, 0x80, 0x00)
    neg = (rng.random((N, K // 256)) < 0.3) & ~zero
    W[:, :, 209][neg] ^= 0x80
    W = W.reshape(N, -1)
    x = synth.activations(rng, 1, K, outliers=True)
    print(f"[q6k long rows] M=1 N={N} K={K}", flush=True)
    rq, rd, _ = oracle.quantize_act(x)
    ref = oracle_mm("q6k", W, rq, rd, N, K)
    q, d, s = gpu_plane(x)
    for path in (mq.MQ_PATH_AUTO, mq.MQ_PATH_GEMV):
        got = host(run_matmul("q6k", W, q, d, s, N, K, path=path))
        check_close(got, ref, f"q6k long rows N={N} K={K} path {path}")
        again = host(run_matmul("q6k", W, q, d, s, N, K, path=path))
        assert np.array_equal(got, again), "bitwise repeatable"
