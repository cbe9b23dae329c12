"""GPU parity of the producer-fused quantizers (RMSNorm / SwiGLU -> int8
plane) against the oracle, through the C ABI.

Bars:
  * the plane the GPU writes is exactly the quantizer's plane of the f32
    values y the GPU computed (y is read back through the optional output);
  * RMSNorm: y is bit-identical to the oracle's (the scale comes from an
    exactly rounded sum on both sides), so the whole plane is too;
  * SwiGLU: y is within one f32 ulp of the oracle's everywhere (the f64 exp
    of the two sides may differ in its last bit; its f32 rounding then agrees
    except within 2^-29 of a rounding boundary), and every 32-value block
    whose y agrees has an identical plane.
"""
import numpy as np
import pytest

import oracle
from oracle import producers
import quant_gemm_amd as mq
from quant_gemm_amd import synth

pytestmark = pytest.mark.gpu


def to_dev(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda")


def host(t):
    import torch
    torch.cuda.synchronize()
    return t.cpu().numpy()


def gpu_rms(x, w, eps, ldx=None):
    import torch
    M, K = x.shape
    if ldx is None or ldx == K:
        xd = to_dev(x)
    else:
        buf = torch.zeros((M, ldx), dtype=torch.float32, device="cuda")
        buf[:, :K] = to_dev(x)
        xd = buf[:, :K]
    y = torch.empty((M, K), dtype=torch.float32, device="cuda")
    q, d, s, y = mq.rmsnorm_quantize(xd, to_dev(w), eps, y=y)
    q2, d2, s2 = mq.rmsnorm_quantize(xd, to_dev(w), eps)        # without the f32 output
    return host(q), host(d), host(s), host(y), host(q2), host(d2), host(s2)


def assert_plane_of(q, d, s, y, what):
    rq, rd, rs = oracle.quantize_act(y)
    assert np.array_equal(q, rq), f"{what}: plane differs from the quantizer of its own y"
    assert np.array_equal(d, rd) and np.array_equal(s, rs), what


RMS_SHAPES = [(1, 256, None), (7, 3584, None), (64, 1024, 1100), (33, 18944, None),
              (3314, 3584, None), (5, 8192, 8196), (2, 9216, None), (300, 1024, 1028),
              (256, 3840, None), (257, 4096, None), (301, 768, None)]


@pytest.mark.parametrize("M,K,ldx", RMS_SHAPES)
@pytest.mark.parametrize("eps", [1e-6, 0.0])
def test_rmsnorm_quantize_bit_exact(dev, M, K, ldx, eps):
    rng = np.random.default_rng(M * 31 + K + int(eps == 0))
    x = synth.activations(rng, M, K, outliers=True) * np.float32(rng.uniform(0.1, 10.0))
    w = (1.0 + 0.3 * rng.standard_normal(K)).astype(np.float32)
    print(f"[producers] rmsnorm M={M} K={K} ldx={ldx} eps={eps}", flush=True)
    q, d, s, y, q2, d2, s2 = gpu_rms(x, w, eps, ldx)
    rq, rd, rs, ry = producers.rmsnorm_quantize(x, w, eps)
    assert np.array_equal(y, ry), f"y differs in {np.count_nonzero(y != ry)} elements"
    assert np.array_equal(q, rq) and np.array_equal(d, rd) and np.array_equal(s, rs)
    assert np.array_equal(q2, q) and np.array_equal(d2, d) and np.array_equal(s2, s)


def _rows_near_scale_boundary(rng, M, K, eps):
    """Rows whose exact sum of squares puts r = f32(1/sqrt(ss/K + eps)) on the
    midpoint between two f32 values, to within about 2^-70 of ss: a sum of
    squares that is off by a few f64 ulps rounds r the other way. A random
    body is completed by three entries that take up the remainder."""
    import math
    eps64 = float(np.float32(eps))
    x = np.empty((M, K), np.float32)
    for t in range(M):
        r0 = np.float32(rng.uniform(0.3, 3.0))
        m = (float(r0) + float(np.nextafter(r0, np.float32(np.inf)))) / 2
        target = K * (1.0 / (m * m) - eps64)
        row = (rng.standard_normal(K) * 0.5 * math.sqrt(target / K)).astype(np.float32)
        pos = rng.choice(K, 3, replace=False)
        row[pos] = 0
        rest = target - math.fsum((row.astype(np.float64) ** 2).tolist())
        for p in pos:
            if rest <= 0:
                break
            a = np.float32(math.sqrt(rest))
            while float(a) ** 2 > rest:
                a = np.nextafter(a, np.float32(0))
            row[p] = a if rng.random() < 0.5 else -a
            rest -= float(a) ** 2
        x[t] = row
    return x


@pytest.mark.parametrize("M,K", [(27, 256), (300, 256), (27, 3584), (300, 3584), (9, 8192)])
@pytest.mark.parametrize("eps", [1e-6, 0.0])
def test_rmsnorm_scale_on_rounding_boundary(dev, M, K, eps):
    """Where r sits on an f32 rounding boundary only an exactly rounded sum of
    squares gives the oracle's r: the kernels' certified fast sum must notice
    and take the exact one."""
    import math
    rng = np.random.default_rng(M * 7 + K + int(eps == 0))
    x = _rows_near_scale_boundary(rng, M, K, eps)
    w = (1.0 + 0.3 * rng.standard_normal(K)).astype(np.float32)
    e64 = float(np.float32(eps))
    for t in range(M):                       # the construction holds: the rows are hard
        ss = math.fsum((x[t].astype(np.float64) ** 2).tolist())
        lo, hi = ss * (1 - 2.0 ** -46), ss * (1 + 2.0 ** -46)
        assert np.float32(1 / math.sqrt(lo / K + e64)) != np.float32(1 / math.sqrt(hi / K + e64))
    print(f"[producers] rmsnorm boundary rows M={M} K={K} eps={eps}", flush=True)
    q, d, s, y, q2, d2, s2 = gpu_rms(x, w, eps)
    rq, rd, rs, ry = producers.rmsnorm_quantize(x, w, eps)
    assert np.array_equal(y, ry), f"y differs in rows {np.nonzero((y != ry).any(axis=1))[0]}"
    assert np.array_equal(q, rq) and np.array_equal(d, rd) and np.array_equal(s, rs)


def test_rmsnorm_quantize_edge_rows(dev):
    K = 512
    rng = np.random.default_rng(5)
    x = rng.standard_normal((6, K)).astype(np.float32)
    x[0] = 0.0                                   # all zero: y = 0, plane zero
    x[1] = np.float32(1e-30)                     # far below sqrt(eps)
    x[2] = np.float32(3e18) * np.sign(x[2])      # large, squares near 1e37
    x[3, :] = 0.0
    x[3, 17] = -5.0                              # a single nonzero value
    x[4] *= np.float32(2.0 ** -60)               # tiny: eps dominates the scale
    w = rng.standard_normal(K).astype(np.float32)
    q, d, s, y, *_ = gpu_rms(x, w, 1e-6)
    rq, rd, rs, ry = producers.rmsnorm_quantize(x, w, 1e-6)
    assert np.array_equal(y, ry)
    assert np.array_equal(q, rq) and np.array_equal(d, rd) and np.array_equal(s, rs)
    assert not q[0].any() and not d[0].any()


def gpu_swiglu(g, u, concat):
    import torch
    M, K = g.shape
    if concat:
        buf = to_dev(np.concatenate([g, u], axis=1))       # gate|up output, [M][2K]
        gd, ud = buf[:, :K], buf[:, K:]
    else:
        gd, ud = to_dev(g), to_dev(u)
    y = torch.empty((M, K), dtype=torch.float32, device="cuda")
    q, d, s, y = mq.swiglu_quantize(gd, ud, y=y)
    q2, d2, s2 = mq.swiglu_quantize(gd, ud)
    return host(q), host(d), host(s), host(y), host(q2), host(d2), host(s2)


def check_swiglu(g, u, concat, what):
    q, d, s, y, q2, d2, s2 = gpu_swiglu(g, u, concat)
    assert_plane_of(q, d, s, y, what)
    assert np.array_equal(q2, q) and np.array_equal(d2, d) and np.array_equal(s2, s)
    rq, rd, rs, ry = producers.swiglu_quantize(g, u)
    ulp = np.spacing(np.maximum(np.abs(ry), np.abs(y)).astype(np.float32))
    assert np.all(np.abs(y.astype(np.float64) - ry.astype(np.float64)) <= ulp), what
    M, K = g.shape
    same = np.all((y == ry).reshape(M, K // 32, 32), axis=2)
    assert np.array_equal(q.reshape(M, K // 32, 32)[same], rq.reshape(M, K // 32, 32)[same]), what
    assert np.array_equal(d[same], rd[same]) and np.array_equal(s[same], rs[same]), what
    return np.count_nonzero(y != ry)


@pytest.mark.parametrize("M,K,concat", [(1, 18944, False), (5, 256, True), (512, 18944, True),
                                        (3314, 18944, True), (129, 3584, False)])
def test_swiglu_quantize(dev, M, K, concat):
    rng = np.random.default_rng(M + 7 * K)
    g = (rng.standard_normal((M, K)) * 2.5).astype(np.float32)
    u = synth.activations(rng, M, K, outliers=True)
    print(f"[producers] swiglu M={M} K={K} concat={concat}", flush=True)
    n = check_swiglu(g, u, concat, f"swiglu M={M} K={K}")
    print(f"[producers] swiglu M={M} K={K}: {n} f32 values differ by one ulp", flush=True)


def test_swiglu_quantize_edge_values(dev):
    K = 256
    vals = np.array([0.0, -0.0, 1.0, -1.0, 30.0, -30.0, 100.0, -100.0, 1e30, -1e30,
                     88.0, -88.0, 710.0, -710.0, 1e-30, -1e-30], np.float32)
    g = np.resize(vals, (4, K)).astype(np.float32)
    u = np.resize(np.array([1.0, -2.0, 0.5, 3e4, 1e-20, 0.0, 7.0, -1.0], np.float32), (4, K))
    check_swiglu(g, u, False, "edge values")
    # rows whose SiLU is zero everywhere give an all-zero plane
    q, d, s, y, *_ = gpu_swiglu(np.zeros((2, K), np.float32), u[:2], False)
    assert not q.any() and not d.any() and not s.any()


# ---------------------------------------------------------------- fused FFN up half

# Up to 128 tokens the FFN runs two passes (g and u into a workspace, then
# the SwiGLU quantizer): decode sizes whose plane fits the persistent stream
# run gate and up as one stream, longer rows (K = 11008, 12288) two GEMVs,
# path 2 the GEMMs (32-token tiles to 64 tokens, 128-token tiles at 100).
# Beyond 128 tokens (130, 3314) one GEMM launch with SwiGLU in its epilogue.
FFN_CASES = [(1, 256, 1024, (1, 2)), (3, 512, 3584, (1, 2)), (8, 768, 2048, (1, 2)),
             (8, 512, 3584, (1,)), (2, 512, 11008, (1,)), (4, 256, 12288, (1,)),
             (9, 256, 1024, (2,)), (100, 256, 2048, (2,)), (130, 512, 3584, (2,)),
             (1, 18944, 3584, (1,)), (3314, 18944, 3584, (2,))]


@pytest.mark.parametrize("M,N,K,paths", FFN_CASES)
def test_ffn_q4k(dev, M, N, K, paths):
    import torch
    rng = np.random.default_rng(M * 131 + N + K)
    Wg = synth.q4k_weights(rng, N, K)
    Wu = synth.q4k_weights(rng, N, K)
    x = synth.activations(rng, M, K, outliers=True)
    q, d, s = mq.quantize_act(to_dev(x))
    toks = None if M <= 130 else np.array([0, 1, 127, 128, 1000, 2047, 3200, M - 1])
    rq, rd, _ = oracle.quantize_act(x)
    _, _, _, ry = producers.ffn_q4k(Wg, Wu, rq, rd, N, K, tokens=toks)
    Wgd, Wud = to_dev(Wg.reshape(-1)), to_dev(Wu.reshape(-1))
    for path in paths:
        print(f"[producers] ffn M={M} N={N} K={K} path={path}", flush=True)
        y = torch.empty((M, N), dtype=torch.float32, device="cuda")
        qo, do, so, y = mq.ffn_q4k(Wgd, Wud, q, d, s, N, K, y=y, path=path)
        qo2, do2, so2 = mq.ffn_q4k(Wgd, Wud, q, d, s, N, K, path=path)
        qo, do, so, y = host(qo), host(do), host(so), host(y)
        assert_plane_of(qo, do, so, y, f"ffn path {path}")
        assert np.array_equal(host(qo2), qo) and np.array_equal(host(do2), do) and np.array_equal(host(so2), so)
        got = y if toks is None else y[toks]
        err = np.abs(got.astype(np.float64) - ry).max()
        bar = 1e-4 * np.abs(ry).max()
        assert err <= bar, f"ffn path {path}: max|d| {err:.3e} > {bar:.3e}"
        print(f"[producers] ffn M={M} N={N} K={K} path={path}: max|d|/max|y| = {err / np.abs(ry).max():.2e}", flush=True)

