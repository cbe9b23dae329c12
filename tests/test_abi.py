"""The C ABI on the host (no GPU needed).

libmq.so must load, export every function include/mq.h declares, and reject
every invalid argument with its documented status and a message naming the
argument, before any HIP call. Every call here fails validation, so nothing
reaches a device (fake pointers are never dereferenced).
"""
import os
import re

import pytest

import quant_gemm_amd as mq

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mq.h")

OK, INVALID, SHAPE, ALIGN, WORKSPACE = 0, 1, 2, 3, 7
P = 0x7f0000000000          # a 256-byte aligned fake device address


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mq_\w+)\s*\(", text)))


@pytest.fixture(scope="module")
def L():
    return mq.load()


def test_header_declares_the_boundary():
    names = declared_functions()
    for n in ("mq_quantize_act", "mq_matmul_q4k", "mq_matmul_q6k", "mq_last_error"):
        assert n in names
    assert set(names) == set(mq.SIGNATURES)


def test_library_exports_every_declared_symbol(L):
    for name in declared_functions():
        assert hasattr(L, name), name


def test_abi_version_and_constants(L):
    assert L.mq_abi_version() == mq.ABI_VERSION
    assert L.mq_gemv_max_m() >= 1
    hdr = open(HEADER).read()
    assert f"#define MQ_ABI_VERSION {mq.ABI_VERSION}" in hdr
    assert f"#define MQ_Q6K_EXPAND_MIN_M {mq.Q6K_EXPAND_MIN_M}" in hdr
    assert mq.Q6K_EXPAND_MAX_WEIGHTS == 1 << 28 and "#define MQ_Q6K_EXPAND_MAX_WEIGHTS (1ll << 28)" in hdr


def _q4k(L, W=P, q=P, d=P, s=P, M=4, N=8, K=256, out=P, path=0):
    return L.mq_matmul_q4k_ex(W, q, d, s, M, N, K, out, None, path)


def _q5k(L, W=P, q=P, d=P, s=P, M=4, N=8, K=256, out=P, path=0):
    return L.mq_matmul_q5k_ex(W, q, d, s, M, N, K, out, None, path)


def _q6k(L, W=P, q=P, d=P, s=None, M=4, N=8, K=256, out=P, path=0):
    return L.mq_matmul_q6k_ex(W, q, d, s, M, N, K, out, None, path)


def _quant(L, x=P, M=4, K=256, ldx=256, q=P, d=P, s=P):
    return L.mq_quantize_act(x, M, K, ldx, q, d, s, None)


@pytest.mark.parametrize("kw,status,needle", [
    (dict(W=None), INVALID, "W is NULL"),
    (dict(q=None), INVALID, "q is NULL"),
    (dict(d=None), INVALID, "d is NULL"),
    (dict(s=None), INVALID, "s is NULL"),
    (dict(out=None), INVALID, "out is NULL"),
    (dict(M=0), INVALID, "M=0"),
    (dict(M=-3), INVALID, "M=-3"),
    (dict(N=0), INVALID, "N=0"),
    (dict(K=0), SHAPE, "K=0"),
    (dict(K=100), SHAPE, "K=100"),
    (dict(K=384), SHAPE, "K=384"),
    (dict(M=2 ** 31), SHAPE, "M=2147483648"),
    (dict(N=0x7fff0001), SHAPE, "N=2147418113"),
    (dict(path=3), INVALID, "path=3"),
    (dict(path=1, M=17), INVALID, "M=17"),
    (dict(W=P + 4), ALIGN, "W="),
    (dict(q=P + 8), ALIGN, "q="),
    (dict(d=P + 4), ALIGN, "d="),
    (dict(s=P + 12), ALIGN, "s="),
    (dict(out=P + 2), ALIGN, "out="),
])
def test_q4k_validation(L, kw, status, needle):
    rc = _q4k(L, **kw)
    assert rc == status
    msg = L.mq_last_error().decode()
    assert "mq_matmul_q4k" in msg and needle in msg


@pytest.mark.parametrize("kw,status,needle", [
    (dict(W=None), INVALID, "W is NULL"),
    (dict(s=None), INVALID, "s is NULL"),
    (dict(K=512 + 128), SHAPE, "K=640"),
    (dict(M=0), INVALID, "M=0"),
    (dict(path=1, M=17), INVALID, "M=17"),
    (dict(W=P + 8), ALIGN, "W="),
    (dict(out=P + 2), ALIGN, "out="),
])
def test_q5k_validation(L, kw, status, needle):
    rc = _q5k(L, **kw)
    assert rc == status
    msg = L.mq_last_error().decode()
    assert "mq_matmul_q5k" in msg and needle in msg
    assert L.mq_matmul_q5k(P, P, P, None, 4, 8, 256, P, None) == INVALID


@pytest.mark.parametrize("kw,status,needle", [
    (dict(W=None), INVALID, "W is NULL"),
    (dict(K=512 + 128), SHAPE, "K=640"),
    (dict(N=-1), INVALID, "N=-1"),
    (dict(W=P + 2), ALIGN, "W="),
    (dict(s=P + 4), ALIGN, "s="),
])
def test_q6k_validation(L, kw, status, needle):
    rc = _q6k(L, **kw)
    assert rc == status
    msg = L.mq_last_error().decode()
    assert "mq_matmul_q6k" in msg and needle in msg


@pytest.mark.parametrize("kw,status,needle", [
    (dict(x=None), INVALID, "x is NULL"),
    (dict(q=None), INVALID, "q is NULL"),
    (dict(d=None), INVALID, "d is NULL"),
    (dict(s=None), INVALID, "s is NULL"),
    (dict(M=0), INVALID, "M=0"),
    (dict(K=96), SHAPE, "K=96"),
    (dict(ldx=255), SHAPE, "ldx=255"),
    (dict(x=P + 2), ALIGN, "x="),
    (dict(q=P + 4), ALIGN, "q="),
    (dict(M=2 ** 40), SHAPE, "M="),
])
def test_quantize_validation(L, kw, status, needle):
    rc = _quant(L, **kw)
    assert rc == status
    msg = L.mq_last_error().decode()
    assert "mq_quantize_act" in msg and needle in msg



def _rms(L, x=P, w=P, M=4, K=256, ldx=256, eps=1e-6, q=P, d=P, s=P, y=None):
    return L.mq_rmsnorm_quantize(x, w, M, K, ldx, eps, q, d, s, y, None)


def _swi(L, g=P, u=P, M=4, K=256, ldg=512, ldu=512, q=P, d=P, s=P, y=None):
    return L.mq_swiglu_quantize(g, u, M, K, ldg, ldu, q, d, s, y, None)


@pytest.mark.parametrize("kw,status,needle", [
    (dict(x=None), INVALID, "x is NULL"),
    (dict(w=None), INVALID, "w is NULL"),
    (dict(q=None), INVALID, "q is NULL"),
    (dict(M=0), INVALID, "M=0"),
    (dict(eps=-1.0), INVALID, "eps="),
    (dict(eps=float("nan")), INVALID, "eps="),
    (dict(eps=float("inf")), INVALID, "eps="),
    (dict(K=160), SHAPE, "K=160"),
    (dict(ldx=200), SHAPE, "ldx=200"),
    (dict(ldx=258), ALIGN, "ldx=258"),
    (dict(x=P + 4), ALIGN, "x="),
    (dict(w=P + 8), ALIGN, "w="),
    (dict(s=P + 4), ALIGN, "s="),
    (dict(y=P + 4), ALIGN, "y="),
])
def test_rmsnorm_quantize_validation(L, kw, status, needle):
    rc = _rms(L, **kw)
    assert rc == status
    msg = L.mq_last_error().decode()
    assert "mq_rmsnorm_quantize" in msg and needle in msg


@pytest.mark.parametrize("kw,status,needle", [
    (dict(g=None), INVALID, "g is NULL"),
    (dict(u=None), INVALID, "u is NULL"),
    (dict(d=None), INVALID, "d is NULL"),
    (dict(M=-1), INVALID, "M=-1"),
    (dict(K=300), SHAPE, "K=300"),
    (dict(ldg=128), SHAPE, "ldg=128"),
    (dict(ldu=255), SHAPE, "ldu=255"),
    (dict(ldu=258), ALIGN, "ldu=258"),
    (dict(g=P + 4), ALIGN, "g="),
    (dict(u=P + 12), ALIGN, "u="),
    (dict(q=P + 1), ALIGN, "q="),
    (dict(y=P + 8), ALIGN, "y="),
    (dict(M=2 ** 40), SHAPE, "M="),
])
def test_swiglu_quantize_validation(L, kw, status, needle):
    rc = _swi(L, **kw)
    assert rc == status
    msg = L.mq_last_error().decode()
    assert "mq_swiglu_quantize" in msg and needle in msg


def _ffn(L, Wg=P, Wu=P, q=P, d=P, s=P, M=4, N=256, K=256, qo=P, do=P, so=P, y=None, path=0):
    return L.mq_ffn_q4k_ex(Wg, Wu, q, d, s, M, N, K, qo, do, so, y, None, path)


@pytest.mark.parametrize("kw,status,needle", [
    (dict(Wg=None), INVALID, "Wg is NULL"),
    (dict(Wu=None), INVALID, "Wu is NULL"),
    (dict(s=None), INVALID, "s is NULL"),
    (dict(qo=None), INVALID, "qo is NULL"),
    (dict(so=None), INVALID, "so is NULL"),
    (dict(M=0), INVALID, "M=0"),
    (dict(N=128), SHAPE, "N=128"),
    (dict(N=0), SHAPE, "N=0"),
    (dict(K=320), SHAPE, "K=320"),
    (dict(path=5), INVALID, "path=5"),
    (dict(path=1, M=9), INVALID, "M=9"),
    (dict(Wu=P + 2), ALIGN, "Wu="),
    (dict(qo=P + 4), ALIGN, "qo="),
    (dict(y=P + 4), ALIGN, "y="),
])
def test_ffn_validation(L, kw, status, needle):
    rc = _ffn(L, **kw)
    assert rc == status
    msg = L.mq_last_error().decode()
    assert "mq_ffn_q4k" in msg and needle in msg

def test_error_is_cleared_by_next_call(L):
    assert _q4k(L, W=None) == INVALID
    assert L.mq_last_error().decode() != ""
    assert _q6k(L, N=0) == INVALID
    assert "N=0" in L.mq_last_error().decode()


# ---------------------------------------------------------------- registration-time planes

@pytest.mark.parametrize("call,status,needle", [
    (lambda L: L.mq_expand_q6k(None, 8, 256, P, P, P, None), INVALID, "W is NULL"),
    (lambda L: L.mq_expand_q6k(P, 0, 256, P, P, P, None), INVALID, "N=0"),
    (lambda L: L.mq_expand_q6k(P, 8, 300, P, P, P, None), SHAPE, "K=300"),
    (lambda L: L.mq_expand_q6k(P, 8, 256, None, P, P, None), INVALID, "lo is NULL"),
    (lambda L: L.mq_expand_q6k(P, 8, 256, P, P + 4, P, None), ALIGN, "hi="),
    (lambda L: L.mq_expand_q6k(P, 8, 256, P, P, P + 8, None), ALIGN, "dw="),
    (lambda L: L.mq_matmul_q6k_x(P, P, None, P, P, 4, 8, 256, P, None, 0, None), INVALID, "dw is NULL"),
    (lambda L: L.mq_matmul_q6k_x(P, P, P, P, P, 0, 8, 256, P, None, 0, None), INVALID, "M=0"),
    (lambda L: L.mq_matmul_q6k_x(P, P, P, P, P, 4, 8, 512 + 64, P, None, 0, None), SHAPE, "K=576"),
    (lambda L: L.mq_matmul_q6k_x(P + 8, P, P, P, P, 4, 8, 256, P, None, 0, None), ALIGN, "lo="),
    (lambda L: L.mq_matmul_q6k_x(P, P, P, P + 4, P, 4, 8, 256, P, None, 0, None), ALIGN, "q="),
    (lambda L: L.mq_dsc_q4k(P, 8, 256, None, P, None), INVALID, "fw is NULL"),
    (lambda L: L.mq_dsc_q4k(P + 4, 8, 256, P, P, None), ALIGN, "W="),
    (lambda L: L.mq_dsc_q4k(P, 8, 256, P, P + 4, None), ALIGN, "fm="),
    (lambda L: L.mq_matmul_q4k_dsc(P, P, P, P, P, None, 4, 8, 256, P, None, 0, None), INVALID, "s is NULL"),
    (lambda L: L.mq_matmul_q4k_dsc(P, None, P, P, P, P, 4, 8, 256, P, None, 0, None), INVALID, "fw is NULL"),
    (lambda L: L.mq_matmul_q4k_dsc(P, P, P, P, P, P, 4, -2, 256, P, None, 0, None), INVALID, "N=-2"),
    (lambda L: L.mq_matmul_q4k_dsc(P, P, P + 8, P, P, P, 4, 8, 256, P, None, 0, None), ALIGN, "fm="),
    (lambda L: L.mq_matmul_q4k_dsc(P, P, P, P, P, P, 4, 8, 256, P + 2, None, 0, None), ALIGN, "out="),
    (lambda L: L.mq_expand_q6k(P + 2, 8, 256, P, P, P, None), ALIGN, "W="),
    (lambda L: L.mq_matmul_q6k_x(P, P, P, P, P, 4, 8, 256, P, None, 16, None), INVALID, "ws is NULL"),
    (lambda L: L.mq_matmul_q4k_dsc(P, P, P, P, P, P, 4, 8, 256, P, P + 8, 64, None), ALIGN, "ws="),
    (lambda L: L.mq_matmul_q6k_x(P, P, P, P, P, 512, 3584, 18944, P, P, 4096, None), WORKSPACE, "needs"),
])
def test_plane_entry_validation(L, call, status, needle):
    assert call(L) == status
    assert needle in L.mq_last_error().decode()


def test_probe_library_exports_and_rejects_bad_arguments():
    """libmq_probes.so (the ceiling probes of bench.py --ceilings) exports its
    three entry points; malformed arguments return hipErrorInvalidValue (1)
    before any HIP call, so this runs without a GPU."""
    import ctypes
    from quant_gemm_amd import build as mq_build
    assert os.path.exists(mq_build.PROBES_LIB), "build() also builds libmq_probes.so"
    P = ctypes.CDLL(mq_build.PROBES_LIB)
    P.mqp_read.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int,
                           ctypes.c_void_p, ctypes.c_void_p]
    P.mqp_mix.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    dummy = ctypes.c_void_p(0x1000)
    assert P.mqp_read(0, 4, dummy, 1000, 64, dummy, None) == 1        # not a multiple of 1024
    assert P.mqp_read(0, 4, None, 1024, 64, dummy, None) == 1         # no source
    assert P.mqp_read(0, 4, dummy, 1024, 0, dummy, None) == 1         # empty grid
    assert P.mqp_mix(3, 0, 64, dummy, None) == 1                      # no iterations
    assert P.mqp_mix(3, 10, 64, None, None) == 1                      # no sink
    P.mqp_valu.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p,
                           ctypes.c_void_p]
    assert P.mqp_valu(3, 0, 64, dummy, dummy, None) == 1              # no iterations
    assert P.mqp_valu(3, 10, 64, None, dummy, None) == 1              # no sink
    assert P.mqp_valu(3, 10, 64, dummy, None, None) == 1              # no clock array
    assert P.mqp_valu(5, 10, 64, dummy, dummy, None) == 1             # no such kind


def test_bench_refuses_more_than_one_gpu():
    """bench.py measures one GPU: --gpus above 1 exits with status 2 and says
    why, before it touches a device."""
    import subprocess
    import sys
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2, (r.returncode, r.stderr[-400:])
    assert "one GPU" in r.stderr


# ---------------------------------------------------------------- caller-owned workspace

import ctypes  # noqa: E402


def _ws_bytes(L, fmt, M, N, K, path=0):
    n = ctypes.c_int64(-1)
    assert L.mq_matmul_workspace(fmt, M, N, K, path, ctypes.byref(n)) == OK
    return n.value


def test_workspace_query_matches_the_split_planes(L):
    """The query is nsplit * M * N * 4 bytes for a GEMM that splits K (a
    whole number of [M][N] f32 planes, 2..16 of them), 0 for the GEMV and
    for GEMMs with enough tiles (the 3314-token FFN shapes)."""
    for fmt, M, N, K in ((mq.MQ_FMT_Q6K, 384, 3584, 18944), (mq.MQ_FMT_Q4K, 64, 18944, 3584),
                         (mq.MQ_FMT_Q5K, 16, 18944, 3584), (mq.MQ_FMT_Q6K, 16, 3584, 18944)):
        b = _ws_bytes(L, fmt, M, N, K, path=mq.MQ_PATH_GEMM)
        plane = M * N * 4
        assert b % plane == 0 and 2 <= b // plane <= 16, (fmt, M, N, K, b)
    assert _ws_bytes(L, mq.MQ_FMT_Q4K, 3314, 18944, 3584) == 0
    assert _ws_bytes(L, mq.MQ_FMT_Q4K, 1, 18944, 3584) == 0          # GEMV
    assert _ws_bytes(L, mq.MQ_FMT_Q6K, 1, 3584, 18944) == 0


def test_workspace_query_q6k_expansion(L):
    """A Q6_K GEMM of at least 512 tokens on a matrix of at most 2^28
    weights also keeps W's expansion planes in its workspace: the query is
    the planes plus a whole number of split-K [M][N] f32 planes. Below 512
    tokens, on larger matrices and on the GEMV there are no planes."""
    assert mq.Q6K_EXPAND_MIN_M == 512
    for M, N, K in ((3314, 3584, 18944), (512, 300, 4608), (1100, 3584, 3584), (512, 3584, 18944)):
        b = _ws_bytes(L, mq.MQ_FMT_Q6K, M, N, K, path=mq.MQ_PATH_GEMM)
        split = b - mq.q6k_expansion_bytes(N, K)
        assert split == mq.matmul_split_workspace(mq.MQ_FMT_Q6K, M, N, K, mq.MQ_PATH_GEMM)
        assert split >= 0 and split % (M * N * 4) == 0 and split // (M * N * 4) in (0,) + tuple(range(2, 17)), \
            (M, N, K, b)
    for M, N, K in ((511, 300, 4608), (3314, 152064, 3584), (384, 3584, 18944)):
        b = _ws_bytes(L, mq.MQ_FMT_Q6K, M, N, K, path=mq.MQ_PATH_GEMM)
        assert b % (M * N * 4) == 0, (M, N, K, b)
        assert b == mq.matmul_split_workspace(mq.MQ_FMT_Q6K, M, N, K, mq.MQ_PATH_GEMM)
    # Q4_K and Q5_K never expand
    assert _ws_bytes(L, mq.MQ_FMT_Q4K, 3314, 18944, 3584) == 0


def test_workspace_query_validates_like_the_call(L):
    n = ctypes.c_int64(-1)
    assert L.mq_matmul_workspace(3, 4, 8, 256, 0, ctypes.byref(n)) == INVALID
    assert "fmt=3" in L.mq_last_error().decode()
    assert L.mq_matmul_workspace(mq.MQ_FMT_Q4K, 4, 8, 300, 0, ctypes.byref(n)) == SHAPE
    assert "mq_matmul_q4k" in L.mq_last_error().decode() and "K=300" in L.mq_last_error().decode()
    assert L.mq_matmul_workspace(mq.MQ_FMT_Q6K, 4, 8, 256, 0, None) == INVALID
    assert L.mq_ffn_q4k_workspace(4, 100, 256, 0, ctypes.byref(n)) == SHAPE
    assert L.mq_ffn_q4k_workspace(9, 256, 256, mq.MQ_PATH_GEMV, ctypes.byref(n)) == INVALID


def test_ffn_workspace_query(L):
    """The two-pass FFN keeps g and u (2 * M * N f32) in the workspace, plus
    the GEMMs' split planes above the GEMV band; the one-launch GEMM (above
    128 tokens) needs none."""
    n = ctypes.c_int64(-1)
    assert L.mq_ffn_q4k_workspace(1, 18944, 3584, 0, ctypes.byref(n)) == OK
    assert n.value == 2 * 1 * 18944 * 4
    assert L.mq_ffn_q4k_workspace(64, 18944, 3584, 0, ctypes.byref(n)) == OK
    gu = 2 * 64 * 18944 * 4
    assert n.value >= gu and (n.value - gu) % (64 * 18944 * 4) == 0
    assert L.mq_ffn_q4k_workspace(3314, 18944, 3584, 0, ctypes.byref(n)) == OK and n.value == 0


@pytest.mark.parametrize("fn,fmt,s", [("mq_matmul_q4k_ws", mq.MQ_FMT_Q4K, P),
                                      ("mq_matmul_q5k_ws", mq.MQ_FMT_Q5K, P),
                                      ("mq_matmul_q6k_ws", mq.MQ_FMT_Q6K, None)])
def test_matmul_workspace_errors(L, fn, fmt, s):
    """A workspace smaller than the query is MQ_ERR_WORKSPACE naming both
    sizes; ws NULL with a size, a negative size or a misaligned ws are
    argument errors. All fail before any HIP call."""
    f = getattr(L, fn)
    M, N, K = 384, 3584, 18944      # below the Q6_K expansion plan: the split part is all
    need = _ws_bytes(L, fmt, M, N, K, path=mq.MQ_PATH_GEMM)
    assert need > 0
    assert f(P, P, P, s, M, N, K, P, P, need - 16, None, mq.MQ_PATH_GEMM) == WORKSPACE
    msg = L.mq_last_error().decode()
    assert str(need) in msg and str(need - 16) in msg
    assert f(P, P, P, s, M, N, K, P, None, 64, None, 0) == INVALID
    assert f(P, P, P, s, M, N, K, P, P, -1, None, 0) == INVALID
    assert f(P, P, P, s, M, N, K, P, P + 4, need, None, 0) == ALIGN
    assert "ws=" in L.mq_last_error().decode()


def test_ffn_gemv_path_needs_a_workspace(L):
    rc = L.mq_ffn_q4k_ex(P, P, P, P, P, 1, 256, 256, P, P, P, None, None, mq.MQ_PATH_GEMV)
    assert rc == WORKSPACE and "needs a workspace" in L.mq_last_error().decode()
    rc = L.mq_ffn_q4k_ws(P, P, P, P, P, 1, 256, 256, P, P, P, None, P, 8, None, mq.MQ_PATH_GEMV)
    assert rc == WORKSPACE


def test_q6k_weights_need_only_4_byte_alignment(L):
    """Q6_K W is accepted at 4-byte alignment (a row slice of a matrix whose
    rows are 4 bytes mod 16); the call below then stops at the misaligned
    output, after W passed. Q4_K / Q5_K keep 16 bytes."""
    assert _q6k(L, W=P + 4, out=P + 2) == ALIGN
    assert "out=" in L.mq_last_error().decode()
    assert _q6k(L, W=P + 2) == ALIGN and "4-byte" in L.mq_last_error().decode()
    assert _q4k(L, W=P + 4) == ALIGN and "16-byte" in L.mq_last_error().decode()
