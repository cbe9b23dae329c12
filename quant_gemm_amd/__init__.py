"""quant_gemm_amd: the k-quant weight matmul on AMD MI355X (gfx950).

A thin ctypes binding over libmq's C ABI (include/mq.h). The functions keep
the C names without the ``mq_`` prefix, take torch device tensors and only
marshal arguments: every step of the computation runs in the HIP kernels of
libmq. torch provides device memory and streams. There is no CPU fallback:
if libmq.so is missing, ``load()`` raises.

    q, d, s = quantize_act(x)                  # x: f32 [M, K] on cuda
    q, d, s = rmsnorm_quantize(x, w, eps)      # plane of RMSNorm(x) * w
    q, d, s = swiglu_quantize(g, u)            # plane of SiLU(g) * u
    out = matmul_q4k(W, q, d, s, N, K)         # W: uint8 [N, K/256*144]
    out = matmul_q5k(W, q, d, s, N, K)         # W: uint8 [N, K/256*176]
    out = matmul_q6k(W, q, d, None, N, K)      # W: uint8 [N, K/256*210]
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmq.so")

MQ_PATH_AUTO, MQ_PATH_GEMV, MQ_PATH_GEMM = 0, 1, 2
MQ_FMT_Q4K, MQ_FMT_Q5K, MQ_FMT_Q6K = 0, 1, 2
STATUS_NAMES = {0: "MQ_OK", 1: "MQ_ERR_INVALID_ARG", 2: "MQ_ERR_SHAPE",
                3: "MQ_ERR_ALIGN", 4: "MQ_ERR_UNSUPPORTED", 5: "MQ_ERR_DEVICE",
                6: "MQ_ERR_LAUNCH", 7: "MQ_ERR_WORKSPACE"}
ABI_VERSION = 6
Q4K_BLOCK_BYTES = 144
Q5K_BLOCK_BYTES = 176
Q6K_BLOCK_BYTES = 210

# Exported symbols of libmq and their C signatures (see include/mq.h).
_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_I = ctypes.c_int
_MATMUL_ARGS = [_P, _P, _P, _P, _I64, _I64, _I64, _P, _P]
_MATMUL_WS_ARGS = [_P, _P, _P, _P, _I64, _I64, _I64, _P, _P, _I64, _P, _I]
_FFN_ARGS = [_P, _P, _P, _P, _P, _I64, _I64, _I64, _P, _P, _P, _P]
SIGNATURES = {
    "mq_quantize_act": ([_P, _I64, _I64, _I64, _P, _P, _P, _P], _I),
    "mq_rmsnorm_quantize": ([_P, _P, _I64, _I64, _I64, ctypes.c_float, _P, _P, _P, _P, _P], _I),
    "mq_swiglu_quantize": ([_P, _P, _I64, _I64, _I64, _I64, _P, _P, _P, _P, _P], _I),
    "mq_ffn_q4k": (_FFN_ARGS + [_P], _I),
    "mq_ffn_q4k_ex": (_FFN_ARGS + [_P, _I], _I),
    "mq_ffn_q4k_ws": (_FFN_ARGS + [_P, _I64, _P, _I], _I),
    "mq_ffn_q4k_workspace": ([_I64, _I64, _I64, _I, ctypes.POINTER(_I64)], _I),
    "mq_matmul_q4k": (_MATMUL_ARGS, _I),
    "mq_matmul_q5k": (_MATMUL_ARGS, _I),
    "mq_matmul_q6k": (_MATMUL_ARGS, _I),
    "mq_matmul_q4k_ex": (_MATMUL_ARGS + [_I], _I),
    "mq_matmul_q5k_ex": (_MATMUL_ARGS + [_I], _I),
    "mq_matmul_q6k_ex": (_MATMUL_ARGS + [_I], _I),
    "mq_matmul_q4k_ws": (_MATMUL_WS_ARGS, _I),
    "mq_matmul_q5k_ws": (_MATMUL_WS_ARGS, _I),
    "mq_matmul_q6k_ws": (_MATMUL_WS_ARGS, _I),
    "mq_matmul_workspace": ([_I, _I64, _I64, _I64, _I, ctypes.POINTER(_I64)], _I),
    "mq_matmul_q6k_static": (_MATMUL_ARGS, _I),
    "mq_expand_q6k": ([_P, _I64, _I64, _P, _P, _P, _P], _I),
    "mq_matmul_q6k_x": ([_P, _P, _P, _P, _P, _I64, _I64, _I64, _P, _P, _I64, _P], _I),
    "mq_dsc_q4k": ([_P, _I64, _I64, _P, _P, _P], _I),
    "mq_matmul_q4k_dsc": ([_P, _P, _P, _P, _P, _P, _I64, _I64, _I64, _P, _P, _I64, _P], _I),
    "mq_time_next_kernel": ([_P, _P], _I),
    "mq_gemv_max_m": ([], _I64),
    "mq_last_error": ([], ctypes.c_char_p),
    "mq_abi_version": ([], _I),
}


class MQError(RuntimeError):
    """A libmq call returned a nonzero status."""

    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {message}")
        self.status = status


_lib = None


def load() -> ctypes.CDLL:
    """Load libmq.so (once). torch is imported first so that libmq binds to
    the HIP runtime torch already loaded."""
    global _lib
    if _lib is not None:
        return _lib
    import torch  # noqa: F401  (must precede the load: one HIP runtime per process)
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            f"{LIB_PATH} is not built; build it with `python -m quant_gemm_amd.build` "
            "(there is no fallback implementation)")
    L = ctypes.CDLL(LIB_PATH)
    for name, (argtypes, restype) in SIGNATURES.items():
        f = getattr(L, name)
        f.argtypes = argtypes
        f.restype = restype
    if L.mq_abi_version() != ABI_VERSION:
        raise RuntimeError(f"libmq ABI {L.mq_abi_version()} != binding ABI {ABI_VERSION}")
    _lib = L
    return L


def last_error() -> str:
    return load().mq_last_error().decode()


def _check(rc: int) -> None:
    if rc != 0:
        raise MQError(rc, last_error())


# Argument checks. The C ABI receives pointers and sizes only, so these are
# what keeps a wrongly sized tensor from reaching a kernel: explicit
# exceptions (not asserts, which `python -O` strips).
def _need(cond, msg, exc=ValueError):
    if not cond:
        raise exc(msg)


def _tensor(name, t, dtype, shape=None, contiguous=True, cuda=True):
    """t is a tensor of dtype (on a GPU), of the given shape, contiguous."""
    import torch
    _need(isinstance(t, torch.Tensor), f"{name} must be a torch.Tensor, got {type(t).__name__}", TypeError)
    _need(t.dtype == dtype, f"{name} must be {dtype}, got {t.dtype}", TypeError)
    if cuda:
        _need(t.is_cuda, f"{name} must be a GPU tensor (device {t.device})")
    if shape is not None:
        _need(tuple(t.shape) == tuple(shape), f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if contiguous:
        _need(t.is_contiguous(), f"{name} must be contiguous")


def _rows(name, t, dtype):
    """t is a 2-D tensor of dtype on a GPU with unit column stride."""
    _tensor(name, t, dtype, contiguous=False)
    _need(t.dim() == 2, f"{name} must be 2-D, got {t.dim()}-D")
    _need(t.stride(1) == 1, f"{name} must have unit column stride, got {t.stride(1)}")


def _weights(name, W, N, K, block_bytes):
    import torch
    _tensor(name, W, torch.uint8)
    _need(K > 0 and K % 256 == 0, f"K={K} must be a positive multiple of 256")
    _need(W.numel() == N * (K // 256) * block_bytes,
          f"{name} holds {W.numel()} bytes, N={N} rows of K={K} need {N * (K // 256) * block_bytes}")


def _plane(q, d, s, K, s_required=True):
    """(q, d, s) is an activation plane of row length K; returns M."""
    import torch
    _tensor("q", q, torch.int8)
    _need(q.dim() == 2 and q.shape[1] == K, f"q has shape {tuple(q.shape)}, expected (M, {K})")
    M = q.shape[0]
    _tensor("d", d, torch.float32, (M, K // 32))
    if s is not None or s_required:
        _tensor("s", s, torch.float32, (M, K // 32))
    return M


def _torch_stream(stream):
    import torch
    if stream is None:
        return torch.cuda.current_stream()
    if isinstance(stream, torch.cuda.Stream):
        return stream
    return torch.cuda.ExternalStream(int(stream))


def _stream(stream):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _workspace(nbytes, device, stream, given=None):
    """The caller-owned workspace of one call: None when the plan needs
    none; else `given` or a fresh uint8 tensor from torch's
    allocator on the call's stream, so that torch keeps it from other
    streams until the call's work is done."""
    import torch
    if nbytes == 0:
        return None
    if given is not None:
        _tensor("workspace", given, torch.uint8)
        return given            # the library checks its size (MQ_ERR_WORKSPACE)
    with torch.cuda.stream(_torch_stream(stream)):
        return torch.empty(nbytes, dtype=torch.uint8, device=device)


def _ws_args(ws):
    return (None, 0) if ws is None else (ws.data_ptr(), ws.numel())


def matmul_workspace(fmt, M, N, K, path=MQ_PATH_AUTO) -> int:
    """Bytes of workspace a matmul of format fmt (MQ_FMT_Q4K / Q5K / Q6K)
    with these sizes and path needs (0 when its plan needs none)."""
    n = ctypes.c_int64()
    _check(load().mq_matmul_workspace(fmt, M, N, K, path, ctypes.byref(n)))
    return n.value


# A Q6_K GEMM of at least Q6K_EXPAND_MIN_M tokens on a matrix of at most
# Q6K_EXPAND_MAX_WEIGHTS weights, given its full workspace, expands W there
# (mq.h: MQ_Q6K_EXPAND_MIN_M, MQ_Q6K_EXPAND_MAX_WEIGHTS).
Q6K_EXPAND_MIN_M = 512
Q6K_EXPAND_MAX_WEIGHTS = 1 << 28


def q6k_expansion_bytes(N, K) -> int:
    """Bytes the expansion planes of an N x K Q6_K matrix take in a
    workspace (lo, hi and d, each rounded up to 256)."""
    r = lambda v: (v + 255) // 256 * 256
    return 2 * r(N * K) + r(N * (K // 256) * 4)


def matmul_split_workspace(fmt, M, N, K, path=MQ_PATH_AUTO) -> int:
    """Bytes of the split-K part of a matmul's workspace: the query's figure,
    less the expansion planes where the call would expand W. A workspace of
    this size runs a Q6_K GEMM on the raw blocks, with the same result."""
    full = matmul_workspace(fmt, M, N, K, path)
    if (fmt == MQ_FMT_Q6K and path != MQ_PATH_GEMV and M >= Q6K_EXPAND_MIN_M
            and N * K <= Q6K_EXPAND_MAX_WEIGHTS):
        return full - q6k_expansion_bytes(N, K)
    return full


def ffn_q4k_workspace(M, N, K, path=MQ_PATH_AUTO) -> int:
    """Bytes of workspace mq_ffn_q4k_ws needs for these sizes and path."""
    n = ctypes.c_int64()
    _check(load().mq_ffn_q4k_workspace(M, N, K, path, ctypes.byref(n)))
    return n.value


def gemv_max_m() -> int:
    return int(load().mq_gemv_max_m())


def quantize_act(x, q=None, d=None, s=None, stream=None):
    """Per-32 int8 quantization of x (f32 [M, K], row stride x.stride(0)).

    Returns (q int8 [M, K], d f32 [M, K/32], s f32 [M, K/32]); preallocated
    outputs may be passed in.
    """
    import torch
    L = load()
    _rows("x", x, torch.float32)
    M, K = x.shape
    q, d, s = _plane_outputs(M, K, x.device, q, d, s)
    _check(L.mq_quantize_act(x.data_ptr(), M, K, x.stride(0), q.data_ptr(),
                             d.data_ptr(), s.data_ptr(), _stream(stream)))
    return q, d, s


def _plane_outputs(M, K, device, q, d, s):
    import torch
    _need(K % 32 == 0, f"K={K} must be a multiple of 32")
    if q is None:
        q = torch.empty((M, K), dtype=torch.int8, device=device)
    if d is None:
        d = torch.empty((M, K // 32), dtype=torch.float32, device=device)
    if s is None:
        s = torch.empty((M, K // 32), dtype=torch.float32, device=device)
    _tensor("q", q, torch.int8, (M, K))
    _tensor("d", d, torch.float32, (M, K // 32))
    _tensor("s", s, torch.float32, (M, K // 32))
    return q, d, s


def rmsnorm_quantize(x, w, eps, q=None, d=None, s=None, y=None, stream=None):
    """The int8 plane of RMSNorm(x) * w (x f32 [M, K], row stride x.stride(0);
    w f32 [K]). Returns (q, d, s), plus y f32 [M, K] (the normalised values)
    when a y tensor is passed."""
    import torch
    L = load()
    _rows("x", x, torch.float32)
    M, K = x.shape
    _tensor("w", w, torch.float32, (K,))
    q, d, s = _plane_outputs(M, K, x.device, q, d, s)
    if y is not None:
        _tensor("y", y, torch.float32, (M, K))
    _check(L.mq_rmsnorm_quantize(x.data_ptr(), w.data_ptr(), M, K, x.stride(0), float(eps),
                                 q.data_ptr(), d.data_ptr(), s.data_ptr(),
                                 None if y is None else y.data_ptr(), _stream(stream)))
    return (q, d, s) if y is None else (q, d, s, y)


def swiglu_quantize(g, u, q=None, d=None, s=None, y=None, stream=None):
    """The int8 plane of SiLU(g) * u (g, u f32 [M, K] with their own row
    strides, e.g. the two halves of a gate|up output). Returns (q, d, s),
    plus y when a y tensor is passed."""
    import torch
    L = load()
    _rows("g", g, torch.float32)
    _rows("u", u, torch.float32)
    _need(g.shape == u.shape, f"g {tuple(g.shape)} and u {tuple(u.shape)} differ in shape")
    M, K = g.shape
    q, d, s = _plane_outputs(M, K, g.device, q, d, s)
    if y is not None:
        _tensor("y", y, torch.float32, (M, K))
    _check(L.mq_swiglu_quantize(g.data_ptr(), u.data_ptr(), M, K, g.stride(0), u.stride(0),
                                q.data_ptr(), d.data_ptr(), s.data_ptr(),
                                None if y is None else y.data_ptr(), _stream(stream)))
    return (q, d, s) if y is None else (q, d, s, y)


def _out(out, M, N, device):
    import torch
    if out is None:
        out = torch.empty((M, N), dtype=torch.float32, device=device)
    _tensor("out", out, torch.float32, (M, N))
    return out


def _matmul(fmt, W, q, d, s, N, K, out, stream, path, workspace):
    name = {MQ_FMT_Q4K: "q4k", MQ_FMT_Q5K: "q5k", MQ_FMT_Q6K: "q6k"}[fmt]
    block = {MQ_FMT_Q4K: Q4K_BLOCK_BYTES, MQ_FMT_Q5K: Q5K_BLOCK_BYTES, MQ_FMT_Q6K: Q6K_BLOCK_BYTES}[fmt]
    L = load()
    _weights("W", W, N, K, block)
    M = _plane(q, d, s, K, s_required=fmt != MQ_FMT_Q6K)
    out = _out(out, M, N, q.device)
    sp = None if s is None else s.data_ptr()
    if workspace is False:
        f = getattr(L, f"mq_matmul_{name}_ex")
        _check(f(W.data_ptr(), q.data_ptr(), d.data_ptr(), sp, M, N, K, out.data_ptr(), _stream(stream), path))
        return out
    ws = _workspace(matmul_workspace(fmt, M, N, K, path), q.device, stream,
                    None if workspace is True else workspace)
    f = getattr(L, f"mq_matmul_{name}_ws")
    _check(f(W.data_ptr(), q.data_ptr(), d.data_ptr(), sp, M, N, K, out.data_ptr(), *_ws_args(ws),
             _stream(stream), path))
    return out


def matmul_q4k(W, q, d, s, N, K, out=None, stream=None, path=MQ_PATH_AUTO, workspace=True):
    """out [M, N] f32 = Q4_K weights W (N rows of K) times the activation plane (q, d, s).

    workspace: True (default) gives the call the workspace its full plan
    needs, allocated through torch; a uint8 tensor is used as given; False
    runs the workspace-free plan (mq_matmul_q4k_ex: no split of K)."""
    return _matmul(MQ_FMT_Q4K, W, q, d, s, N, K, out, stream, path, workspace)


def matmul_q5k(W, q, d, s, N, K, out=None, stream=None, path=MQ_PATH_AUTO, workspace=True):
    """out [M, N] f32 = Q5_K weights W (N rows of K) times the activation plane (q, d, s)."""
    return _matmul(MQ_FMT_Q5K, W, q, d, s, N, K, out, stream, path, workspace)


def matmul_q6k(W, q, d, s, N, K, out=None, stream=None, path=MQ_PATH_AUTO, workspace=True):
    """out [M, N] f32 = Q6_K weights W (N rows of K) times the activation plane (q, d); s unused."""
    return _matmul(MQ_FMT_Q6K, W, q, d, s, N, K, out, stream, path, workspace)


STATIC_SCRATCH_BYTES = 32 << 20


def matmul_q6k_static(W, q, d, N, K, out=None, stream=None):
    """matmul_q6k without any allocation: split-K partial sums in the
    library's static device array (STATIC_SCRATCH_BYTES per GPU). Calls that
    overlap in time on one GPU race; a plan needing more raises
    MQError(MQ_ERR_WORKSPACE)."""
    L = load()
    _weights("W", W, N, K, Q6K_BLOCK_BYTES)
    M = _plane(q, d, None, K, s_required=False)
    out = _out(out, M, N, q.device)
    _check(L.mq_matmul_q6k_static(W.data_ptr(), q.data_ptr(), d.data_ptr(), None, M, N, K, out.data_ptr(),
                                  _stream(stream)))
    return out


def expand_q6k(W, N, K, lo=None, hi=None, dw=None, stream=None):
    """Q6_K expansion planes of W (uint8, N rows of K): (lo, hi) int8 [N, K]
    and dw f32 [N, K/256], for matmul_q6k_x."""
    import torch
    L = load()
    _weights("W", W, N, K, Q6K_BLOCK_BYTES)
    lo = torch.empty((N, K), dtype=torch.int8, device=W.device) if lo is None else lo
    hi = torch.empty((N, K), dtype=torch.int8, device=W.device) if hi is None else hi
    dw = torch.empty((N, K // 256), dtype=torch.float32, device=W.device) if dw is None else dw
    _tensor("lo", lo, torch.int8, (N, K))
    _tensor("hi", hi, torch.int8, (N, K))
    _tensor("dw", dw, torch.float32, (N, K // 256))
    _check(L.mq_expand_q6k(W.data_ptr(), N, K, lo.data_ptr(), hi.data_ptr(), dw.data_ptr(), _stream(stream)))
    return lo, hi, dw


def matmul_q6k_x(lo, hi, dw, q, d, N, K, out=None, stream=None, workspace=True):
    """out [M, N] f32 from the Q6_K expansion planes and the activation plane (q, d)."""
    import torch
    L = load()
    _tensor("lo", lo, torch.int8, (N, K))
    _tensor("hi", hi, torch.int8, (N, K))
    _tensor("dw", dw, torch.float32, (N, K // 256))
    M = _plane(q, d, None, K, s_required=False)
    out = _out(out, M, N, q.device)
    ws = None
    if workspace is not False:
        ws = _workspace(matmul_workspace(MQ_FMT_Q6K, M, N, K, MQ_PATH_GEMM), q.device, stream,
                        None if workspace is True else workspace)
    _check(L.mq_matmul_q6k_x(lo.data_ptr(), hi.data_ptr(), dw.data_ptr(), q.data_ptr(), d.data_ptr(),
                             M, N, K, out.data_ptr(), *_ws_args(ws), _stream(stream)))
    return out


def dsc_q4k(W, N, K, fw=None, fm=None, stream=None):
    """Q4_K decoded-scale planes of W: (fw, fm) f32 [N, K/32], for matmul_q4k_dsc."""
    import torch
    L = load()
    _weights("W", W, N, K, Q4K_BLOCK_BYTES)
    fw = torch.empty((N, K // 32), dtype=torch.float32, device=W.device) if fw is None else fw
    fm = torch.empty((N, K // 32), dtype=torch.float32, device=W.device) if fm is None else fm
    _tensor("fw", fw, torch.float32, (N, K // 32))
    _tensor("fm", fm, torch.float32, (N, K // 32))
    _check(L.mq_dsc_q4k(W.data_ptr(), N, K, fw.data_ptr(), fm.data_ptr(), _stream(stream)))
    return fw, fm


def matmul_q4k_dsc(W, fw, fm, q, d, s, N, K, out=None, stream=None, workspace=True):
    """out [M, N] f32 = Q4_K W times the plane (q, d, s), factors from (fw, fm)."""
    import torch
    L = load()
    _weights("W", W, N, K, Q4K_BLOCK_BYTES)
    _tensor("fw", fw, torch.float32, (N, K // 32))
    _tensor("fm", fm, torch.float32, (N, K // 32))
    M = _plane(q, d, s, K)
    out = _out(out, M, N, q.device)
    ws = None
    if workspace is not False:
        ws = _workspace(matmul_workspace(MQ_FMT_Q4K, M, N, K, MQ_PATH_GEMM), q.device, stream,
                        None if workspace is True else workspace)
    _check(L.mq_matmul_q4k_dsc(W.data_ptr(), fw.data_ptr(), fm.data_ptr(), q.data_ptr(), d.data_ptr(),
                               s.data_ptr(), M, N, K, out.data_ptr(), *_ws_args(ws), _stream(stream)))
    return out


def time_next_kernel(start_event, stop_event):
    """Have the next matmul call of this thread record the raw hipEvent_t
    handles start_event / stop_event (ints, or None) at its main kernel's own
    start and end (see mq_time_next_kernel)."""
    _check(load().mq_time_next_kernel(start_event, stop_event))


def ffn_q4k(Wg, Wu, q, d, s, N, K, qo=None, do=None, so=None, y=None, stream=None, path=MQ_PATH_AUTO,
            workspace=True):
    """The int8 plane of SiLU(x Wg^T) * (x Wu^T) for Q4_K gate and up weights
    (each N rows of K) and the activation plane (q, d, s). Returns (qo, do, so),
    plus y when a y tensor is passed. workspace as for matmul_q4k (False:
    the one-launch GEMM at every M)."""
    import torch
    L = load()
    _weights("Wg", Wg, N, K, Q4K_BLOCK_BYTES)
    _weights("Wu", Wu, N, K, Q4K_BLOCK_BYTES)
    M = _plane(q, d, s, K)
    qo, do, so = _plane_outputs(M, N, q.device, qo, do, so)
    if y is not None:
        _tensor("y", y, torch.float32, (M, N))
    args = (Wg.data_ptr(), Wu.data_ptr(), q.data_ptr(), d.data_ptr(), s.data_ptr(), M, N, K,
            qo.data_ptr(), do.data_ptr(), so.data_ptr(), None if y is None else y.data_ptr())
    if workspace is False:
        _check(L.mq_ffn_q4k_ex(*args, _stream(stream), path))
    else:
        ws = _workspace(ffn_q4k_workspace(M, N, K, path), q.device, stream,
                        None if workspace is True else workspace)
        _check(L.mq_ffn_q4k_ws(*args, *_ws_args(ws), _stream(stream), path))
    return (qo, do, so) if y is None else (qo, do, so, y)
