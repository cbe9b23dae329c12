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
STATUS_NAMES = {0: "MQ_OK", 1: "MQ_ERR_INVALID_ARG", 2: "MQ_ERR_SHAPE",
                3: "MQ_ERR_ALIGN", 4: "MQ_ERR_UNSUPPORTED", 5: "MQ_ERR_DEVICE",
                6: "MQ_ERR_LAUNCH"}
ABI_VERSION = 3
Q4K_BLOCK_BYTES = 144
Q5K_BLOCK_BYTES = 176
Q6K_BLOCK_BYTES = 210

# Exported symbols of libmq and their C signatures (see include/mq.h).
_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_MATMUL_ARGS = [_P, _P, _P, _P, _I64, _I64, _I64, _P, _P]
SIGNATURES = {
    "mq_quantize_act": ([_P, _I64, _I64, _I64, _P, _P, _P, _P], ctypes.c_int),
    "mq_rmsnorm_quantize": ([_P, _P, _I64, _I64, _I64, ctypes.c_float, _P, _P, _P, _P, _P], ctypes.c_int),
    "mq_swiglu_quantize": ([_P, _P, _I64, _I64, _I64, _I64, _P, _P, _P, _P, _P], ctypes.c_int),
    "mq_ffn_q4k": ([_P, _P, _P, _P, _P, _I64, _I64, _I64, _P, _P, _P, _P, _P], ctypes.c_int),
    "mq_ffn_q4k_ex": ([_P, _P, _P, _P, _P, _I64, _I64, _I64, _P, _P, _P, _P, _P, ctypes.c_int], ctypes.c_int),
    "mq_matmul_q4k": (_MATMUL_ARGS, ctypes.c_int),
    "mq_matmul_q5k": (_MATMUL_ARGS, ctypes.c_int),
    "mq_matmul_q6k": (_MATMUL_ARGS, ctypes.c_int),
    "mq_matmul_q4k_ex": (_MATMUL_ARGS + [ctypes.c_int], ctypes.c_int),
    "mq_matmul_q5k_ex": (_MATMUL_ARGS + [ctypes.c_int], ctypes.c_int),
    "mq_matmul_q6k_ex": (_MATMUL_ARGS + [ctypes.c_int], ctypes.c_int),
    "mq_expand_q6k": ([_P, _I64, _I64, _P, _P, _P, _P], ctypes.c_int),
    "mq_matmul_q6k_x": ([_P, _P, _P, _P, _P, _I64, _I64, _I64, _P, _P], ctypes.c_int),
    "mq_dsc_q4k": ([_P, _I64, _I64, _P, _P, _P], ctypes.c_int),
    "mq_matmul_q4k_dsc": ([_P, _P, _P, _P, _P, _P, _I64, _I64, _I64, _P, _P], ctypes.c_int),
    "mq_time_next_kernel": ([_P, _P], ctypes.c_int),
    "mq_gemv_max_m": ([], ctypes.c_int64),
    "mq_last_error": ([], ctypes.c_char_p),
    "mq_abi_version": ([], ctypes.c_int),
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


def _stream(stream):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def gemv_max_m() -> int:
    return int(load().mq_gemv_max_m())


def quantize_act(x, q=None, d=None, s=None, stream=None):
    """Per-32 int8 quantization of x (f32 [M, K], row stride x.stride(0)).

    Returns (q int8 [M, K], d f32 [M, K/32], s f32 [M, K/32]); preallocated
    outputs may be passed in.
    """
    import torch
    L = load()
    assert x.is_cuda and x.dtype == torch.float32 and x.dim() == 2 and x.stride(1) == 1
    M, K = x.shape
    if q is None:
        q = torch.empty((M, K), dtype=torch.int8, device=x.device)
    if d is None:
        d = torch.empty((M, K // 32), dtype=torch.float32, device=x.device)
    if s is None:
        s = torch.empty((M, K // 32), dtype=torch.float32, device=x.device)
    assert q.is_contiguous() and d.is_contiguous() and s.is_contiguous()
    _check(L.mq_quantize_act(x.data_ptr(), M, K, x.stride(0), q.data_ptr(),
                             d.data_ptr(), s.data_ptr(), _stream(stream)))
    return q, d, s


def _plane_outputs(M, K, device, q, d, s):
    import torch
    if q is None:
        q = torch.empty((M, K), dtype=torch.int8, device=device)
    if d is None:
        d = torch.empty((M, K // 32), dtype=torch.float32, device=device)
    if s is None:
        s = torch.empty((M, K // 32), dtype=torch.float32, device=device)
    assert q.is_contiguous() and d.is_contiguous() and s.is_contiguous()
    return q, d, s


def rmsnorm_quantize(x, w, eps, q=None, d=None, s=None, y=None, stream=None):
    """The int8 plane of RMSNorm(x) * w (x f32 [M, K], row stride x.stride(0);
    w f32 [K]). Returns (q, d, s), plus y f32 [M, K] (the normalised values)
    when a y tensor is passed."""
    import torch
    L = load()
    assert x.is_cuda and x.dtype == torch.float32 and x.dim() == 2 and x.stride(1) == 1
    M, K = x.shape
    assert w.is_cuda and w.dtype == torch.float32 and w.is_contiguous() and w.numel() == K
    q, d, s = _plane_outputs(M, K, x.device, q, d, s)
    if y is not None:
        assert y.dtype == torch.float32 and y.is_contiguous() and tuple(y.shape) == (M, K)
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
    for a in (g, u):
        assert a.is_cuda and a.dtype == torch.float32 and a.dim() == 2 and a.stride(1) == 1
    assert g.shape == u.shape
    M, K = g.shape
    q, d, s = _plane_outputs(M, K, g.device, q, d, s)
    if y is not None:
        assert y.dtype == torch.float32 and y.is_contiguous() and tuple(y.shape) == (M, K)
    _check(L.mq_swiglu_quantize(g.data_ptr(), u.data_ptr(), M, K, g.stride(0), u.stride(0),
                                q.data_ptr(), d.data_ptr(), s.data_ptr(),
                                None if y is None else y.data_ptr(), _stream(stream)))
    return (q, d, s) if y is None else (q, d, s, y)


def _matmul(fn, block_bytes, W, q, d, s, N, K, out, stream, path):
    import torch
    L = load()
    assert W.is_cuda and W.dtype == torch.uint8 and W.is_contiguous()
    assert W.numel() == N * (K // 256) * block_bytes, "W size does not match N, K"
    assert q.dtype == torch.int8 and q.is_contiguous() and q.dim() == 2 and q.shape[1] == K
    M = q.shape[0]
    assert d.dtype == torch.float32 and d.is_contiguous() and tuple(d.shape) == (M, K // 32)
    if s is not None:
        assert s.dtype == torch.float32 and s.is_contiguous() and tuple(s.shape) == (M, K // 32)
    if out is None:
        out = torch.empty((M, N), dtype=torch.float32, device=q.device)
    assert out.dtype == torch.float32 and out.is_contiguous() and tuple(out.shape) == (M, N)
    f = getattr(L, fn)
    _check(f(W.data_ptr(), q.data_ptr(), d.data_ptr(), None if s is None else s.data_ptr(),
             M, N, K, out.data_ptr(), _stream(stream), path))
    return out


def matmul_q4k(W, q, d, s, N, K, out=None, stream=None, path=MQ_PATH_AUTO):
    """out [M, N] f32 = Q4_K weights W (N rows of K) times the activation plane (q, d, s)."""
    return _matmul("mq_matmul_q4k_ex", Q4K_BLOCK_BYTES, W, q, d, s, N, K, out, stream, path)


def matmul_q5k(W, q, d, s, N, K, out=None, stream=None, path=MQ_PATH_AUTO):
    """out [M, N] f32 = Q5_K weights W (N rows of K) times the activation plane (q, d, s)."""
    return _matmul("mq_matmul_q5k_ex", Q5K_BLOCK_BYTES, W, q, d, s, N, K, out, stream, path)


def matmul_q6k(W, q, d, s, N, K, out=None, stream=None, path=MQ_PATH_AUTO):
    """out [M, N] f32 = Q6_K weights W (N rows of K) times the activation plane (q, d); s unused."""
    return _matmul("mq_matmul_q6k_ex", Q6K_BLOCK_BYTES, W, q, d, s, N, K, out, stream, path)


def expand_q6k(W, N, K, lo=None, hi=None, dw=None, stream=None):
    """Q6_K expansion planes of W (uint8, N rows of K): (lo, hi) int8 [N, K]
    and dw f32 [N, K/256], for matmul_q6k_x."""
    import torch
    L = load()
    assert W.is_cuda and W.dtype == torch.uint8 and W.is_contiguous()
    assert W.numel() == N * (K // 256) * Q6K_BLOCK_BYTES, "W size does not match N, K"
    lo = torch.empty((N, K), dtype=torch.int8, device=W.device) if lo is None else lo
    hi = torch.empty((N, K), dtype=torch.int8, device=W.device) if hi is None else hi
    dw = torch.empty((N, K // 256), dtype=torch.float32, device=W.device) if dw is None else dw
    for t, dt, shp in ((lo, torch.int8, (N, K)), (hi, torch.int8, (N, K)), (dw, torch.float32, (N, K // 256))):
        assert t.dtype == dt and t.is_contiguous() and tuple(t.shape) == shp
    _check(L.mq_expand_q6k(W.data_ptr(), N, K, lo.data_ptr(), hi.data_ptr(), dw.data_ptr(), _stream(stream)))
    return lo, hi, dw


def matmul_q6k_x(lo, hi, dw, q, d, N, K, out=None, stream=None):
    """out [M, N] f32 from the Q6_K expansion planes and the activation plane (q, d)."""
    import torch
    L = load()
    assert lo.dtype == torch.int8 and hi.dtype == torch.int8 and dw.dtype == torch.float32
    assert tuple(lo.shape) == (N, K) and tuple(hi.shape) == (N, K) and tuple(dw.shape) == (N, K // 256)
    assert lo.is_contiguous() and hi.is_contiguous() and dw.is_contiguous()
    M = q.shape[0]
    assert q.dtype == torch.int8 and q.is_contiguous() and tuple(q.shape) == (M, K)
    assert d.dtype == torch.float32 and d.is_contiguous() and tuple(d.shape) == (M, K // 32)
    if out is None:
        out = torch.empty((M, N), dtype=torch.float32, device=q.device)
    assert out.dtype == torch.float32 and out.is_contiguous() and tuple(out.shape) == (M, N)
    _check(L.mq_matmul_q6k_x(lo.data_ptr(), hi.data_ptr(), dw.data_ptr(), q.data_ptr(), d.data_ptr(),
                             M, N, K, out.data_ptr(), _stream(stream)))
    return out


def dsc_q4k(W, N, K, fw=None, fm=None, stream=None):
    """Q4_K decoded-scale planes of W: (fw, fm) f32 [N, K/32], for matmul_q4k_dsc."""
    import torch
    L = load()
    assert W.is_cuda and W.dtype == torch.uint8 and W.is_contiguous()
    assert W.numel() == N * (K // 256) * Q4K_BLOCK_BYTES, "W size does not match N, K"
    fw = torch.empty((N, K // 32), dtype=torch.float32, device=W.device) if fw is None else fw
    fm = torch.empty((N, K // 32), dtype=torch.float32, device=W.device) if fm is None else fm
    for t in (fw, fm):
        assert t.dtype == torch.float32 and t.is_contiguous() and tuple(t.shape) == (N, K // 32)
    _check(L.mq_dsc_q4k(W.data_ptr(), N, K, fw.data_ptr(), fm.data_ptr(), _stream(stream)))
    return fw, fm


def matmul_q4k_dsc(W, fw, fm, q, d, s, N, K, out=None, stream=None):
    """out [M, N] f32 = Q4_K W times the plane (q, d, s), factors from (fw, fm)."""
    import torch
    L = load()
    assert W.is_cuda and W.dtype == torch.uint8 and W.is_contiguous()
    assert W.numel() == N * (K // 256) * Q4K_BLOCK_BYTES, "W size does not match N, K"
    for t in (fw, fm):
        assert t.dtype == torch.float32 and t.is_contiguous() and tuple(t.shape) == (N, K // 32)
    M = q.shape[0]
    assert q.dtype == torch.int8 and q.is_contiguous() and tuple(q.shape) == (M, K)
    for t in (d, s):
        assert t.dtype == torch.float32 and t.is_contiguous() and tuple(t.shape) == (M, K // 32)
    if out is None:
        out = torch.empty((M, N), dtype=torch.float32, device=q.device)
    assert out.dtype == torch.float32 and out.is_contiguous() and tuple(out.shape) == (M, N)
    _check(L.mq_matmul_q4k_dsc(W.data_ptr(), fw.data_ptr(), fm.data_ptr(), q.data_ptr(), d.data_ptr(),
                               s.data_ptr(), M, N, K, out.data_ptr(), _stream(stream)))
    return out


def time_next_kernel(start_event, stop_event):
    """Have the next matmul call of this thread record the raw hipEvent_t
    handles start_event / stop_event (ints, or None) at its main kernel's own
    start and end (see mq_time_next_kernel)."""
    _check(load().mq_time_next_kernel(start_event, stop_event))


def ffn_q4k(Wg, Wu, q, d, s, N, K, qo=None, do=None, so=None, y=None, stream=None, path=MQ_PATH_AUTO):
    """The int8 plane of SiLU(x Wg^T) * (x Wu^T) for Q4_K gate and up weights
    (each N rows of K) and the activation plane (q, d, s). Returns (qo, do, so),
    plus y when a y tensor is passed."""
    import torch
    L = load()
    for W in (Wg, Wu):
        assert W.is_cuda and W.dtype == torch.uint8 and W.is_contiguous()
        assert W.numel() == N * (K // 256) * Q4K_BLOCK_BYTES, "W size does not match N, K"
    assert q.dtype == torch.int8 and q.is_contiguous() and q.dim() == 2 and q.shape[1] == K
    M = q.shape[0]
    for t in (d, s):
        assert t.dtype == torch.float32 and t.is_contiguous() and tuple(t.shape) == (M, K // 32)
    qo, do, so = _plane_outputs(M, N, q.device, qo, do, so)
    if y is not None:
        assert y.dtype == torch.float32 and y.is_contiguous() and tuple(y.shape) == (M, N)
    _check(L.mq_ffn_q4k_ex(Wg.data_ptr(), Wu.data_ptr(), q.data_ptr(), d.data_ptr(), s.data_ptr(),
                           M, N, K, qo.data_ptr(), do.data_ptr(), so.data_ptr(),
                           None if y is None else y.data_ptr(), _stream(stream), path))
    return (qo, do, so) if y is None else (qo, do, so, y)

