"""ctypes binding of libfa.so: argument marshalling only.

Every step of the attention forward and backward passes runs in the HIP kernels of libfa.so; this
module checks tensor metadata, passes raw device pointers, sizes and the stream
handle, and turns status codes into exceptions. There is no fallback: if the
library is missing, importing the package fails.
"""

from __future__ import annotations

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libfa.so")

FA_OK = 0
FA_ERR_INVALID_ARGUMENT = 1
FA_ERR_UNSUPPORTED = 2
FA_ERR_MISALIGNED = 3
FA_ERR_LAUNCH = 4
FA_ERR_JIT = 5
FA_ERR_SCRATCH_LIMIT = 6
FA_DTYPE_F32 = 0
FA_DTYPE_BF16 = 1

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is not built; run `python -c 'import __graft_entry__ as g; g.build()'`")

_lib = ctypes.CDLL(LIB_PATH)
_lib.fa_fwd.restype = ctypes.c_int
_lib.fa_fwd.argtypes = [
    ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
    ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
    ctypes.c_int, ctypes.c_float, ctypes.c_void_p, ctypes.c_int,
]
_lib.fa_fwd_strided.restype = ctypes.c_int
_lib.fa_fwd_strided.argtypes = [ctypes.c_void_p] * 5 + [ctypes.c_int64] * 5 + [ctypes.c_void_p] * 5 + [
    ctypes.c_int, ctypes.c_float, ctypes.c_void_p, ctypes.c_int,
]
_lib.fa_fwd_specialized.restype = ctypes.c_int
_lib.fa_fwd_specialized.argtypes = _lib.fa_fwd.argtypes
_lib.fa_jit_code_object.restype = ctypes.c_int
_lib.fa_jit_code_object.argtypes = [ctypes.c_int, ctypes.c_int64, ctypes.c_int, ctypes.c_int64, ctypes.c_int64,
                                    ctypes.c_int64, ctypes.c_void_p, ctypes.POINTER(ctypes.c_size_t)]
_lib.fa_bwd.restype = ctypes.c_int
_lib.fa_bwd.argtypes = [ctypes.c_void_p] * 10 + [
    ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
    ctypes.c_int, ctypes.c_float, ctypes.c_void_p, ctypes.c_int,
]
_lib.fa_bwd_noalloc.restype = ctypes.c_int
_lib.fa_bwd_noalloc.argtypes = [ctypes.c_void_p] * 9 + [
    ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
    ctypes.c_int, ctypes.c_float, ctypes.c_void_p, ctypes.c_int,
]
_lib.fa_status_string.restype = ctypes.c_char_p
_lib.fa_status_string.argtypes = [ctypes.c_int]
_lib.fa_version.restype = ctypes.c_int
_lib.fa_version.argtypes = []


class FaError(RuntimeError):
    def __init__(self, status: int, entry: str = "fa_fwd"):
        super().__init__(f"{entry} failed: {fa_status_string(status)} (status {status})")
        self.status = status


def fa_status_string(status: int) -> str:
    return _lib.fa_status_string(int(status)).decode()


def fa_version() -> int:
    return int(_lib.fa_version())


def raw_fa_fwd(Q, K, V, O, L, B, H, N, d, causal, scale, stream, dtype) -> int:
    """The C entry point with integer pointers; returns the status code."""
    return int(_lib.fa_fwd(Q, K, V, O, L, B, H, N, d, int(causal), float(scale), stream, int(dtype)))


def raw_fa_fwd_specialized(Q, K, V, O, L, B, H, N, d, causal, scale, stream, dtype) -> int:
    """The shape-specialized C entry point with integer pointers; returns the status code."""
    return int(_lib.fa_fwd_specialized(Q, K, V, O, L, B, H, N, d, int(causal), float(scale), stream, int(dtype)))


def jit_code_object(dtype: int, d: int, causal: bool, B: int, H: int, N: int) -> bytes:
    """The code object fa_fwd_specialized compiles for this shape (no GPU needed)."""
    size = ctypes.c_size_t(0)
    st = _lib.fa_jit_code_object(int(dtype), d, int(causal), B, H, N, None, ctypes.byref(size))
    if st != FA_OK:
        raise FaError(st, "fa_jit_code_object")
    buf = ctypes.create_string_buffer(size.value)
    st = _lib.fa_jit_code_object(int(dtype), d, int(causal), B, H, N, buf, ctypes.byref(size))
    if st != FA_OK:
        raise FaError(st, "fa_jit_code_object")
    return buf.raw[: size.value]


def _strides3(st):
    """Three element strides as a C int64[3] (None passes NULL)."""
    if st is None:
        return None
    st = tuple(int(x) for x in st)
    if len(st) != 3:
        raise ValueError("expected three strides (batch, head, row)")
    return (ctypes.c_int64 * 3)(*st)


def raw_fa_fwd_strided(Q, K, V, O, L, B, H, Nq, Nk, d, q_strides, k_strides, v_strides, o_strides,
                       l_strides, causal, scale, stream, dtype) -> int:
    """The strided C entry point with integer pointers and stride triples; returns the status code."""
    arrs = [_strides3(x) for x in (q_strides, k_strides, v_strides, o_strides, l_strides)]
    ptrs = [ctypes.cast(a, ctypes.c_void_p) if a is not None else None for a in arrs]
    return int(_lib.fa_fwd_strided(Q, K, V, O, L, B, H, Nq, Nk, d, *ptrs, int(causal), float(scale),
                                   stream, int(dtype)))


def raw_fa_bwd(Q, K, V, O, L, dO, dQ, dK, dV, work, B, H, N, d, causal, scale, stream, dtype) -> int:
    """The C backward entry point with integer pointers; returns the status code."""
    return int(_lib.fa_bwd(Q, K, V, O, L, dO, dQ, dK, dV, work, B, H, N, d, int(causal),
                           float(scale), stream, int(dtype)))


def raw_fa_bwd_noalloc(Q, K, V, O, L, dO, dQ, dK, dV, B, H, N, d, causal, scale, stream, dtype) -> int:
    """The allocation-free C backward entry point with integer pointers; returns the status code."""
    return int(_lib.fa_bwd_noalloc(Q, K, V, O, L, dO, dQ, dK, dV, B, H, N, d, int(causal),
                                   float(scale), stream, int(dtype)))


_DTYPES = {torch.bfloat16: FA_DTYPE_BF16, torch.float32: FA_DTYPE_F32}


def _ptr(t):
    return t.data_ptr() if isinstance(t, torch.Tensor) else int(t)


def fa_fwd(Q, K, V, O, L, B, H, N, d, causal, scale, stream=None):
    """Enqueue the forward pass on ``stream`` (default: torch's current stream).

    Q, K, V, O: contiguous [B, H, N, d] device tensors of one dtype (bf16 or fp32);
    L: contiguous [B, H, N] fp32 device tensor. Raises FaError on a bad argument.
    """
    tensors = (Q, K, V, O)
    dt = Q.dtype
    if dt not in _DTYPES:
        raise TypeError(f"unsupported dtype {dt}")
    for t in tensors:
        if t.dtype != dt or tuple(t.shape) != (B, H, N, d) or not t.is_contiguous():
            raise ValueError("Q, K, V, O must be contiguous [B, H, N, d] tensors of one dtype")
        if t.device.type != "cuda" or t.device != Q.device:
            raise ValueError("all tensors must live on the same GPU")
    if L.dtype != torch.float32 or tuple(L.shape) != (B, H, N) or not L.is_contiguous() or L.device != Q.device:
        raise ValueError("L must be a contiguous fp32 [B, H, N] tensor on the same GPU")
    if stream is None:
        stream = torch.cuda.current_stream(Q.device).cuda_stream
    elif isinstance(stream, torch.cuda.Stream):
        stream = stream.cuda_stream
    st = raw_fa_fwd(_ptr(Q), _ptr(K), _ptr(V), _ptr(O), _ptr(L), B, H, N, d, causal, scale,
                    stream, _DTYPES[dt])
    if st != FA_OK:
        raise FaError(st)


def forward(q, k, v, causal: bool = False, scale: float | None = None, stream=None):
    """Allocate O (like q) and fp32 L, run fa_fwd, return (O, L)."""
    if q.dim() != 4:
        raise ValueError("expected [B, H, N, d] tensors")
    B, H, N, d = q.shape
    if scale is None:
        scale = float(torch.tensor(d ** -0.5, dtype=torch.float32).item())
    O = torch.empty_like(q)
    L = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    fa_fwd(q, k, v, O, L, B, H, N, d, causal, scale, stream)
    return O, L


def fa_fwd_strided(Q, K, V, O, L, causal, scale, stream=None):
    """Enqueue the general forward pass: Q, O [B, H, Nq, d] and K, V [B, H, Nk, d]
    device tensors of one dtype with any strides and unit stride along d (expanded,
    stride-0 batch or head dimensions of K and V broadcast them); L an fp32
    [B, H, Nq] tensor. Raises FaError on a bad argument."""
    dt = Q.dtype
    if dt not in _DTYPES:
        raise TypeError(f"unsupported dtype {dt}")
    if Q.dim() != 4 or K.dim() != 4 or V.dim() != 4 or O.dim() != 4 or L.dim() != 3:
        raise ValueError("expected 4-D Q, K, V, O and 3-D L")
    B, H, Nq, d = Q.shape
    Nk = K.shape[2]
    if tuple(K.shape) != (B, H, Nk, d) or tuple(V.shape) != (B, H, Nk, d) or tuple(O.shape) != (B, H, Nq, d):
        raise ValueError("shapes must be Q, O [B, H, Nq, d] and K, V [B, H, Nk, d]")
    if tuple(L.shape) != (B, H, Nq) or L.dtype != torch.float32:
        raise ValueError("L must be an fp32 [B, H, Nq] tensor")
    for t in (Q, K, V, O):
        if t.dtype != dt or t.stride(-1) != 1:
            raise ValueError("Q, K, V, O must share a dtype and have unit stride along d")
    for t in (Q, K, V, O, L):
        if t.device.type != "cuda" or t.device != Q.device:
            raise ValueError("all tensors must live on the same GPU")
    st = raw_fa_fwd_strided(_ptr(Q), _ptr(K), _ptr(V), _ptr(O), _ptr(L), B, H, Nq, Nk, d,
                            Q.stride()[:3], K.stride()[:3], V.stride()[:3], O.stride()[:3], L.stride(),
                            causal, scale, _stream_handle(stream, Q.device), _DTYPES[dt])
    if st != FA_OK:
        raise FaError(st, "fa_fwd_strided")


def fa_fwd_specialized(Q, K, V, O, L, B, H, N, d, causal, scale, stream=None):
    """fa_fwd through the shape-specialized entry point (same checks as ``fa_fwd``)."""
    dt = Q.dtype
    if dt not in _DTYPES:
        raise TypeError(f"unsupported dtype {dt}")
    for t in (Q, K, V, O):
        if t.dtype != dt or tuple(t.shape) != (B, H, N, d) or not t.is_contiguous():
            raise ValueError("Q, K, V, O must be contiguous [B, H, N, d] tensors of one dtype")
        if t.device.type != "cuda" or t.device != Q.device:
            raise ValueError("all tensors must live on the same GPU")
    if L.dtype != torch.float32 or tuple(L.shape) != (B, H, N) or not L.is_contiguous() or L.device != Q.device:
        raise ValueError("L must be a contiguous fp32 [B, H, N] tensor on the same GPU")
    st = raw_fa_fwd_specialized(_ptr(Q), _ptr(K), _ptr(V), _ptr(O), _ptr(L), B, H, N, d, causal, scale,
                                _stream_handle(stream, Q.device), _DTYPES[dt])
    if st != FA_OK:
        raise FaError(st, "fa_fwd_specialized")


def forward_specialized(q, k, v, causal: bool = False, scale: float | None = None, stream=None):
    """Allocate O (like q) and fp32 L, run fa_fwd_specialized, return (O, L)."""
    if q.dim() != 4:
        raise ValueError("expected [B, H, N, d] tensors")
    B, H, N, d = q.shape
    if scale is None:
        scale = float(torch.tensor(d ** -0.5, dtype=torch.float32).item())
    O = torch.empty_like(q)
    L = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    fa_fwd_specialized(q, k, v, O, L, B, H, N, d, causal, scale, stream)
    return O, L


def forward_strided(q, k, v, causal: bool = False, scale: float | None = None, stream=None):
    """Allocate O (with q's memory layout) and a contiguous fp32 L, run fa_fwd_strided,
    return (O, L). q is [B, H, Nq, d]; k and v are [B, H, Nk, d]."""
    if q.dim() != 4:
        raise ValueError("expected [B, H, N, d] tensors")
    B, H, Nq, d = q.shape
    if scale is None:
        scale = float(torch.tensor(d ** -0.5, dtype=torch.float32).item())
    O = torch.empty_like(q)
    L = torch.empty((B, H, Nq), dtype=torch.float32, device=q.device)
    fa_fwd_strided(q, k, v, O, L, causal, scale, stream)
    return O, L


def _stream_handle(stream, device):
    if stream is None:
        return torch.cuda.current_stream(device).cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return stream


def fa_bwd(Q, K, V, O, L, dO, dQ, dK, dV, work, B, H, N, d, causal, scale, stream=None):
    """Enqueue the backward pass on ``stream`` (default: torch's current stream).

    Q, K, V, O, dO, dQ, dK, dV: contiguous [B, H, N, d] device tensors of one dtype;
    L: contiguous fp32 [B, H, N]; work: contiguous fp32 device tensor of at least
    2*B*H*N elements. Raises FaError on a bad argument.
    """
    dt = Q.dtype
    if dt not in _DTYPES:
        raise TypeError(f"unsupported dtype {dt}")
    for t in (Q, K, V, O, dO, dQ, dK, dV):
        if t.dtype != dt or tuple(t.shape) != (B, H, N, d) or not t.is_contiguous():
            raise ValueError("Q, K, V, O, dO, dQ, dK, dV must be contiguous [B, H, N, d] tensors of one dtype")
        if t.device.type != "cuda" or t.device != Q.device:
            raise ValueError("all tensors must live on the same GPU")
    if L.dtype != torch.float32 or tuple(L.shape) != (B, H, N) or not L.is_contiguous() or L.device != Q.device:
        raise ValueError("L must be a contiguous fp32 [B, H, N] tensor on the same GPU")
    if (work.dtype != torch.float32 or not work.is_contiguous() or work.device != Q.device
            or work.numel() < 2 * B * H * N):
        raise ValueError("work must be a contiguous fp32 tensor of 2*B*H*N elements on the same GPU")
    st = raw_fa_bwd(_ptr(Q), _ptr(K), _ptr(V), _ptr(O), _ptr(L), _ptr(dO), _ptr(dQ), _ptr(dK),
                    _ptr(dV), _ptr(work), B, H, N, d, causal, scale,
                    _stream_handle(stream, Q.device), _DTYPES[dt])
    if st != FA_OK:
        raise FaError(st, "fa_bwd")


def fa_bwd_noalloc(Q, K, V, O, L, dO, dQ, dK, dV, B, H, N, d, causal, scale, stream=None):
    """fa_bwd without a workspace argument: the library's static per-GPU workspace is used
    (B*H*N <= 2^20 rows; calls that overlap in time on one GPU race on it). Same tensor
    requirements as fa_bwd. Raises FaError on a bad argument or a too-large problem."""
    dt = Q.dtype
    if dt not in _DTYPES:
        raise TypeError(f"unsupported dtype {dt}")
    for t in (Q, K, V, O, dO, dQ, dK, dV):
        if t.dtype != dt or tuple(t.shape) != (B, H, N, d) or not t.is_contiguous():
            raise ValueError("Q, K, V, O, dO, dQ, dK, dV must be contiguous [B, H, N, d] tensors of one dtype")
        if t.device.type != "cuda" or t.device != Q.device:
            raise ValueError("all tensors must live on the same GPU")
    if L.dtype != torch.float32 or tuple(L.shape) != (B, H, N) or not L.is_contiguous() or L.device != Q.device:
        raise ValueError("L must be a contiguous fp32 [B, H, N] tensor on the same GPU")
    st = raw_fa_bwd_noalloc(_ptr(Q), _ptr(K), _ptr(V), _ptr(O), _ptr(L), _ptr(dO), _ptr(dQ), _ptr(dK),
                            _ptr(dV), B, H, N, d, causal, scale, _stream_handle(stream, Q.device), _DTYPES[dt])
    if st != FA_OK:
        raise FaError(st, "fa_bwd_noalloc")


def backward(q, k, v, o, lse, do, causal: bool = False, scale: float | None = None, stream=None):
    """Allocate dQ, dK, dV (like q) and the fp32 workspace, run fa_bwd, return (dQ, dK, dV).

    ``o`` and ``lse`` are the outputs of ``forward(q, k, v, causal, scale)``.
    """
    if q.dim() != 4:
        raise ValueError("expected [B, H, N, d] tensors")
    B, H, N, d = q.shape
    if scale is None:
        scale = float(torch.tensor(d ** -0.5, dtype=torch.float32).item())
    dq = torch.empty_like(q)
    dk = torch.empty_like(q)
    dv = torch.empty_like(q)
    work = torch.empty(2 * B * H * N, dtype=torch.float32, device=q.device)
    fa_bwd(q, k, v, o, lse, do, dq, dk, dv, work, B, H, N, d, causal, scale, stream)
    return dq, dk, dv


class _Attention(torch.autograd.Function):
    """fa_fwd in the forward pass (O and L kept), fa_bwd in the backward pass."""

    @staticmethod
    def forward(ctx, q, k, v, causal, scale):
        o, lse = forward(q, k, v, causal=causal, scale=scale)
        ctx.save_for_backward(q, k, v, o, lse)
        ctx.causal, ctx.scale = causal, scale
        return o

    @staticmethod
    def backward(ctx, do):
        q, k, v, o, lse = ctx.saved_tensors
        dq, dk, dv = backward(q, k, v, o, lse, do.contiguous(), causal=ctx.causal, scale=ctx.scale)
        return dq, dk, dv, None, None


def attention(q, k, v, causal: bool = False, scale: float | None = None):
    """O = softmax(scale q k^T) v (optionally causal) for contiguous [B, H, N, d] device
    tensors, differentiable: the gradient runs fa_bwd on the saved O and L. The forward
    pass takes d in {16, 32, 64, 128}; the backward pass d in {64, 128} (fp32 also 32)
    and raises FaError otherwise. ``scale`` defaults to 1/sqrt(d) rounded to fp32."""
    if q.dim() != 4:
        raise ValueError("expected [B, H, N, d] tensors")
    if scale is None:
        scale = float(torch.tensor(q.shape[-1] ** -0.5, dtype=torch.float32).item())
    return _Attention.apply(q, k, v, bool(causal), float(scale))
