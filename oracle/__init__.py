"""Oracle for the attention forward pass: plain, slow, obviously correct, fp64, CPU.

TEST INFRASTRUCTURE ONLY. Only the test suite, the package smoke check and the
benchmark's CPU-baseline leg may import this package. The product path (the HIP
library and its Python binding) never imports, links or calls anything here,
and nothing here imports the product path.

Four parts:

* ``attention`` -- standard attention by its definition (``attention.c``):
  "Writing a FlashAttention kernel in Metal", section "Standard attention", with
  the causal rule of its section "Blockwise attention and causal masking", and L
  as defined in "FlashAttention-2 from PyTorch to Triton", section "What We Are
  Building".
* ``attention_cross`` -- the same definition between Nq query rows and Nk key/value
  rows, with the causal mask aligned at the top-left corner as in the kernel of
  "FlashAttention-2 from PyTorch to Triton", section "The Triton Kernel"
  (``attention_cross.c``).
* ``attention_bwd`` -- the gradients of that function with respect to Q, K and V
  for a given output gradient, by the chain rule through its definition
  (``attention_bwd.c``).
* ``blockwise`` -- fp64 models of the pages' online-softmax recurrences (the
  method itself), used by the tests to tie the recurrence to the definition.

Pins: every function here is checked, in ``tests/test_oracle.py``,
``tests/test_oracle_bwd.py``, ``tests/test_oracle_cross.py`` and ``tests/test_blockwise.py``, against closed
forms, invariants, brute force on tiny inputs (central differences of the
forward oracle for the gradients), torch's own scaled-dot-product attention in
fp64 (and its autograd) and the worked two-block example of the first page's
"Online softmax" section.
"""

from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "attention.c")
_SRC_BWD = os.path.join(_HERE, "attention_bwd.c")
_SRC_CROSS = os.path.join(_HERE, "attention_cross.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None


def build(verbose: bool = False) -> str:
    """Compile the oracle's C sources into ``liboracle.so`` with gcc (no fast-math)."""
    cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11",
           "-o", _LIB_PATH, _SRC, _SRC_BWD, _SRC_CROSS, "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    return _LIB_PATH


def load_library(path: str):
    """Open a compiled copy of the oracle sources and declare its signatures (a copy
    built from one source file has only that file's entry points)."""
    lib = ctypes.CDLL(path)
    lib.oracle_attention_f64.restype = ctypes.c_int
    lib.oracle_attention_f64.argtypes = [
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
        ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
        ctypes.c_int, ctypes.c_double, ctypes.c_void_p, ctypes.c_int64,
    ]
    lib.oracle_num_threads.restype = ctypes.c_int
    lib.oracle_num_threads.argtypes = []
    if hasattr(lib, "oracle_attention_cross_f64"):
        lib.oracle_attention_cross_f64.restype = ctypes.c_int
        lib.oracle_attention_cross_f64.argtypes = [ctypes.c_void_p] * 5 + [ctypes.c_int64] * 5 + [
            ctypes.c_int, ctypes.c_double,
        ]
    if hasattr(lib, "oracle_attention_bwd_f64"):
        lib.oracle_attention_bwd_f64.restype = ctypes.c_int
        lib.oracle_attention_bwd_f64.argtypes = [ctypes.c_void_p] * 7 + [
            ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
            ctypes.c_int, ctypes.c_double,
        ]
    return lib


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < max(
                os.path.getmtime(_SRC), os.path.getmtime(_SRC_BWD), os.path.getmtime(_SRC_CROSS)):
            build()
        _lib = load_library(_LIB_PATH)
    return _lib


def num_threads() -> int:
    """OpenMP threads the oracle runs on (all host cores unless OMP_NUM_THREADS says otherwise)."""
    return int(_load().oracle_num_threads())


def attention(Q, K, V, causal: bool, scale: float, rows=None, lib=None):
    """Standard attention in fp64.

    Q, K, V: array-likes of shape [B, H, N, d] (or [N, d], treated as B=H=1),
    up-cast losslessly to fp64. ``scale`` multiplies the scores as given.
    ``rows``: None for every query row, else a 1-D list of query indices.

    Returns (O, L) as fp64 numpy arrays: O [B, H, R, d], L [B, H, R] with R = N
    or len(rows) (squeezed back to [R, d] / [R] for 2-D input).
    ``lib`` selects another compiled copy (from ``load_library``); default: this one.
    """
    lib = lib or _load()
    q = np.ascontiguousarray(np.asarray(Q, dtype=np.float64))
    k = np.ascontiguousarray(np.asarray(K, dtype=np.float64))
    v = np.ascontiguousarray(np.asarray(V, dtype=np.float64))
    squeeze = q.ndim == 2
    if squeeze:
        q, k, v = q[None, None], k[None, None], v[None, None]
    if q.ndim != 4 or q.shape != k.shape or q.shape != v.shape:
        raise ValueError(f"expected equal [B,H,N,d] shapes, got {q.shape} {k.shape} {v.shape}")
    B, H, N, d = q.shape
    if rows is None:
        idx = None
        R = N
        rows_ptr = None
    else:
        idx = np.ascontiguousarray(np.asarray(rows, dtype=np.int64).reshape(-1))
        R = int(idx.size)
        rows_ptr = idx.ctypes.data
    O = np.empty((B, H, R, d), dtype=np.float64)
    L = np.empty((B, H, R), dtype=np.float64)
    st = lib.oracle_attention_f64(q.ctypes.data, k.ctypes.data, v.ctypes.data,
                                  O.ctypes.data, L.ctypes.data, B, H, N, d,
                                  1 if causal else 0, float(scale), rows_ptr, R)
    if st != 0:
        raise RuntimeError(f"oracle_attention_f64 failed with status {st}")
    if squeeze:
        return O[0, 0], L[0, 0]
    return O, L


def attention_cross(Q, K, V, causal: bool, scale: float, lib=None):
    """Attention between Nq query rows and Nk key/value rows in fp64.

    Q: array-like [B, H, Nq, d]; K, V: [B, H, Nk, d] (or [Nq, d] / [Nk, d], treated
    as B = H = 1), up-cast losslessly to fp64. When ``causal``, query i keeps keys
    j <= i (mask aligned at the top-left corner).

    Returns (O, L) as fp64 numpy arrays: O [B, H, Nq, d], L [B, H, Nq] (squeezed back
    for 2-D input). ``lib`` selects another compiled copy; default: this one.
    """
    lib = lib or _load()
    q = np.ascontiguousarray(np.asarray(Q, dtype=np.float64))
    k = np.ascontiguousarray(np.asarray(K, dtype=np.float64))
    v = np.ascontiguousarray(np.asarray(V, dtype=np.float64))
    squeeze = q.ndim == 2
    if squeeze:
        q, k, v = q[None, None], k[None, None], v[None, None]
    if (q.ndim != 4 or k.shape != v.shape or q.shape[:2] != k.shape[:2]
            or q.shape[3] != k.shape[3]):
        raise ValueError(f"expected [B,H,Nq,d] and two [B,H,Nk,d], got {q.shape} {k.shape} {v.shape}")
    B, H, Nq, d = q.shape
    Nk = k.shape[2]
    O = np.empty((B, H, Nq, d), dtype=np.float64)
    L = np.empty((B, H, Nq), dtype=np.float64)
    st = lib.oracle_attention_cross_f64(q.ctypes.data, k.ctypes.data, v.ctypes.data,
                                        O.ctypes.data, L.ctypes.data, B, H, Nq, Nk, d,
                                        1 if causal else 0, float(scale))
    if st != 0:
        raise RuntimeError(f"oracle_attention_cross_f64 failed with status {st}")
    if squeeze:
        return O[0, 0], L[0, 0]
    return O, L


def attention_bwd(Q, K, V, dO, causal: bool, scale: float, lib=None):
    """Gradients of standard attention in fp64.

    Q, K, V, dO: array-likes of shape [B, H, N, d] (or [N, d], treated as B=H=1),
    up-cast losslessly to fp64; dO is the gradient of the loss with respect to the
    output O = softmax(scale Q K^T) V (causal as in ``attention``).

    Returns (dQ, dK, dV) as fp64 numpy arrays of the input shape.
    ``lib`` selects another compiled copy (from ``load_library``); default: this one.
    """
    lib = lib or _load()
    arrs = [np.ascontiguousarray(np.asarray(x, dtype=np.float64)) for x in (Q, K, V, dO)]
    squeeze = arrs[0].ndim == 2
    if squeeze:
        arrs = [a[None, None] for a in arrs]
    q, k, v, go = arrs
    if q.ndim != 4 or any(a.shape != q.shape for a in arrs):
        raise ValueError(f"expected equal [B,H,N,d] shapes, got {[a.shape for a in arrs]}")
    B, H, N, d = q.shape
    dQ = np.empty_like(q)
    dK = np.empty_like(q)
    dV = np.empty_like(q)
    st = lib.oracle_attention_bwd_f64(q.ctypes.data, k.ctypes.data, v.ctypes.data, go.ctypes.data,
                                      dQ.ctypes.data, dK.ctypes.data, dV.ctypes.data,
                                      B, H, N, d, 1 if causal else 0, float(scale))
    if st != 0:
        raise RuntimeError(f"oracle_attention_bwd_f64 failed with status {st}")
    if squeeze:
        return dQ[0, 0], dK[0, 0], dV[0, 0]
    return dQ, dK, dV
