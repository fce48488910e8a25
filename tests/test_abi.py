"""The C ABI: the library loads without a GPU, exports what include/fa.h declares,
and rejects bad arguments synchronously, before any device work (CPU only)."""

import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa.h")

fa = pytest.importorskip("tiled_online_softmax_amd", reason="libfa.so not built")

A = 1 << 20  # fake, 16-byte aligned "device" addresses: never dereferenced on these paths


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fa_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_entry_points():
    assert declared_functions() == ["fa_bwd", "fa_bwd_noalloc", "fa_fwd", "fa_fwd_specialized", "fa_fwd_strided",
                                    "fa_jit_code_object", "fa_status_string", "fa_version"]


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(fa.LIB_PATH)
    for name in declared_functions():
        assert hasattr(lib, name), f"{name} not exported"


def test_status_strings_and_version():
    assert fa.fa_status_string(0) == "ok"
    for s in range(1, 7):
        assert fa.fa_status_string(s) not in ("ok", "unknown status")
    assert fa.fa_status_string(99) == "unknown status"
    assert fa.fa_version() >= 100


def call(Q=A, K=2 * A, V=3 * A, O=4 * A, L=5 * A, B=1, H=1, N=64, d=64, causal=0, scale=0.125,
         dtype=fa.FA_DTYPE_BF16):
    return fa.raw_fa_fwd(Q, K, V, O, L, B, H, N, d, causal, scale, None, dtype)


@pytest.mark.parametrize("kw", [dict(Q=0), dict(K=0), dict(V=0), dict(O=0), dict(L=0)])
def test_null_pointer(kw):
    assert call(**kw) == fa.FA_ERR_INVALID_ARGUMENT


@pytest.mark.parametrize("kw", [dict(B=0), dict(H=0), dict(N=0), dict(N=-5), dict(B=-1)])
def test_bad_sizes(kw):
    assert call(**kw) == fa.FA_ERR_INVALID_ARGUMENT


@pytest.mark.parametrize("scale", [0.0, -1.0, float("inf"), float("nan"), 3.0e38])
def test_bad_scale(scale):
    """Non-positive or non-finite scales, and finite ones whose scale * log2(e) overflows fp32."""
    assert call(scale=scale) == fa.FA_ERR_INVALID_ARGUMENT


def test_bad_dtype():
    assert call(dtype=7) == fa.FA_ERR_INVALID_ARGUMENT


@pytest.mark.parametrize("d", [8, 48, 63, 96, 256])
def test_unsupported_head_dim(d):
    assert call(d=d) == fa.FA_ERR_UNSUPPORTED


def test_too_long_sequence():
    assert call(N=(1 << 24) + 1) == fa.FA_ERR_UNSUPPORTED


@pytest.mark.parametrize("kw", [dict(B=1 << 32, H=1 << 32), dict(B=1 << 40), dict(H=(1 << 31) + 1)])
def test_head_count_overflow(kw):
    # B * H = 2^64 wraps to 0 in 64 bits: B and H are bounded before they are multiplied.
    assert call(**kw) == fa.FA_ERR_UNSUPPORTED
    assert call_spec(**kw) == fa.FA_ERR_UNSUPPORTED


def test_overlapping_output():
    # O overlaps K
    assert call(O=2 * A + 64) == fa.FA_ERR_INVALID_ARGUMENT
    # L overlaps O
    assert call(L=4 * A + 16) == fa.FA_ERR_INVALID_ARGUMENT


@pytest.mark.parametrize("kw", [dict(Q=A + 8), dict(V=3 * A + 2), dict(L=5 * A + 4)])
def test_misaligned(kw):
    assert call(**kw) == fa.FA_ERR_MISALIGNED


def test_validation_order_null_before_unsupported():
    assert call(Q=0, d=96) == fa.FA_ERR_INVALID_ARGUMENT


# fa_bwd: ten 1 MiB-spaced fake buffers (tensors of 1*1*64*64 bf16 are 8 KiB).
BWD = dict(Q=A, K=2 * A, V=3 * A, O=4 * A, L=5 * A, dO=6 * A, dQ=7 * A, dK=8 * A, dV=9 * A, work=10 * A)


def call_bwd(B=1, H=1, N=64, d=64, causal=0, scale=0.125, dtype=fa.FA_DTYPE_BF16, **kw):
    p = dict(BWD, **kw)
    return fa.raw_fa_bwd(p["Q"], p["K"], p["V"], p["O"], p["L"], p["dO"], p["dQ"], p["dK"], p["dV"],
                         p["work"], B, H, N, d, causal, scale, None, dtype)


@pytest.mark.parametrize("name", sorted(BWD))
def test_bwd_null_pointer(name):
    assert call_bwd(**{name: 0}) == fa.FA_ERR_INVALID_ARGUMENT


@pytest.mark.parametrize("kw", [dict(B=0), dict(H=0), dict(N=0), dict(scale=0.0), dict(scale=float("nan")),
                                dict(scale=3.0e38), dict(dtype=7)])
def test_bwd_bad_arguments(kw):
    assert call_bwd(**kw) == fa.FA_ERR_INVALID_ARGUMENT


@pytest.mark.parametrize("kw", [dict(d=32), dict(d=96), dict(N=(1 << 24) + 1),
                                dict(d=96, dtype=fa.FA_DTYPE_F32), dict(d=16, dtype=fa.FA_DTYPE_F32)])
def test_bwd_unsupported(kw):
    assert call_bwd(**kw) == fa.FA_ERR_UNSUPPORTED


@pytest.mark.parametrize("kw", [dict(B=1 << 32, H=1 << 32), dict(H=1 << 40)])
def test_bwd_head_count_overflow(kw):
    assert call_bwd(**kw) == fa.FA_ERR_UNSUPPORTED


def test_bwd_overlap_uses_element_size():
    # 64 x 64 fp32 tensors span 16 KiB: dQ 12 KiB after Q overlaps it (as bf16 it would not).
    assert call_bwd(dtype=fa.FA_DTYPE_F32, dQ=A + 12 * 1024) == fa.FA_ERR_INVALID_ARGUMENT


@pytest.mark.parametrize("kw", [dict(dQ=2 * A + 64), dict(dK=6 * A), dict(dV=7 * A + 4096),
                                dict(work=A + 32), dict(work=8 * A + 16), dict(dQ=5 * A)])
def test_bwd_overlapping_outputs(kw):
    assert call_bwd(**kw) == fa.FA_ERR_INVALID_ARGUMENT


@pytest.mark.parametrize("name", ["Q", "dO", "dK", "work", "L"])
def test_bwd_misaligned(name):
    assert call_bwd(**{name: BWD[name] + 4}) == fa.FA_ERR_MISALIGNED


# fa_bwd_noalloc: the same checks as fa_bwd (no workspace argument), and a size limit of
# 2^20 rows (B*H*N) checked first, before the library's workspace is looked up.
def call_bwd_noalloc(B=1, H=1, N=64, d=64, causal=0, scale=0.125, dtype=fa.FA_DTYPE_BF16, **kw):
    p = dict(BWD, **kw)
    return fa.raw_fa_bwd_noalloc(p["Q"], p["K"], p["V"], p["O"], p["L"], p["dO"], p["dQ"], p["dK"], p["dV"],
                                 B, H, N, d, causal, scale, None, dtype)


@pytest.mark.parametrize("kw", [dict(N=(1 << 20) + 1), dict(B=2, H=4, N=(1 << 17) + 1), dict(B=1 << 21),
                                dict(B=1 << 40, H=1 << 40), dict(N=1 << 24),
                                dict(B=1 << 21, H=1 << 21, N=1 << 21)])  # 2 B H N = 2^64 wraps to 0
def test_bwd_noalloc_size_limit(kw):
    assert call_bwd_noalloc(**kw) == fa.FA_ERR_SCRATCH_LIMIT


@pytest.mark.parametrize("kw", [dict(B=0), dict(N=0), dict(H=-1), dict(Q=0), dict(dV=0), dict(scale=0.0),
                                dict(dtype=7), dict(dK=6 * A), dict(dQ=2 * A + 64)])
def test_bwd_noalloc_bad_arguments(kw):
    assert call_bwd_noalloc(**kw) == fa.FA_ERR_INVALID_ARGUMENT


@pytest.mark.parametrize("kw,status", [(dict(d=96), fa.FA_ERR_UNSUPPORTED), (dict(d=32), fa.FA_ERR_UNSUPPORTED),
                                       (dict(dO=6 * A + 4), fa.FA_ERR_MISALIGNED)])
def test_bwd_noalloc_validation(kw, status):
    assert call_bwd_noalloc(**kw) == status


# fa_fwd_strided: every call below fails validation, so nothing is ever launched on
# the fake addresses. Default: B = 1, H = 2, Nq = 64, Nk = 96, d = 64, contiguous.
def _contig(H, N, d):
    return (H * N * d, N * d, d)


STR = dict(q=_contig(2, 64, 64), k=_contig(2, 96, 64), v=_contig(2, 96, 64), o=_contig(2, 64, 64),
           l=(2 * 64, 64, 1))


def call_strided(B=1, H=2, Nq=64, Nk=96, d=64, causal=0, scale=0.125, dtype=fa.FA_DTYPE_BF16,
                 Q=A, K=2 * A, V=3 * A, O=4 * A, L=5 * A, **st):
    s = dict(STR, **st)
    return fa.raw_fa_fwd_strided(Q, K, V, O, L, B, H, Nq, Nk, d, s["q"], s["k"], s["v"], s["o"], s["l"],
                                 causal, scale, None, dtype)


@pytest.mark.parametrize("kw", [dict(Q=0), dict(K=0), dict(V=0), dict(O=0), dict(L=0), dict(q=None),
                                dict(k=None), dict(v=None), dict(o=None), dict(l=None)])
def test_strided_null(kw):
    assert call_strided(**kw) == fa.FA_ERR_INVALID_ARGUMENT


@pytest.mark.parametrize("kw", [dict(Nq=0), dict(Nk=0), dict(B=0), dict(H=-1), dict(scale=0.0), dict(scale=3.0e38),
                                dict(dtype=5)])
def test_strided_bad_sizes(kw):
    assert call_strided(**kw) == fa.FA_ERR_INVALID_ARGUMENT


@pytest.mark.parametrize("kw", [
    dict(q=(8192, 4096, -64)),          # negative stride
    dict(k=(12288, 6144, 32)),          # K rows overlap (row stride < d)
    dict(o=(8192, 32, 128)),            # O heads 32 elements apart: rows of d = 64 overlap
    dict(o=(0, 4096, 64), B=2),         # two batches of O at one address
    dict(l=(128, 0, 1)),                # both heads of L at one address
    dict(O=2 * A + 64),                 # O overlaps K
    dict(B=1 << 30, H=1, q=(1 << 40, 4096, 64), k=(1 << 40, 6144, 64), v=(1 << 40, 6144, 64),
         o=(1 << 40, 4096, 64), l=(1 << 20, 64, 1)),  # spans past 2^62 bytes
    dict(L=4 * A + 64),                 # L overlaps O
])
def test_strided_invalid_layouts(kw):
    assert call_strided(**kw) == fa.FA_ERR_INVALID_ARGUMENT


_D256 = dict(d=256, q=_contig(2, 64, 256), k=_contig(2, 96, 256), v=_contig(2, 96, 256), o=_contig(2, 64, 256))


_NQ = (1 << 24) + 1
_BIG_NQ = dict(Nq=_NQ, q=_contig(2, _NQ, 64), o=_contig(2, _NQ, 64), l=(2 * _NQ, _NQ, 1))


@pytest.mark.parametrize("kw", [dict(d=48), _D256, _BIG_NQ, dict(Nk=(1 << 24) + 1),
                                dict(k=(1 << 26, 1 << 25, 1 << 24))])
def test_strided_unsupported(kw):
    assert call_strided(**kw) == fa.FA_ERR_UNSUPPORTED


@pytest.mark.parametrize("kw", [dict(Q=A + 8), dict(V=3 * A + 4), dict(L=5 * A + 2),
                                dict(q=(8192, 4096, 68)), dict(o=(8192 + 4, 4096, 64), B=2),
                                dict(k=(12288, 6144, 64), v=(12288, 6148, 64))])
def test_strided_misaligned(kw):
    assert call_strided(**kw) == fa.FA_ERR_MISALIGNED


def test_strided_fp32_alignment_unit():
    # fp32 rows are 16-byte aligned at multiples of 4 elements: 68 passes the alignment
    # check, so it is made to fail on the overlap check instead (O overlaps Q).
    assert call_strided(dtype=fa.FA_DTYPE_F32, q=(8192 * 2, 4096 * 2, 68), O=A + 64) == fa.FA_ERR_INVALID_ARGUMENT
    assert call_strided(dtype=fa.FA_DTYPE_F32, q=(8192, 4096, 66)) == fa.FA_ERR_MISALIGNED


# fa_fwd_specialized validates exactly as fa_fwd, before compiling or launching anything.
def call_spec(**kw):
    a = dict(Q=A, K=2 * A, V=3 * A, O=4 * A, L=5 * A, B=1, H=1, N=64, d=64, causal=0, scale=0.125,
             dtype=fa.FA_DTYPE_BF16)
    a.update(kw)
    return fa.raw_fa_fwd_specialized(a["Q"], a["K"], a["V"], a["O"], a["L"], a["B"], a["H"], a["N"], a["d"],
                                     a["causal"], a["scale"], None, a["dtype"])


@pytest.mark.parametrize("kw,status", [(dict(Q=0), fa.FA_ERR_INVALID_ARGUMENT), (dict(N=0), fa.FA_ERR_INVALID_ARGUMENT),
                                       (dict(scale=-1.0), fa.FA_ERR_INVALID_ARGUMENT), (dict(dtype=3), fa.FA_ERR_INVALID_ARGUMENT),
                                       (dict(d=96), fa.FA_ERR_UNSUPPORTED), (dict(O=2 * A + 64), fa.FA_ERR_INVALID_ARGUMENT),
                                       (dict(K=2 * A + 8), fa.FA_ERR_MISALIGNED)])
def test_specialized_validation(kw, status):
    assert call_spec(**kw) == status


def test_jit_code_object_arguments():
    import ctypes

    lib = ctypes.CDLL(fa.LIB_PATH)
    lib.fa_jit_code_object.restype = ctypes.c_int
    lib.fa_jit_code_object.argtypes = [ctypes.c_int, ctypes.c_int64, ctypes.c_int, ctypes.c_int64, ctypes.c_int64,
                                       ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p]
    assert lib.fa_jit_code_object(fa.FA_DTYPE_BF16, 64, 0, 1, 1, 64, None, None) == fa.FA_ERR_INVALID_ARGUMENT
    size = ctypes.c_size_t(0)
    assert lib.fa_jit_code_object(fa.FA_DTYPE_BF16, 96, 0, 1, 1, 64, None, ctypes.byref(size)) == fa.FA_ERR_UNSUPPORTED
    assert lib.fa_jit_code_object(7, 64, 0, 1, 1, 64, None, ctypes.byref(size)) == fa.FA_ERR_INVALID_ARGUMENT
    assert lib.fa_jit_code_object(fa.FA_DTYPE_BF16, 64, 0, 0, 1, 64, None, ctypes.byref(size)) == fa.FA_ERR_INVALID_ARGUMENT
    # B * H = 2^64 would wrap to 0: rejected before anything is compiled.
    assert lib.fa_jit_code_object(fa.FA_DTYPE_BF16, 64, 0, 1 << 32, 1 << 32, 64, None,
                                  ctypes.byref(size)) == fa.FA_ERR_UNSUPPORTED


def test_attention_checks_rank():
    """The differentiable wrapper rejects tensors that are not [B, H, N, d] before any GPU call."""
    import torch

    x = torch.zeros(4, 8)
    with pytest.raises(ValueError):
        fa.attention(x, x, x)
