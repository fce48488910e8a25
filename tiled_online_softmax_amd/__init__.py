"""Tiled online-softmax attention forward and backward passes for MI355X (gfx950).

``fa_fwd``, ``fa_fwd_strided``, ``fa_fwd_specialized``, ``fa_bwd`` and ``fa_bwd_noalloc``
mirror the C entry points of ``libfa.so``; ``forward``, ``forward_strided``, ``forward_specialized``
and ``backward`` allocate the outputs (and the backward workspace) and call them;
``attention`` is the differentiable form (fa_fwd forward, fa_bwd backward).
Importing fails loudly when the HIP library is not built.
"""

from ._binding import (  # noqa: F401
    FA_DTYPE_BF16,
    FA_DTYPE_F32,
    FA_ERR_INVALID_ARGUMENT,
    FA_ERR_JIT,
    FA_ERR_LAUNCH,
    FA_ERR_MISALIGNED,
    FA_ERR_SCRATCH_LIMIT,
    FA_ERR_UNSUPPORTED,
    FA_OK,
    LIB_PATH,
    FaError,
    attention,
    backward,
    fa_bwd,
    fa_bwd_noalloc,
    fa_fwd,
    fa_fwd_specialized,
    fa_fwd_strided,
    fa_status_string,
    fa_version,
    forward,
    forward_specialized,
    forward_strided,
    jit_code_object,
    raw_fa_bwd,
    raw_fa_bwd_noalloc,
    raw_fa_fwd,
    raw_fa_fwd_specialized,
    raw_fa_fwd_strided,
)
