"""Tiled online-softmax attention forward pass for MI355X (gfx950).

``fa_fwd`` mirrors the C entry point of ``libfa.so``; ``forward`` allocates the
outputs and calls it. Importing fails loudly when the HIP library is not built.
"""

from ._binding import (  # noqa: F401
    FA_DTYPE_BF16,
    FA_DTYPE_F32,
    FA_ERR_INVALID_ARGUMENT,
    FA_ERR_LAUNCH,
    FA_ERR_MISALIGNED,
    FA_ERR_UNSUPPORTED,
    FA_OK,
    LIB_PATH,
    FaError,
    fa_fwd,
    fa_status_string,
    fa_version,
    forward,
    raw_fa_fwd,
)
