"""MI355X (gfx950) MoE-layer hot path: router, dispatch, grouped SwiGLU FFN, combine, backward.

The compute lives in the HIP library libmoe_amd.so (C ABI in include/moe.h);
this package is its ctypes binding plus a buffer-owning layer helper.  There
is no CPU or PyTorch fallback: loading fails if the library is not built.
"""
from . import _lib  # noqa: F401
from ._lib import (  # noqa: F401
    MOE_BF16, MOE_F32, MOE_F_ACCUM_GRAD, MOE_F_RENORM, Dims, MoeError, dims, load,
)
from .layer import MoDMoELayer, MoELayer  # noqa: F401
