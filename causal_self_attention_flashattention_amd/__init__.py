"""MI355X-native tiled causal self-attention (FlashAttention-2 style), forward and backward.

The computation lives in ``libattn.so`` (HIP kernels for gfx950 behind a C ABI, see
``include/attn.h``); this package is a thin ctypes binding plus the seeded input generator.
"""

from .binding import (  # noqa: F401
    AttnError,
    bwd,
    bwd_workspace_bytes,
    bwd_launches,
    bwd_noalloc,
    bwd_dkdv,
    bwd_dq,
    fwd,
    fwd_workspace_bytes,
    load_library,
    rowdot,
    status_string,
    supported,
)
from .function import FlashAttention, flash_attention  # noqa: F401

__all__ = ["FlashAttention", "flash_attention", "fwd", "fwd_workspace_bytes", "bwd", "bwd_workspace_bytes", "bwd_launches", "bwd_noalloc", "rowdot", "bwd_dkdv", "bwd_dq", "supported", "load_library", "status_string", "AttnError"]
