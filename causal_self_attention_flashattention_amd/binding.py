"""Thin ctypes binding over libattn's C ABI (include/attn.h).

Argument marshalling only: torch supplies device memory and the current HIP stream; every step
of the computation runs in the library's HIP kernels.  There is no fallback: if the library is
not built, or no GPU is present, these functions raise.
"""

from __future__ import annotations

import ctypes
import functools
import math
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libattn.so")

DTYPE_F32, DTYPE_BF16 = 0, 1
_DTYPES = {torch.float32: DTYPE_F32, torch.bfloat16: DTYPE_BF16}

# Names and C signatures of every exported entry point (kept in step with include/attn.h).
_vp, _i, _f, _sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
SIGNATURES = {
    "attn_fwd": (_i, [_vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _f, _i, _vp, _vp]),
    "attn_bwd": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _f, _i, _vp, _vp]),
    "attn_bwd_rowdot": (_i, [_vp, _vp, _vp, _i, _i, _i, _i, _i, _vp]),
    "attn_bwd_dkdv": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _f, _i, _vp, _vp]),
    "attn_bwd_dq": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _f, _i, _vp, _vp]),
    "attn_fwd_blocksparse": (_i, [_vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _f, _i, _vp, _vp, _vp]),
    "attn_bwd_blocksparse": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _f, _i, _vp, _vp,
                                  _vp]),
    "attn_fwd_workspace_bytes": (_sz, [_i, _i, _i, _i, _i]),
    "attn_fwd_ex": (_i, [_vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _f, _i, _vp, _vp, _vp, _sz, _vp]),
    "attn_bwd_workspace_bytes": (_sz, [_i, _i, _i, _i, _i]),
    "attn_bwd_ex": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _f, _i, _vp, _vp, _vp,
                         _sz, _vp]),
    "attn_bwd_noalloc": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _f, _i, _vp, _vp,
                              _vp]),
    "attn_status_string": (ctypes.c_char_p, [_i]),
    "attn_supported": (_i, [_i, _i]),
    "attn_bwd_launches": (_i, [_i, _i, _i, _i, _i]),
    "attn_version": (_i, []),
}

_lib = None


class AttnError(RuntimeError):
    """A non-zero status returned by the C ABI."""

    def __init__(self, fn: str, status: int, text: str):
        super().__init__(f"{fn} failed with status {status}: {text}")
        self.status = status


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libattn.so (once) and declare its signatures. Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(
            f"libattn.so not found at {path}: build it with "
            "`python -m causal_self_attention_flashattention_amd.build` (or __graft_entry__.build())")
    lib = ctypes.CDLL(path)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def status_string(status: int) -> str:
    return load_library().attn_status_string(int(status)).decode()


def _check(fn: str, status: int) -> None:
    if status != 0:
        raise AttnError(fn, status, status_string(status))


def _ptr(t) -> int | None:
    return None if t is None else t.data_ptr()


def _stream() -> int:
    return torch.cuda.current_stream().cuda_stream


def _check_qkv(*ts):
    ref = ts[0]
    if ref.dim() != 4:
        raise ValueError("expected [B, H, N, d] tensors")
    if ref.dtype not in _DTYPES:
        raise TypeError(f"dtype {ref.dtype} not supported (float32, bfloat16)")
    for t in ts:
        if not t.is_cuda:
            raise ValueError("tensors must live on the GPU")
        if t.shape != ref.shape or t.dtype != ref.dtype:
            raise ValueError("Q, K, V, O, dO must share shape and dtype")
        if not t.is_contiguous():
            raise ValueError("tensors must be contiguous [B, H, N, d]")
    return ref.shape


def kv_len_tensor(kv_len, B, device):
    """kv_len (None, an int, a sequence of B ints or an int tensor) as a device int32[B] tensor or None."""
    if kv_len is None:
        return None
    if isinstance(kv_len, torch.Tensor):
        t = kv_len
    else:
        t = torch.tensor([int(kv_len)] * B if isinstance(kv_len, int) else list(kv_len), dtype=torch.int32)
    t = t.to(device=device, dtype=torch.int32).contiguous()
    if t.numel() != B:
        raise ValueError("kv_len must hold one length per batch row")
    return t


def mask_blocks(N: int) -> int:
    """Side of a block-sparse mask for sequence length N (one entry per 64 x 64 block)."""
    return (N + 63) // 64


def block_mask_tensor(block_mask, N, device):
    """block_mask (array-like or tensor, [ceil(N/64)]^2, non-zero = attend) as a device uint8 tensor."""
    if block_mask is None:
        return None
    tb = mask_blocks(N)
    m = block_mask if isinstance(block_mask, torch.Tensor) else torch.as_tensor(block_mask)
    if tuple(m.shape) != (tb, tb):
        raise ValueError(f"block_mask must be [{tb}, {tb}] for N={N} (one entry per 64 x 64 block)")
    return (m != 0).to(device=device, dtype=torch.uint8).contiguous()


@functools.lru_cache(maxsize=1024)
def fwd_workspace_bytes(B: int, H: int, N: int, d: int, dtype) -> int:
    """Workspace attn_fwd_ex can use for this shape (0 when the plain single launch is best)."""
    return int(load_library().attn_fwd_workspace_bytes(B, H, N, d, _DTYPES[dtype]))


def fwd(q, k, v, causal: bool = True, scale: float | None = None, kv_len=None, out=None, lse=None,
        block_mask=None, workspace="auto"):
    """Attention forward. Returns ``(O, L)``: O like q, L float32 [B, H, N] (natural log).

    ``block_mask`` (optional, [ceil(N/64)]^2, non-zero = attend) restricts the scores to whole
    64 x 64 blocks (block-sparse attention); masked blocks are skipped by the kernels.
    ``workspace``: "auto" allocates the scratch the library asks for (grids too small to fill the
    chip then split each query tile's keys over several workgroups), None runs the plain single
    launch, or pass a float32 CUDA tensor of at least ``fwd_workspace_bytes`` bytes."""
    B, H, N, d = _check_qkv(q, k, v)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    o = torch.empty_like(q) if out is None else out
    L = torch.empty((B, H, N), dtype=torch.float32, device=q.device) if lse is None else lse
    kv = kv_len_tensor(kv_len, B, q.device)
    bm = block_mask_tensor(block_mask, N, q.device)
    lib = load_library()
    if isinstance(workspace, str):
        need = fwd_workspace_bytes(B, H, N, d, q.dtype)
        workspace = torch.empty((need + 3) // 4, dtype=torch.float32, device=q.device) if need else None
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib.attn_fwd_ex(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(L), B, H, N, d, int(bool(causal)), scale,
                         _DTYPES[q.dtype], _ptr(kv), _ptr(bm), _ptr(workspace), ws_bytes, _stream())
    _check("attn_fwd_ex", st)
    return o, L


@functools.lru_cache(maxsize=1024)
def bwd_workspace_bytes(B: int, H: int, N: int, d: int, dtype) -> int:
    """Workspace attn_bwd_ex can use for this shape (0 when the plain launches are best)."""
    return int(load_library().attn_bwd_workspace_bytes(B, H, N, d, _DTYPES[dtype]))


def bwd(q, k, v, o, do, lse, causal: bool = True, scale: float | None = None, kv_len=None, outs=None,
        block_mask=None, workspace="auto"):
    """Attention backward. Returns ``(dQ, dK, dV, D)``; D = rowsum(O o dO) float32 [B, H, N].
    ``block_mask`` as for :func:`fwd` (the same mask the forward used); ``workspace`` as for
    :func:`fwd` (``bwd_workspace_bytes``)."""
    B, H, N, d = _check_qkv(q, k, v, o, do)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    if outs is None:
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
        D = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    else:
        dq, dk, dv, D = outs
    kv = kv_len_tensor(kv_len, B, q.device)
    bm = block_mask_tensor(block_mask, N, q.device)
    if isinstance(workspace, str):
        need = bwd_workspace_bytes(B, H, N, d, q.dtype)
        workspace = torch.empty((need + 3) // 4, dtype=torch.float32, device=q.device) if need else None
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = load_library().attn_bwd_ex(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(do), _ptr(lse), _ptr(dq), _ptr(dk),
                                    _ptr(dv), _ptr(D), B, H, N, d, int(bool(causal)), scale, _DTYPES[q.dtype],
                                    _ptr(kv), _ptr(bm), _ptr(workspace), ws_bytes, _stream())
    _check("attn_bwd_ex", st)
    return dq, dk, dv, D


NOALLOC_SCRATCH_BYTES = 64 << 20  # ATTN_NOALLOC_SCRATCH_BYTES


def bwd_noalloc(q, k, v, o, do, lse, outs, causal: bool = True, scale: float | None = None, kv_len=None,
                block_mask=None):
    """:func:`bwd` through attn_bwd_noalloc: no workspace, the library's static scratch takes the
    split partials.  ``outs = (dQ, dK, dV, D)`` must be given (nothing is allocated here); kv_len and
    block_mask, if given, should already be device tensors."""
    B, H, N, d = _check_qkv(q, k, v, o, do)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    dq, dk, dv, D = outs
    st = load_library().attn_bwd_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(do), _ptr(lse), _ptr(dq), _ptr(dk),
                                         _ptr(dv), _ptr(D), B, H, N, d, int(bool(causal)), scale, _DTYPES[q.dtype],
                                         _ptr(kv_len), _ptr(block_mask), _stream())
    _check("attn_bwd_noalloc", st)
    return dq, dk, dv, D


def rowdot(o, do, out=None):
    """D = rowsum(O o dO) in float32 (the backward's first step alone)."""
    B, H, N, d = _check_qkv(o, do)
    D = torch.empty((B, H, N), dtype=torch.float32, device=o.device) if out is None else out
    st = load_library().attn_bwd_rowdot(_ptr(o), _ptr(do), _ptr(D), B, H, N, d, _DTYPES[o.dtype], _stream())
    _check("attn_bwd_rowdot", st)
    return D


def bwd_dkdv(q, k, v, do, lse, D, causal: bool = True, scale: float | None = None, kv_len=None, outs=None):
    """dK, dV alone (the backward's second step), given L and D. Returns ``(dK, dV)``."""
    B, H, N, d = _check_qkv(q, k, v, do)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    dk, dv = (torch.empty_like(k), torch.empty_like(v)) if outs is None else outs
    kv = kv_len_tensor(kv_len, B, q.device)
    st = load_library().attn_bwd_dkdv(_ptr(q), _ptr(k), _ptr(v), _ptr(do), _ptr(lse), _ptr(D), _ptr(dk), _ptr(dv),
                                      B, H, N, d, int(bool(causal)), scale, _DTYPES[q.dtype], _ptr(kv), _stream())
    _check("attn_bwd_dkdv", st)
    return dk, dv


def bwd_dq(q, k, v, do, lse, D, causal: bool = True, scale: float | None = None, kv_len=None, out=None, o=None):
    """dQ alone, given L.  With ``o`` (the forward output) the kernel also computes D = rowsum(O o dO)
    into ``D`` (an output then); without it ``D`` is an input.  Returns dQ."""
    B, H, N, d = _check_qkv(q, k, v, do)
    if o is not None:
        _check_qkv(q, o)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    dq = torch.empty_like(q) if out is None else out
    kv = kv_len_tensor(kv_len, B, q.device)
    st = load_library().attn_bwd_dq(_ptr(q), _ptr(k), _ptr(v), _ptr(do), _ptr(o), _ptr(lse), _ptr(D), _ptr(dq), B, H,
                                    N, d, int(bool(causal)), scale, _DTYPES[q.dtype], _ptr(kv), _stream())
    _check("attn_bwd_dq", st)
    return dq


def bwd_launches(B: int, H: int, N: int, d: int, dtype) -> int:
    """Number of kernels attn_bwd launches for this problem (1: dQ and dK/dV share one launch)."""
    n = load_library().attn_bwd_launches(int(B), int(H), int(N), int(d), _DTYPES[dtype])
    if n < 0:
        raise AttnError("attn_bwd_launches", n, status_string(n))
    return n


def supported(dtype, d: int) -> bool:
    return bool(load_library().attn_supported(_DTYPES[dtype], int(d)))
