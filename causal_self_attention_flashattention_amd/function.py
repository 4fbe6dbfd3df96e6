"""Drop-in autograd function over the HIP kernels.

CS336 Assignment 2 (systems), §4.2.2 Problem (flash_forward): a ``torch.autograd.Function``
whose forward takes Q, K, V and an ``is_causal`` flag, saves L together with Q, K, V and O for the
backward, and returns O; its backward (Problem (flash_backward)) returns dQ, dK, dV.  Both passes
run in libattn's kernels (``attn_fwd`` / ``attn_bwd``); this module only reshapes and marshals.

Inputs are ``[batch, N, d]`` (the hand-out's layout) or ``[B, H, N, d]``; float32 or bfloat16, on
the GPU.  ``scale`` defaults to 1/sqrt(d); ``kv_len`` (optional, one length per leading batch
row) masks keys at or beyond that position, as a key-padding mask; ``block_mask`` (optional,
``[ceil(N/64)]^2``, non-zero = attend) makes it block-sparse attention over 64 x 64 blocks.
"""

from __future__ import annotations

import torch

from . import binding


class FlashAttention(torch.autograd.Function):
    @staticmethod
    def forward(ctx, q, k, v, is_causal: bool = False, scale: float | None = None, kv_len=None, block_mask=None):
        three_d = q.dim() == 3
        if three_d:
            q, k, v = (t.unsqueeze(1) for t in (q, k, v))
        q, k, v = (t.contiguous() for t in (q, k, v))
        kv = binding.kv_len_tensor(kv_len, q.shape[0], q.device)
        bm = None if block_mask is None else binding.block_mask_tensor(block_mask, q.shape[2], q.device)
        o, L = binding.fwd(q, k, v, causal=is_causal, scale=scale, kv_len=kv, block_mask=bm)
        ctx.save_for_backward(q, k, v, o, L, kv, bm)
        ctx.is_causal, ctx.scale, ctx.three_d = bool(is_causal), scale, three_d
        return o.squeeze(1) if three_d else o

    @staticmethod
    def backward(ctx, do):
        q, k, v, o, L, kv, bm = ctx.saved_tensors
        if ctx.three_d:
            do = do.unsqueeze(1)
        dq, dk, dv, _ = binding.bwd(q, k, v, o, do.contiguous(), L, causal=ctx.is_causal, scale=ctx.scale,
                                    kv_len=kv, block_mask=bm)
        if ctx.three_d:
            dq, dk, dv = dq.squeeze(1), dk.squeeze(1), dv.squeeze(1)
        return dq, dk, dv, None, None, None, None


def flash_attention(q, k, v, is_causal: bool = False, scale: float | None = None, kv_len=None, block_mask=None):
    """softmax(mask(scale Q K^T)) V with gradients, computed by the HIP kernels."""
    return FlashAttention.apply(q, k, v, is_causal, scale, kv_len, block_mask)
