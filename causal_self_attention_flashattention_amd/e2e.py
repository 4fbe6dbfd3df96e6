"""End-to-end timing of a Transformer language model with the attention swapped in.

CS336 Assignment 2 (systems), §2.1.2 Table 1 (model sizes; vocabulary 10,000, batch 4, context
512 unless stated) and §2.1.3 Problem (benchmarking_script): random weights and data, time the
forward pass, forward + backward, and a full training step with AdamW, 5 warm-up steps then the
mean and standard deviation over 10 measured steps.

The model is the assignment's pre-norm decoder-only Transformer as the pages describe it: token
embedding, per block RMSNorm -> causal multi-head self-attention with rotary position embedding
-> residual, RMSNorm -> SwiGLU feed-forward (d_ff) -> residual, a final RMSNorm and an output
projection.  Only the attention is ours; everything else is plain PyTorch.

    python -m causal_self_attention_flashattention_amd.e2e --size small --attn flash,sdpa,materialised

Attention implementations:
  flash         this package's HIP kernels (``flash_attention``)
  sdpa          torch.nn.functional.scaled_dot_product_attention (PyTorch-ROCm's own kernels)
  materialised  S and P built explicitly (eq. 1), backward by eqs. 7-11 written out
"""

from __future__ import annotations

import argparse
import math
import statistics
import time

import torch
import torch.nn as nn
import torch.nn.functional as F

from .function import flash_attention
from .sweep import materialised_backward, materialised_forward

# Table 1: d_model, d_ff, num_layers, num_heads
SIZES = {
    "small": (768, 3072, 12, 12),
    "medium": (1024, 4096, 24, 16),
    "large": (1280, 5120, 36, 20),
    "xl": (2560, 10240, 32, 32),
    "10B": (4608, 12288, 50, 36),
}


class _Materialised(torch.autograd.Function):
    """Causal attention with S and P materialised; backward by the explicit eqs. 7-11."""

    @staticmethod
    def forward(ctx, q, k, v, scale):
        o, p = materialised_forward(q, k, v, scale)
        ctx.save_for_backward(q, k, v, p)
        ctx.scale = scale
        return o

    @staticmethod
    def backward(ctx, do):
        q, k, v, p = ctx.saved_tensors
        dq, dk, dv = materialised_backward(q, k, v, do.contiguous(), p, ctx.scale)
        return dq, dk, dv, None


def attention(q, k, v, impl):
    """Causal attention of [B, H, N, d] tensors with the chosen implementation (a name above, or a
    callable ``impl(q, k, v, scale)``)."""
    scale = 1.0 / math.sqrt(q.shape[-1])
    if callable(impl):
        return impl(q, k, v, scale)
    if impl == "flash":
        return flash_attention(q, k, v, is_causal=True, scale=scale)
    if impl == "sdpa":
        return F.scaled_dot_product_attention(q, k, v, is_causal=True, scale=scale)
    if impl == "materialised":
        return _Materialised.apply(q.contiguous(), k.contiguous(), v.contiguous(), scale)
    raise ValueError(f"unknown attention implementation {impl!r}")


def _up(x):
    """At least float32 (bfloat16 activations are normalised and rotated in float32)."""
    return x.float() if x.dtype in (torch.bfloat16, torch.float16) else x


class RMSNorm(nn.Module):
    def __init__(self, d: int, eps: float = 1e-5):
        super().__init__()
        self.weight = nn.Parameter(torch.ones(d))
        self.eps = eps

    def forward(self, x):
        xf = _up(x)
        return (xf * torch.rsqrt(xf.pow(2).mean(-1, keepdim=True) + self.eps)).to(x.dtype) * self.weight


def rope_tables(head_dim: int, n: int, theta: float = 10000.0, device=None):
    inv = theta ** (-torch.arange(0, head_dim, 2, device=device, dtype=torch.float32) / head_dim)
    ang = torch.arange(n, device=device, dtype=torch.float32)[:, None] * inv[None, :]
    return torch.cos(ang), torch.sin(ang)


def apply_rope(x, cos, sin):
    """Rotate consecutive pairs (x_2i, x_2i+1) of the last dim by position-dependent angles."""
    x1, x2 = _up(x[..., 0::2]), _up(x[..., 1::2])
    r1, r2 = x1 * cos - x2 * sin, x1 * sin + x2 * cos
    return torch.stack((r1, r2), dim=-1).flatten(-2).to(x.dtype)


class Block(nn.Module):
    def __init__(self, d_model: int, d_ff: int, n_heads: int, impl: str):
        super().__init__()
        self.h, self.impl = n_heads, impl
        self.norm1, self.norm2 = RMSNorm(d_model), RMSNorm(d_model)
        self.qkv = nn.Linear(d_model, 3 * d_model, bias=False)
        self.out = nn.Linear(d_model, d_model, bias=False)
        self.w1 = nn.Linear(d_model, d_ff, bias=False)
        self.w3 = nn.Linear(d_model, d_ff, bias=False)
        self.w2 = nn.Linear(d_ff, d_model, bias=False)

    def forward(self, x, cos, sin):
        B, N, C = x.shape
        qkv = self.qkv(self.norm1(x)).view(B, N, 3, self.h, C // self.h).permute(2, 0, 3, 1, 4)
        q, k, v = apply_rope(qkv[0], cos, sin), apply_rope(qkv[1], cos, sin), qkv[2]
        a = attention(q.contiguous(), k.contiguous(), v.contiguous(), self.impl)
        x = x + self.out(a.transpose(1, 2).reshape(B, N, C))
        h = self.norm2(x)
        return x + self.w2(F.silu(self.w1(h)) * self.w3(h))


class TransformerLM(nn.Module):
    def __init__(self, vocab: int, d_model: int, d_ff: int, n_layers: int, n_heads: int, impl: str):
        super().__init__()
        self.emb = nn.Embedding(vocab, d_model)
        self.blocks = nn.ModuleList(Block(d_model, d_ff, n_heads, impl) for _ in range(n_layers))
        self.norm = RMSNorm(d_model)
        self.head = nn.Linear(d_model, vocab, bias=False)
        self.head_dim = d_model // n_heads

    def forward(self, tokens):
        n = tokens.shape[1]
        cos, sin = rope_tables(self.head_dim, n, device=tokens.device)
        x = self.emb(tokens)
        for blk in self.blocks:
            x = blk(x, cos, sin)
        return self.head(self.norm(x))


def _timed(fn, warmup: int, steps: int):
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    out = []
    for _ in range(steps):
        t0 = time.perf_counter()
        fn()
        torch.cuda.synchronize()
        out.append((time.perf_counter() - t0) * 1e3)
    return statistics.mean(out), (statistics.stdev(out) if len(out) > 1 else 0.0)


def benchmark(size: str, impl: str, ctx: int = 512, batch: int = 4, vocab: int = 10000,
              dtype=torch.bfloat16, warmup: int = 5, steps: int = 10, seed: int = 0) -> dict:
    d_model, d_ff, n_layers, n_heads = SIZES[size]
    torch.manual_seed(seed)
    with torch.device("cuda"):
        model = TransformerLM(vocab, d_model, d_ff, n_layers, n_heads, impl).to(dtype=dtype)
    opt = torch.optim.AdamW(model.parameters(), lr=1e-4)
    g = torch.Generator(device="cuda").manual_seed(seed)
    x = torch.randint(0, vocab, (batch, ctx), device="cuda", generator=g)
    y = torch.randint(0, vocab, (batch, ctx), device="cuda", generator=g)

    def loss_fn():
        return F.cross_entropy(model(x).float().view(-1, vocab), y.view(-1))

    def fwd():
        with torch.no_grad():
            loss_fn()

    def fwd_bwd():
        model.zero_grad(set_to_none=True)
        loss_fn().backward()

    def step():
        opt.zero_grad(set_to_none=True)
        loss_fn().backward()
        opt.step()

    row = {"size": size, "attn": impl, "ctx": ctx, "dtype": str(dtype).replace("torch.", "")}
    try:
        for name, fn in (("fwd", fwd), ("fwd_bwd", fwd_bwd), ("train_step", step)):
            row[name + "_ms"], row[name + "_std"] = _timed(fn, warmup, steps)
    except torch.OutOfMemoryError:
        row["status"] = "OOM"
    del model, opt
    torch.cuda.empty_cache()
    return row


def main() -> None:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--size", default="small", help="comma list of " + ",".join(SIZES))
    ap.add_argument("--attn", default="flash,sdpa,materialised")
    ap.add_argument("--ctx", type=int, default=512)
    ap.add_argument("--dtype", default="bf16", choices=("bf16", "f32"))
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--steps", type=int, default=10)
    args = ap.parse_args()
    dtype = torch.bfloat16 if args.dtype == "bf16" else torch.float32
    print("| size | attention | ctx | dtype | forward ms | forward+backward ms | train step ms |")
    print("|---|---|---|---|---|---|---|")
    for size in args.size.split(","):
        for impl in args.attn.split(","):
            r = benchmark(size, impl, ctx=args.ctx, dtype=dtype, warmup=args.warmup, steps=args.steps)
            if r.get("status") == "OOM":
                print(f"| {size} | {impl} | {args.ctx} | {r['dtype']} | OOM | OOM | OOM |", flush=True)
                continue
            cells = " | ".join(f"{r[n + '_ms']:.2f} ± {r[n + '_std']:.2f}" for n in ("fwd", "fwd_bwd", "train_step"))
            print(f"| {size} | {impl} | {args.ctx} | {r['dtype']} | {cells} |", flush=True)


if __name__ == "__main__":
    main()
