"""The handout's FlashAttention-2 benchmark sweep on one MI355X (CS336 Assignment 2, Problem
(flash_benchmarking)): batch 1, causal masking, sequence lengths 2^7 .. 2^16, head dims
2^4 .. 2^7, bfloat16 and float32; forward, backward and end-to-end latency of the HIP kernels
next to a plain materialised PyTorch attention (eq. 1 forward, eqs. 7-11 backward).

    python -m causal_self_attention_flashattention_amd.sweep [--quick] [--json]

Times are medians over repeated runs between HIP events on the current stream.  The materialised
baseline uses only contiguous matrix-product operands, builds S and P explicitly, and reports
OOM where its N x N buffers do not fit.
"""

from __future__ import annotations

import argparse
import json
import math
import statistics

import torch

from . import binding as attn
from .inputs import make_inputs


def _time(fn, min_reps: int = 10, max_ms: float = 1500.0) -> float:
    """Median milliseconds of fn() over repeated runs (after two warm-up runs)."""
    fn()
    fn()
    torch.cuda.synchronize()
    times, spent = [], 0.0
    while len(times) < min_reps or (spent < max_ms and len(times) < 100):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        fn()
        b.record()
        b.synchronize()
        t = a.elapsed_time(b)
        times.append(t)
        spent += t
        if spent > max_ms and len(times) >= 3:
            break
    return statistics.median(times)


def materialised_forward(q, k, v, scale):
    """S = scale Q K^T with masked entries at -inf, P = row softmax, O = P V (eq. 1 / eqs. 4-6)."""
    n = q.shape[-2]
    s = torch.matmul(q, k.transpose(-1, -2).contiguous()) * scale
    mask = torch.ones(n, n, dtype=torch.bool, device=q.device).tril_()
    s = s.masked_fill(~mask, float("-inf"))
    p = torch.softmax(s.float(), dim=-1).to(q.dtype)
    return torch.matmul(p, v), p


def materialised_backward(q, k, v, do, p, scale):
    """Eqs. 7-11: dV = P^T dO, dP = dO V^T, dS = P o (dP - rowsum(P o dP)), dQ, dK."""
    dv = torch.matmul(p.transpose(-1, -2).contiguous(), do)
    dp = torch.matmul(do, v.transpose(-1, -2).contiguous())
    pf = p.float()
    ds = (pf * (dp.float() - (pf * dp.float()).sum(-1, keepdim=True))).to(q.dtype)
    dq = torch.matmul(ds, k) * scale
    dk = torch.matmul(ds.transpose(-1, -2).contiguous(), q) * scale
    return dq, dk, dv


def run_case(N: int, d: int, dtype: str, with_baseline: bool = True) -> dict:
    inp = make_inputs(1, 1, N, d, dtype, seed=N + d)
    q, k, v, do = (inp[n].cuda() for n in ("q", "k", "v", "do"))
    scale = 1.0 / math.sqrt(d)
    o, L = attn.fwd(q, k, v, causal=True, scale=scale)
    outs = (torch.empty_like(q), torch.empty_like(k), torch.empty_like(v), torch.empty_like(L))
    row = {"N": N, "d": d, "dtype": dtype}
    row["fwd_ms"] = _time(lambda: attn.fwd(q, k, v, causal=True, scale=scale, out=o, lse=L))
    row["bwd_ms"] = _time(lambda: attn.bwd(q, k, v, o, do, L, causal=True, scale=scale, outs=outs))

    def e2e():
        attn.fwd(q, k, v, causal=True, scale=scale, out=o, lse=L)
        attn.bwd(q, k, v, o, do, L, causal=True, scale=scale, outs=outs)

    row["e2e_ms"] = _time(e2e)
    if with_baseline:
        try:
            _, p = materialised_forward(q, k, v, scale)
            row["base_fwd_ms"] = _time(lambda: materialised_forward(q, k, v, scale), max_ms=3000.0)
            row["base_bwd_ms"] = _time(lambda: materialised_backward(q, k, v, do, p, scale), max_ms=3000.0)
            del p

            def base_e2e():
                _, pp = materialised_forward(q, k, v, scale)
                materialised_backward(q, k, v, do, pp, scale)

            row["base_e2e_ms"] = _time(base_e2e, max_ms=3000.0)
        except torch.OutOfMemoryError:
            row["base_fwd_ms"] = row["base_bwd_ms"] = row["base_e2e_ms"] = "OOM"
        torch.cuda.empty_cache()
    return row


def blocksparse_case(B: int, H: int, N: int, d: int, density: float, seed: int = 0, pattern: str = "random") -> dict:
    """Forward and backward time of causal block-sparse attention (bfloat16) next to the same
    problem dense.  ``pattern`` "random": each 64 x 64 block kept with probability ``density``;
    "band": a local band of blocks around the diagonal plus the first block column (global
    tokens), its width chosen so that about ``density`` of the causal blocks are kept.  The
    diagonal is always kept.  ``kept`` is the fraction of the causal (lower-triangle) blocks kept."""
    import numpy as np

    inp = make_inputs(B, H, N, d, "bf16", seed=seed)
    q, k, v, do = (inp[n].cuda() for n in ("q", "k", "v", "do"))
    tb = attn.mask_blocks(N)
    if pattern == "band":
        width = max(1, int(round(density * (tb + 1) / 2)))
        rr, cc = np.indices((tb, tb))
        m = ((np.abs(rr - cc) < width) | (cc == 0)).astype(np.uint8)
    else:
        r = np.random.default_rng(seed)
        m = (r.random((tb, tb)) < density).astype(np.uint8)
    np.fill_diagonal(m, 1)
    tri = np.tril(np.ones((tb, tb), dtype=bool))
    kept = float(m[tri].sum()) / float(tri.sum())
    bm = attn.block_mask_tensor(m, N, q.device)
    row = {"B": B, "H": H, "N": N, "d": d, "density": density, "kept": kept, "pattern": pattern}
    for tag, mask in (("dense", None), ("sparse", bm)):
        o, L = attn.fwd(q, k, v, causal=True, block_mask=mask)
        outs = (torch.empty_like(q), torch.empty_like(k), torch.empty_like(v), torch.empty_like(L))
        row[tag + "_fwd_ms"] = _time(lambda: attn.fwd(q, k, v, causal=True, block_mask=mask, out=o, lse=L))
        row[tag + "_bwd_ms"] = _time(lambda: attn.bwd(q, k, v, o, do, L, causal=True, block_mask=mask, outs=outs))
    return row


def main() -> None:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--quick", action="store_true", help="N in {2^7, 2^10, 2^13, 2^16} only")
    ap.add_argument("--json", action="store_true", help="one JSON object per case instead of a table")
    ap.add_argument("--no-baseline", action="store_true")
    ap.add_argument("--blocksparse", action="store_true",
                    help="instead: block-sparse timing against density (B=1, H=16, bf16, causal)")
    args = ap.parse_args()
    attn.load_library()
    if args.blocksparse:
        print("| pattern | N | d | causal blocks kept | dense fwd ms | sparse fwd ms | dense bwd ms | sparse bwd ms | "
              "fwd+bwd speed-up |")
        print("|---|---|---|---|---|---|---|---|---|")
        for pattern in ("random", "band"):
            for N in (4096, 16384):
                for d in (64, 128):
                    for dens in (0.5, 0.25, 0.125):
                        r = blocksparse_case(1, 16, N, d, dens, pattern=pattern)
                        sp = (r["dense_fwd_ms"] + r["dense_bwd_ms"]) / (r["sparse_fwd_ms"] + r["sparse_bwd_ms"])
                        print(f"| {pattern} | {N} | {d} | {r['kept']:.3f} | {r['dense_fwd_ms']:.3f} | "
                              f"{r['sparse_fwd_ms']:.3f} | {r['dense_bwd_ms']:.3f} | {r['sparse_bwd_ms']:.3f} | {sp:.2f}x |",
                              flush=True)
        return
    ns = [2 ** e for e in ((7, 10, 13, 16) if args.quick else range(7, 17))]
    if not args.json:
        print("| dtype | d | N | fwd ms | bwd ms | e2e ms | materialised fwd ms | materialised bwd ms | materialised e2e ms |")
        print("|---|---|---|---|---|---|---|---|---|")
    for dtype in ("bf16", "f32"):
        for d in (16, 32, 64, 128):
            for N in ns:
                r = run_case(N, d, dtype, with_baseline=not args.no_baseline)
                if args.json:
                    print(json.dumps(r), flush=True)
                else:
                    f = lambda x: x if isinstance(x, str) else f"{x:.3f}"  # noqa: E731
                    print(f"| {dtype} | {d} | {N} | {f(r['fwd_ms'])} | {f(r['bwd_ms'])} | {f(r['e2e_ms'])} | "
                          f"{f(r.get('base_fwd_ms', '-'))} | {f(r.get('base_bwd_ms', '-'))} | "
                          f"{f(r.get('base_e2e_ms', '-'))} |", flush=True)


if __name__ == "__main__":
    main()
