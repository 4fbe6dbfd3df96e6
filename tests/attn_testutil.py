"""Helpers for the GPU parity tests: run the HIP path through the C ABI, run the CPU oracle on
the same seeded inputs, and compare element by element."""

from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

import causal_self_attention_flashattention_amd as attn
import oracle.attention as O

# Tolerances: float32 inputs -> max |gpu - ref| <= 1e-4; bfloat16 inputs with fp32 accumulation ->
# elementwise |gpu - ref| <= 2e-2 + 1e-2 |ref| (the bf16 output rounding alone is 2^-9 |ref|).
F32_ATOL = 1e-4
BF16_ATOL, BF16_RTOL = 2e-2, 1e-2


def require_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    attn.load_library()


def announce(msg: str):
    print(f"[gpu-case] {msg}", file=sys.stderr, flush=True)


def to_dev(inputs: dict, device="cuda"):
    out = {}
    for k, t in inputs.items():
        out[k] = None if t is None else t.to(device)
    return out


def run_gpu(dev: dict, causal: bool, scale: float, with_bwd: bool = True):
    o, L = attn.fwd(dev["q"], dev["k"], dev["v"], causal=causal, scale=scale, kv_len=dev.get("kv_len"))
    res = {"O": o, "L": L}
    if with_bwd:
        dq, dk, dv, D = attn.bwd(dev["q"], dev["k"], dev["v"], o, dev["do"], L, causal=causal, scale=scale,
                                 kv_len=dev.get("kv_len"))
        res.update(dQ=dq, dK=dk, dV=dv, D=D)
    torch.cuda.synchronize()
    return res


def heads_to_numpy(t: torch.Tensor, heads):
    """Float64 numpy [B, H, ...] holding only the listed heads (NaN elsewhere)."""
    B, H = t.shape[:2]
    out = np.full(tuple(t.shape), np.nan)
    for b, h in heads:
        out[b, h] = t[b, h].double().cpu().numpy()
    return out


def d_slack(o_ref: np.ndarray, do, dtype: str) -> np.ndarray:
    """Extra tolerance for D = rowsum(O o dO).  D is formed from the stored O, which the forward
    rounds to the output dtype: in bfloat16 each O_c carries up to half an ulp (2^-9 relative) of
    rounding on top of a computed error of the same order, so |dD_i| can reach
    2^-8 * sum_c |O_ic dO_ic| even when O itself is within its tolerance.  float32: none."""
    if dtype == "f32":
        return np.zeros(o_ref.shape[:-1])
    do = do.detach().double().cpu().numpy() if hasattr(do, "detach") else np.asarray(do, dtype=np.float64)
    return 2.0 ** -8 * np.abs(o_ref * do).sum(-1)


def oracle_ref(inputs: dict, causal: bool, scale: float, heads=None, with_bwd: bool = True):
    kv = inputs.get("kv_len")
    kv = None if kv is None else kv.tolist()
    o, L = O.attention_forward(inputs["q"], inputs["k"], inputs["v"], causal=causal, scale=scale, kv_len=kv,
                               heads=heads)
    ref = {"O": o, "L": L}
    if with_bwd:
        dq, dk, dv, dref = O.attention_backward(inputs["q"], inputs["k"], inputs["v"], inputs["do"], causal=causal,
                                                scale=scale, kv_len=kv, heads=heads)
        ref.update(dQ=dq, dK=dk, dV=dv, D=dref)
        ref["D_slack"] = d_slack(o, inputs["do"], "f32" if inputs["q"].dtype == torch.float32 else "bf16")
    return ref


def check_close(name: str, got: np.ndarray, ref: np.ndarray, dtype: str, slack=0.0):
    """Assert the tolerance (plus ``slack``, broadcast like ref) on every non-NaN reference element;
    return (max abs, max rel, worst index)."""
    sel = ~np.isnan(ref)
    g, r = got[sel], ref[sel]
    sl = np.broadcast_to(slack, ref.shape)[sel]
    assert np.all(np.isfinite(g)), f"{name}: non-finite GPU values"
    err = np.abs(g - r)
    if dtype == "f32":
        bad = err > F32_ATOL + sl
    else:
        bad = err > BF16_ATOL + BF16_RTOL * np.abs(r) + sl
    worst = int(np.argmax(err)) if err.size else 0
    stats = (float(err.max()) if err.size else 0.0,
             float((err / np.maximum(np.abs(r), 1e-6)).max()) if err.size else 0.0)
    if bad.any():
        idx = np.argwhere(sel)[np.flatnonzero(bad)[0]]
        raise AssertionError(f"{name}: {int(bad.sum())} elements out of tolerance; first at {tuple(idx)} "
                             f"gpu={got[tuple(idx)]!r} ref={ref[tuple(idx)]!r}; max abs err {stats[0]:.3g}")
    return stats, worst


def compare_all(res: dict, ref: dict, dtype: str, heads):
    report = {}
    for key in ref:
        if key == "D_slack":
            continue
        got = heads_to_numpy(res[key], heads)
        slack = ref.get("D_slack", 0.0) if key == "D" else 0.0
        report[key] = check_close(key, got, ref[key], dtype, slack)[0]
    return report
