#!/usr/bin/env python3
"""Benchmark: causal attention forward + backward on one MI355X, through the C ABI.

One step = the whole path over one batch: attn_fwd, then the backward exactly as attn_bwd launches it
-- either its two kernels called one by one (attn_bwd_dq, which also computes D = rowsum(O o dO),
then attn_bwd_dkdv) or, for small problems, attn_bwd itself, whose dQ and dK/dV work share one
launch -- on torch's current HIP stream, with inputs resident in HBM.  W untimed warm-up steps, then K timed steps
bracketed by torch.cuda.synchronize(); on every --event-every-th timed step, HIP events recorded on
the same stream between the kernels give each kernel's average duration (an event record between
two kernels leaves a gap of a few microseconds, which on the small workload would add about a
quarter to every step if each step carried them).  Prints one JSON line.

Algorithmic FLOPs (matrix products only, 2 FLOPs per multiply-add; causal-skipped half and the
dQ kernel's recompute of S and dP not counted):
  npairs = sum_i (number of unmasked keys of query i)
  forward 4*d*npairs per head (Q K^T and P V), backward 10*d*npairs per head (S, dP, dV, dK, dQ).

The headline workload is the largest model shape, B=1 H=36 N=16384 d=128 ("10b-16k"); the
d = 64 long-context shape B=4 H=20 N=4096 ("large-4k") is timed in the same run and reported under
"secondary" with the same fields.  Per-step device times (HIP events between consecutive steps)
give the mean, standard deviation and median; `value` itself is wall-clock throughput over the
K timed steps between two synchronisations.
"""

from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "causal attention fwd+bwd TFLOP/s (bf16) and % of MI355X MFMA peak"
PEAK_BF16_TFLOPS = 2516.6  # 256 CU x 4096 FLOP/clk/CU x 2.4 GHz, dense bf16 MFMA
PEAK_F32_TFLOPS = 157.3
PEAK_HBM_GBS = 8000.0
DEFAULT_WORKLOAD = "10b-16k"
SECONDARY_WORKLOADS = ("large-4k",)
KERNELS_SPLIT = ("fwd", "dq", "dkdv")  # launch order of one step when attn_bwd launches two kernels
KERNELS_FUSED = ("fwd", "bwd")        # ... and when its dQ and dK/dV work share one launch
KERNEL_SOURCES = ("attn_device.h", "block_order.h", "lds_layout.h", "attn_fwd.hip", "attn_bwd.hip")


def npairs(N: int, kv: int, causal: bool) -> int:
    if not causal:
        return N * kv
    # sum_{i<N} min(i+1, kv)
    m = min(N, kv)
    return m * (m + 1) // 2 + (N - m) * kv


def kernel_work(w, kv: int) -> dict:
    """Algorithmic work per launch of each kernel (matrix-product FLOPs)."""
    BH, d = w.B * w.H, w.d
    P = npairs(w.N, kv, w.causal)
    es = 2 if w.dtype == "bf16" else 4
    return {
        "fwd": ("flop", 4 * d * P * BH),
        "dkdv": ("flop", 8 * d * P * BH),   # S, dP, dV, dK
        "dq": ("flop", 2 * d * P * BH),     # dQ (its recompute of S and dP, and D, are not credited)
        "bwd": ("flop", 10 * d * P * BH),   # dQ and dK/dV in one launch
    }


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "causal_self_attention_flashattention_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def load_traffic(kernel: str, workload: str):
    """HBM bytes per launch from committed rocprofv3 counter summaries, if taken on the current kernels."""
    path = os.path.join(ROOT, "profiles", f"hbm_traffic_{workload}.txt")
    if not os.path.exists(path):
        return None
    for line in open(path):
        if line.startswith("traffic-json:"):
            rec = json.loads(line.split(":", 1)[1])
            if rec.get("source_hash") != kernel_source_hash():
                return None
            k = rec.get("kernels", {}).get(kernel)
            return None if k is None else k.get("bytes_per_launch")
    return None


def cpu_baseline(inputs, w, kv_list, target_s: float):
    """Time the float64 oracle (as it stands) on a bounded sample of heads of the same workload:
    whole heads, forward then backward, until ``target_s`` has passed (at least one head)."""
    import numpy as np  # noqa: F401
    from threadpoolctl import threadpool_info

    import oracle.attention as O

    blas = [p for p in threadpool_info() if p.get("user_api") == "blas"]
    threads = max([p.get("num_threads", 1) for p in blas] or [1])
    vendor = ", ".join(f"{p.get('internal_api')} {p.get('version')} ({p.get('threading_layer')})" for p in blas)
    heads = [(b, h) for b in range(w.B) for h in range(w.H)]
    done, flops = 0, 0
    t0 = time.perf_counter()
    while True:
        b, h = heads[done % len(heads)]
        kv = None if kv_list is None else kv_list[b]
        q, k, v, do = (inputs[n][b, h] for n in ("q", "k", "v", "do"))
        O.head_forward(q, k, v, causal=w.causal, scale=w.scale, kv=kv)
        O.head_backward(q, k, v, do, causal=w.causal, scale=w.scale, kv=kv)
        flops += 14 * w.d * npairs(w.N, w.N if kv is None else kv, w.causal)
        done += 1
        el = time.perf_counter() - t0
        if el >= target_s or done >= 64 * len(heads):
            break
    return {
        "value": flops / el / 1e12,
        "unit": "TFLOP/s",
        "cores": int(threads),
        "kind": "oracle",
        "blas": vendor or "unknown",
        "sample": f"{done} (batch, head) fwd+bwd passes of the {w.name} workload "
                  f"({done / len(heads):.3f} x its {len(heads)} heads: whole heads, materialised N x N, "
                  f"float64 numpy), {el:.1f} s, scaled by the same algorithmic FLOP count",
    }


def copy_probe(nbytes: int, reps: int) -> None:
    """Copy ``nbytes`` between two device buffers ``reps`` times: each launch reads and writes exactly
    ``nbytes`` of HBM, so HBM byte counters taken on it give their scale factor."""
    import torch

    src = torch.ones(nbytes, dtype=torch.uint8, device="cuda:0")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t0) / reps
    print(json.dumps({"copy_bytes": nbytes, "reps": reps, "us_per_copy": dt * 1e6,
                      "GB/s (read+write)": 2 * nbytes / dt / 1e9}), flush=True)


def rowdot_bench(args, w, lib, P_, B, H, N, d, dt, stream, step_binding):
    """Time attn_bwd_rowdot alone: it reads O and dO once and writes D (HBM-bound, no reuse)."""
    import torch

    step_binding()  # O (and L) from the forward, as the pass sees them in the backward
    for _ in range(args.warmup):
        lib.attn_bwd_rowdot(P_["o"], P_["do"], P_["D"], B, H, N, d, dt, stream)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    st = 0
    for _ in range(args.steps):
        st |= lib.attn_bwd_rowdot(P_["o"], P_["do"], P_["D"], B, H, N, d, dt, stream)
    e1.record()
    torch.cuda.synchronize()
    if st != 0:
        raise RuntimeError(f"attn_bwd_rowdot failed with status {st}")
    us = e0.elapsed_time(e1) * 1e3 / args.steps
    es = 2 if w.dtype == "bf16" else 4
    nbytes = 2 * B * H * N * d * es + 4 * B * H * N
    gbs = nbytes / (us * 1e-6) / 1e9
    print(json.dumps({
        "metric": "D = rowsum(O o dO) pass, HBM GB/s", "value": gbs, "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "us_per_launch": us, "higher_is_better": True,
        "dtype": w.dtype, "data": "synthetic",
        "config": {"workload": w.name, "B": B, "H": H, "N": N, "d": d, "bytes_per_launch": nbytes},
        "roofline": {"bound": "hbm", "achieved": gbs, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": gbs / PEAK_HBM_GBS, "traffic": None, "kernel": "rowdot"},
    }), flush=True)


def time_workload(args, name, attn, lib, hip, torch):
    """Run W warm-up and K timed steps of one workload; return its JSON record (without cpu_baseline)
    and its CPU inputs."""
    import statistics

    from causal_self_attention_flashattention_amd.inputs import WORKLOADS, make_workload_inputs

    w = WORKLOADS[name]
    inputs = make_workload_inputs(w, args.seed)
    kv_list = None if inputs["kv_len"] is None else inputs["kv_len"].tolist()
    kv = w.N if kv_list is None else kv_list[0]
    assert kv_list is None or len(set(kv_list)) == 1
    dev = torch.device("cuda:0")
    g = {k: (None if t is None else t.to(dev)) for k, t in inputs.items()}
    q, k, v, do, kvd = g["q"], g["k"], g["v"], g["do"], g["kv_len"]
    o, L = torch.empty_like(q), torch.empty(q.shape[:3], dtype=torch.float32, device=dev)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    D = torch.empty(q.shape[:3], dtype=torch.float32, device=dev)

    # The timed loop calls the C ABI directly with pre-resolved pointers and records the HIP events
    # through the runtime, so that host-side overhead stays well below the kernels' own time (the
    # arguments were validated by the same calls through the binding during warm-up).
    stream = torch.cuda.current_stream().cuda_stream
    P_ = {n: t.data_ptr() for n, t in dict(q=q, k=k, v=v, o=o, L=L, do=do, D=D, dq=dq, dk=dk, dv=dv).items()}
    kvp = None if kvd is None else kvd.data_ptr()
    dt = 1 if w.dtype == "bf16" else 0
    B, H, N, d, c, sc = w.B, w.H, w.N, w.d, int(w.causal), w.scale

    def step_binding():
        attn.fwd(q, k, v, causal=w.causal, scale=w.scale, kv_len=kvd, out=o, lse=L)
        attn.bwd(q, k, v, o, do, L, causal=w.causal, scale=w.scale, kv_len=kvd, outs=(dq, dk, dv, D))

    if args.rowdot:
        rowdot_bench(args, w, lib, P_, B, H, N, d, dt, stream, step_binding)
        return None, None

    fused = attn.bwd_launches(B, H, N, d, q.dtype) == 1
    KERNELS = KERNELS_FUSED if fused else KERNELS_SPLIT
    rec = hip.hipEventRecord

    def step(ev=None):
        if ev is not None:
            rec(ev[0], stream)
        st = lib.attn_fwd(P_["q"], P_["k"], P_["v"], P_["o"], P_["L"], B, H, N, d, c, sc, dt, kvp, stream)
        if ev is not None:
            rec(ev[1], stream)
        if fused:
            st |= lib.attn_bwd(P_["q"], P_["k"], P_["v"], P_["o"], P_["do"], P_["L"], P_["dq"], P_["dk"], P_["dv"],
                               P_["D"], B, H, N, d, c, sc, dt, kvp, stream)
            if ev is not None:
                rec(ev[2], stream)
        else:
            st |= lib.attn_bwd_dq(P_["q"], P_["k"], P_["v"], P_["do"], P_["o"], P_["L"], P_["D"], P_["dq"], B, H, N,
                                  d, c, sc, dt, kvp, stream)
            if ev is not None:
                rec(ev[2], stream)
            st |= lib.attn_bwd_dkdv(P_["q"], P_["k"], P_["v"], P_["do"], P_["L"], P_["D"], P_["dk"], P_["dv"], B, H,
                                    N, d, c, sc, dt, kvp, stream)
            if ev is not None:
                rec(ev[3], stream)
        if st != 0:
            raise RuntimeError(f"attention step failed with status {st}")

    for _ in range(max(1, args.warmup // 2)):
        step_binding()
    for _ in range(args.warmup - max(1, args.warmup // 2)):
        step()
    torch.cuda.synchronize()
    every = max(1, args.event_every)
    n_ev = (args.steps + every - 1) // every
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(len(KERNELS) + 1)] for _ in range(n_ev)]
    # one event before every timed step and one after the last: per-step device times
    sev = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    for e in evs + [sev]:  # materialise the events before the timed region
        for x in e:
            x.record()
    torch.cuda.synchronize()
    hev = [[ctypes.c_void_p(x.cuda_event) for x in e] for e in evs]
    hsev = [ctypes.c_void_p(x.cuda_event) for x in sev]
    t0 = time.perf_counter()
    per_step = not args.no_step_events
    for i in range(args.steps):
        if per_step:
            rec(hsev[i], stream)
        step(hev[i // every] if i % every == 0 else None)
    if per_step:
        rec(hsev[args.steps], stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall * 1e3 / args.steps
    per_kernel_ms = {kn: sum(e[j].elapsed_time(e[j + 1]) for e in evs) / n_ev for j, kn in enumerate(KERNELS)}
    event_ms_per_step = sum(e[0].elapsed_time(e[-1]) for e in evs) / n_ev
    # without per-step events, the event-bracketed steps stand in for the distribution
    step_ms = ([sev[i].elapsed_time(sev[i + 1]) for i in range(args.steps)] if per_step
               else [e[0].elapsed_time(e[-1]) for e in evs])

    work = kernel_work(w, kv)
    P = npairs(w.N, kv, w.causal)
    total_flop = 14 * w.d * P * w.B * w.H
    value = total_flop / (ms_per_step * 1e-3) / 1e12
    peak = PEAK_BF16_TFLOPS if w.dtype == "bf16" else PEAK_F32_TFLOPS

    # roofline of the dominant kernel
    dom = max(KERNELS, key=lambda n: per_kernel_ms[n])
    kind, amount = work[dom]
    t = per_kernel_ms[dom] * 1e-3
    if kind == "flop":
        roof = {"bound": "mfma", "achieved": amount / t / 1e12, "peak": peak, "unit": "TFLOP/s"}
    else:
        roof = {"bound": "hbm", "achieved": amount / t / 1e9, "peak": PEAK_HBM_GBS, "unit": "GB/s"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    roof["traffic"] = load_traffic(dom, w.name)
    roof["kernel"] = dom

    kernels = {}
    for n in KERNELS:
        kd, amt = work[n]
        tt = per_kernel_ms[n] * 1e-3
        kernels[n] = {"us": per_kernel_ms[n] * 1e3,
                      ("TFLOP/s" if kd == "flop" else "GB/s"): amt / tt / (1e12 if kd == "flop" else 1e9)}

    out = {
        "metric": METRIC,
        "value": value,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "step_ms": {"mean": statistics.fmean(step_ms),
                    "std": statistics.stdev(step_ms) if len(step_ms) > 1 else 0.0,
                    "median": statistics.median(step_ms), "min": min(step_ms), "max": max(step_ms),
                    "source": "HIP events between consecutive timed steps" if per_step
                    else "HIP events around every --event-every-th timed step"},
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "N": w.N, "d": w.d, "causal": w.causal,
                   "kv_len": kv, "seed": w.seed if args.seed is None else args.seed,
                   "flop_per_step": total_flop, "pct_of_peak": 100.0 * value / peak, "peak_tflops": peak,
                   "event_ms_per_step": event_ms_per_step, "event_steps": n_ev, "kernels": kernels},
        "roofline": roof,
    }
    return out, (inputs, w, kv_list)


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--secondary", default=",".join(SECONDARY_WORKLOADS),
                    help="comma-separated workloads timed after the headline one and reported under "
                         "'secondary' (empty: none)")
    ap.add_argument("--seed", type=int, default=None)
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="target length of the oracle timing")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--event-every", type=int, default=8,
                    help="record the per-kernel HIP events on every n-th timed step (1 = every step)")
    ap.add_argument("--no-step-events", action="store_true",
                    help="record no HIP event between consecutive steps (for launch-bound workloads, where an "
                         "event record adds a few microseconds to each step)")
    ap.add_argument("--rowdot", action="store_true",
                    help="instead of the attention step, time the stand-alone D = rowsum(O o dO) pass "
                         "(attn_bwd_rowdot) on the workload's O and dO and report HBM GB/s")
    ap.add_argument("--copy-bytes", type=int, default=0,
                    help="instead of the attention step, time a plain device-to-device copy of this many bytes "
                         "(the reference kernel that HBM byte counters are scaled against)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py runs on exactly one GPU (asked for {max(args.gpus, world)}): attention is independent "
              "per (batch, head), so more GPUs would only split heads; no multi-GPU run is provided.",
              file=sys.stderr)
        sys.exit(2)

    import torch

    if args.copy_bytes > 0:
        copy_probe(args.copy_bytes, args.steps)
        return

    import causal_self_attention_flashattention_amd as attn

    lib = attn.load_library()
    hip = ctypes.CDLL("libamdhip64.so.7")  # the runtime torch already loaded (same soname)
    hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]

    out, ctx = time_workload(args, args.workload, attn, lib, hip, torch)
    if out is None:  # --rowdot printed its own line
        return
    if not args.rowdot:
        sec = {}
        for name in [n for n in args.secondary.split(",") if n and n != args.workload]:
            r, _ = time_workload(args, name, attn, lib, hip, torch)
            sec[name] = {key: r[key] for key in ("value", "ms_per_step", "step_ms", "config", "roofline")}
            torch.cuda.empty_cache()
        if sec:
            out["secondary"] = sec
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(*ctx, args.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
