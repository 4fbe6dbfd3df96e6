"""GPU parity: the HIP path (through the C ABI) against the CPU float64 oracle on the same seeded
inputs, element by element.

* small shapes spanning several tiles and a ragged tail, every supported head dim, both dtypes,
  causal and not, with and without key padding: every element of every head;
* the five named workloads at full size, in the launch configuration the benchmark times:
  every head where the oracle is quick, else sampled heads in full plus properties that hold
  for every head.
"""

import math

import numpy as np
import pytest
import torch

import oracle.attention as O
from causal_self_attention_flashattention_amd.inputs import WORKLOADS, make_inputs, make_workload_inputs

from attn_testutil import announce, check_close, compare_all, heads_to_numpy, oracle_ref, require_gpu, run_gpu, to_dev

pytestmark = pytest.mark.gpu

SMALL = []
for dtype in ("bf16", "f32"):
    for d in (16, 32, 64, 80, 128):
        SMALL += [
            (dtype, 2, 2, 200, d, True, None),
            (dtype, 2, 1, 257, d, False, [129, 257]),
            (dtype, 2, 2, 33, d, True, [1, 20]),
            (dtype, 1, 1, 1, d, True, None),
        ]
SMALL += [
    ("bf16", 1, 3, 384, 64, True, [300]),
    ("bf16", 1, 2, 130, 128, False, None),
    ("f32", 1, 2, 96, 64, False, [50]),
    # forward with two key groups per workgroup (grids of at most 256 query tiles, N >= 256) and
    # either side of that threshold; the first 64-head case also runs the two-group backward, the
    # 65-head one the plain two-kernel backward
    ("bf16", 2, 3, 700, 128, True, [650, 700]),
    ("bf16", 1, 2, 520, 80, True, [400]),
    ("bf16", 1, 2, 333, 32, True, None),
    ("bf16", 1, 2, 300, 16, False, [70]),
    ("bf16", 1, 64, 512, 64, True, None),
    ("bf16", 1, 65, 512, 64, True, None),
    # backward with two groups per workgroup (small bf16 grids, d <= 80, N >= 512, dense mask)
    ("bf16", 1, 2, 600, 32, True, [550]),
    ("bf16", 2, 1, 513, 16, False, None),
    ("bf16", 1, 3, 1100, 64, False, [1000]),
    # head counts that are not multiples of 8 with tile counts that are multiples of the split
    # period, so the XCD-aware block order (heads shared between XCDs by rank) is the one used
    ("bf16", 1, 36, 1024, 128, True, None),
    ("bf16", 1, 12, 1024, 64, True, [1000]),
    ("bf16", 1, 5, 1024, 64, False, None),
    ("bf16", 1, 7, 2048, 64, True, None),
    ("bf16", 3, 3, 1024, 128, True, [1024, 900, 700]),
    ("bf16", 1, 6, 1024, 80, True, None),
    ("bf16", 2, 1, 1024, 64, True, None),
    # the d = 128 forward's pipelined loop (grids above the two-group threshold) ending at the key
    # length rather than the diagonal, without causal masking, and with a partial last query tile
    ("bf16", 2, 24, 1024, 128, False, [1000, 777]),
    ("bf16", 2, 18, 1100, 128, True, [1100, 900]),
    # d = 80 with one key group per workgroup, key padding, no causal mask
    ("bf16", 2, 20, 1024, 80, False, [1000, 700]),
    # grids small enough and chains long enough for the split paths (forward key chunks, dQ key
    # chunks, dK/dV query chunks merged from float32 partials), whose partial writes carry the
    # 16-wide accumulators at d = 80 (last 16 columns) and d = 16 (all columns)
    ("bf16", 1, 2, 2048, 80, True, [1900]),
    ("bf16", 1, 1, 2048, 16, False, None),
]


@pytest.mark.parametrize("dtype,B,H,N,d,causal,kv", SMALL, ids=lambda x: str(x))
def test_small_shapes_match_oracle(dtype, B, H, N, d, causal, kv):
    require_gpu()
    seed = 1000 + N + d
    announce(f"small dtype={dtype} B={B} H={H} N={N} d={d} causal={causal} kv={kv} seed={seed}")
    inp = make_inputs(B, H, N, d, dtype, seed, kv_len=kv)
    scale = 1.0 / math.sqrt(d)
    res = run_gpu(to_dev(inp), causal, scale)
    heads = [(b, h) for b in range(B) for h in range(H)]
    ref = oracle_ref(inp, causal, scale, heads)
    compare_all(res, ref, dtype, heads)


def _sample_heads(B, H, n):
    allh = [(b, h) for b in range(B) for h in range(H)]
    if n >= len(allh):
        return allh
    idx = np.linspace(0, len(allh) - 1, n).round().astype(int)
    return [allh[i] for i in sorted(set(idx.tolist()))]


# heads checked in full against the oracle, per workload
FULL_HEADS = {"tiny-f32": 10**9, "gpt2-small": 10**9, "large-4k": 3, "xl-d80-pad": 3, "10b-16k": 1}


def _properties_all_heads(inp_dev, res, kv):
    """Facts that hold for every head at any size (checked on the GPU output of all heads)."""
    dk, dv, do = res["dK"].float(), res["dV"].float(), inp_dev["do"].float()
    for key in ("O", "L", "dQ", "dK", "dV", "D"):
        assert torch.isfinite(res[key]).all(), f"{key} has non-finite values"
    # sum_j dK_j = 0 (softmax shift invariance); sum_j dV_j = sum_i dO_i (rows of P sum to 1)
    sk = dk.sum(2).abs()
    bound_k = 2.0 ** -6 * dk.abs().sum(2) + 1e-2
    assert (sk <= bound_k).all(), f"sum_j dK_j not ~0: worst {float((sk - bound_k).max()):.3g} over bound"
    sv = (dv.sum(2) - do.sum(2)).abs()
    bound_v = 2.0 ** -6 * (dv.abs().sum(2) + do.abs().sum(2)) + 1e-2
    assert (sv <= bound_v).all(), f"sum_j dV_j != sum_i dO_i: worst {float((sv - bound_v).max()):.3g} over bound"
    if kv is not None:
        for b, n in enumerate(kv.tolist()):
            assert (res["dK"][b, :, n:] == 0).all() and (res["dV"][b, :, n:] == 0).all()


def _rows_every_head(inp, res, w, seed, nrand=32, ntail=32):
    """Every (batch, head): 32 seeded query rows plus tile-boundary rows (O, L, dQ, D) against the
    row-wise oracle, and the last ntail visible keys' dK, dV against the tail-key oracle, element by
    element.  A head, rank or per-head base mistake anywhere in the grid shows up here."""
    B, H, N = w.B, w.H, w.N
    kvl = None if inp["kv_len"] is None else inp["kv_len"].tolist()
    fixed = [0, 1, 31, 32, 63, 64, 127, 128, 255, 256, N // 2, N - 129, N - 128, N - 2, N - 1]
    got = {key: res[key].double().cpu().numpy() for key in ("O", "L", "dQ", "D", "dK", "dV")}
    for b in range(B):
        kv = None if kvl is None else kvl[b]
        hi = N if kv is None else kv
        for h in range(H):
            rng = np.random.default_rng(seed * 1000 + b * H + h)
            extra = [] if kv is None else [kv - 1, min(kv, N - 1)]
            rows = sorted({r for r in fixed + extra if 0 <= r < N} | set(rng.integers(0, N, nrand).tolist()))
            q, k, v, do = (inp[n][b, h] for n in ("q", "k", "v", "do"))
            ro, rl, rdq, rd = O.head_rows(q, k, v, do, rows, causal=w.causal, scale=w.scale, kv=kv)
            tag = f"(b={b}, h={h})"
            check_close(f"O rows {tag}", got["O"][b, h][rows], ro, w.dtype)
            check_close(f"L rows {tag}", got["L"][b, h][rows], rl, w.dtype)
            check_close(f"dQ rows {tag}", got["dQ"][b, h][rows], rdq, w.dtype)
            # D's slack for O's bf16 rounding, from the oracle's O (as for the full comparison)
            slack = 0.0 if w.dtype == "f32" else 2.0 ** -8 * np.abs(ro * do.double().numpy()[rows]).sum(-1)
            check_close(f"D rows {tag}", got["D"][b, h][rows], rd, w.dtype, slack)
            if w.causal:
                nt = min(ntail, hi)
                tk, tv = O.head_tail_keys(q, k, v, do, nt, scale=w.scale, kv=kv)
                check_close(f"dK tail keys {tag}", got["dK"][b, h][hi - nt:hi], tk, w.dtype)
                check_close(f"dV tail keys {tag}", got["dV"][b, h][hi - nt:hi], tv, w.dtype)


@pytest.mark.parametrize("name", list(WORKLOADS))
def test_workload_matches_oracle(name):
    require_gpu()
    w = WORKLOADS[name]
    announce(f"workload {name} B={w.B} H={w.H} N={w.N} d={w.d} {w.dtype} causal={w.causal} seed={w.seed}")
    inp = make_workload_inputs(w)
    dev = to_dev(inp)
    res = run_gpu(dev, w.causal, w.scale)
    _properties_all_heads(dev, res, inp["kv_len"])
    heads = _sample_heads(w.B, w.H, FULL_HEADS[name])
    ref = oracle_ref(inp, w.causal, w.scale, heads)
    rep = compare_all(res, ref, w.dtype, heads)
    announce(f"workload {name} max abs / rel errors: " + ", ".join(f"{k}={v[0]:.3g}/{v[1]:.3g}" for k, v in rep.items()))
    if FULL_HEADS[name] < w.B * w.H:
        _rows_every_head(inp, res, w, w.seed)
        announce(f"workload {name}: sampled rows and tail keys of all {w.B * w.H} heads match")


# Scores that climb along the key index (a ramp) or jump at scattered keys (spikes), so the
# forward's running row max has to move on many 32-key blocks: this exercises the rescaling of
# the output accumulator and row sum, and (head dims up to 64) the path that recomputes a key
# block's scores when its weights, formed with the stale max, sum past the bound.  Every query
# gets 4 added to each feature and every key c_j (all features), which lifts score (i, j) by about
# 4 d c_j: c_j rises by `lift` log2 units of the scaled score per key (ramp), or jumps by 12 units
# at one key in ten (spikes).  Spreading the pattern over all features keeps every key feature
# small; a pattern carried by one feature alone makes that feature large, and dQ's products with
# bf16-rounded dS then lose more than the tolerance to cancellation (sum_j dS_ij = 0).
RISING = [
    ("bf16", 1, 2, 300, 64, True, None),
    ("bf16", 1, 2, 300, 128, True, [280]),
    ("bf16", 1, 2, 300, 80, False, None),
    ("f32", 1, 2, 200, 64, False, [150]),
    ("f32", 1, 1, 160, 128, True, None),
    ("bf16", 1, 2, 520, 64, True, None),
    ("bf16", 2, 3, 700, 128, True, None),
    ("bf16", 1, 1, 2048, 64, True, None),
]


@pytest.mark.parametrize("pattern", ["ramp", "spikes"])
@pytest.mark.parametrize("dtype,B,H,N,d,causal,kv", RISING, ids=lambda x: str(x))
def test_rising_scores_move_the_running_max(pattern, dtype, B, H, N, d, causal, kv):
    require_gpu()
    seed = 3000 + N + d
    announce(f"rising-{pattern} dtype={dtype} B={B} H={H} N={N} d={d} causal={causal} kv={kv} seed={seed}")
    inp = make_inputs(B, H, N, d, dtype, seed, kv_len=kv)
    scale = 1.0 / math.sqrt(d)
    a = 4.0
    unit = 1.0 / (scale * math.log2(math.e) * a * d)  # key lift per log2 unit of scaled score
    if pattern == "ramp":
        lift = 0.35 if N <= 1024 else 0.06
        c = lift * unit * torch.arange(N, dtype=torch.float32)
    else:
        g = torch.Generator("cpu").manual_seed(seed)
        c = (torch.rand(N, generator=g) < 0.1).float() * (12.0 * unit)
    q = inp["q"].float() + a
    k = inp["k"].float() + c[:, None]
    inp["q"], inp["k"] = q.to(inp["v"].dtype), k.to(inp["v"].dtype)
    res = run_gpu(to_dev(inp), causal, scale)
    heads = [(b, h) for b in range(B) for h in range(H)]
    ref = oracle_ref(inp, causal, scale, heads)
    # O, L and D to the usual bounds.  The gradients also carry, to first order, errors that these
    # peaked weights make larger than the plain bound allows: P and dS enter the products rounded
    # to bf16 (2^-9 relative each), P is recomputed from L, whose row sum adds up the rounded
    # weights (up to 2^-9 relative in P), and D is formed from the stored, rounded O (|dD_i| <=
    # D_slack_i).  With eps = 2^-8 that gives |dV_j - ref| <= eps sum_i P_ij |dO_i| and, through
    # |d dS_ij| <= eps P_ij |dP_ij - D_i| + P_ij dD_i, the dQ and dK terms below -- a bound a
    # wrong term or index would exceed by far.  float32 runs keep the plain bound.
    for key in ("O", "L", "D"):
        check_close(key, heads_to_numpy(res[key], heads), ref[key], dtype,
                    ref["D_slack"] if key == "D" else 0.0)
    qn, kn = inp["q"].double().numpy(), inp["k"].double().numpy()
    vn, don = inp["v"].double().numpy(), inp["do"].double().numpy()
    sl = {key: np.zeros(qn.shape) for key in ("dQ", "dK", "dV")}
    kvl = None if kv is None else list(kv)
    if dtype == "bf16":
        eps = 2.0 ** -8
        for b, h in heads:
            S = scale * qn[b, h] @ kn[b, h].T
            i, j = np.indices(S.shape)
            valid = np.ones(S.shape, dtype=bool)
            if causal:
                valid &= j <= i
            if kvl is not None:
                valid &= j < kvl[b]
            P = np.where(valid, np.exp(np.where(valid, S, 0.0) - ref["L"][b, h][:, None]), 0.0)
            dP = don[b, h] @ vn[b, h].T
            dds = eps * P * np.abs(dP - ref["D"][b, h][:, None]) + P * ref["D_slack"][b, h][:, None]
            sl["dV"][b, h] = eps * (P.T @ np.abs(don[b, h]))
            sl["dQ"][b, h] = scale * (dds @ np.abs(kn[b, h]))
            sl["dK"][b, h] = scale * (dds.T @ np.abs(qn[b, h]))
    for key in ("dQ", "dK", "dV"):
        check_close(key, heads_to_numpy(res[key], heads), ref[key], dtype, sl[key])
