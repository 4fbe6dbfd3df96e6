"""attn_bwd_noalloc (the backward for callers that cannot allocate: the split partials go to the
library's static scratch) against attn_bwd_ex with a caller workspace, through the C ABI.

Two calls in a row, the second on a smaller input, so the second runs on scratch that still holds
the first call's partials; every output must equal attn_bwd_ex's bit for bit (same kernels, same
split, same summation order), and the first call is also checked against the oracle."""

import math

import pytest
import torch

import causal_self_attention_flashattention_amd as attn
from causal_self_attention_flashattention_amd.inputs import make_inputs

from attn_testutil import announce, compare_all, oracle_ref, require_gpu, to_dev

pytestmark = pytest.mark.gpu

# (B, H, N, d, causal, kv): the first needs 32 MiB of split partials, the second 16 MiB
CASES = [(1, 1, 4096, 64, True, None), (1, 2, 2048, 64, False, [1900])]


def _run_pair(B, H, N, d, causal, kv, seed):
    inp = make_inputs(B, H, N, d, "bf16", seed, kv_len=kv)
    dev = to_dev(inp)
    scale = 1.0 / math.sqrt(d)
    need = attn.bwd_workspace_bytes(B, H, N, d, torch.bfloat16)
    assert 0 < need <= attn.binding.NOALLOC_SCRATCH_BYTES, "case must take the split path within the scratch"
    o, L = attn.fwd(dev["q"], dev["k"], dev["v"], causal=causal, scale=scale, kv_len=dev["kv_len"])
    ref = attn.bwd(dev["q"], dev["k"], dev["v"], o, dev["do"], L, causal=causal, scale=scale,
                   kv_len=dev["kv_len"], workspace="auto")
    outs = tuple(torch.full_like(t, float("nan")) for t in ref)
    got = attn.bwd_noalloc(dev["q"], dev["k"], dev["v"], o, dev["do"], L, outs, causal=causal, scale=scale,
                           kv_len=dev["kv_len"])
    torch.cuda.synchronize()
    for name, a, b in zip(("dQ", "dK", "dV", "D"), got, ref):
        assert torch.equal(a, b), f"{name}: attn_bwd_noalloc differs from attn_bwd_ex"
    return inp, {"O": o, "L": L, "dQ": got[0], "dK": got[1], "dV": got[2], "D": got[3]}, causal, scale


def test_noalloc_matches_workspace_backward_twice():
    require_gpu()
    for i, (B, H, N, d, causal, kv) in enumerate(CASES):
        announce(f"noalloc call {i + 1}: B={B} H={H} N={N} d={d} causal={causal} kv={kv}")
        inp, res, causal, scale = _run_pair(B, H, N, d, causal, kv, 500 + i)
        if i == 0:
            heads = [(0, 0)]
            compare_all(res, oracle_ref(inp, causal, scale, heads), "bf16", heads)


# d = 80: the split partials carry the 16-wide accumulators of the last 16 columns
CASES80 = [(1, 2, 2048, 80, True, [1900]), (1, 1, 2048, 80, False, None)]


def test_noalloc_matches_workspace_backward_d80():
    require_gpu()
    for i, (B, H, N, d, causal, kv) in enumerate(CASES80):
        announce(f"noalloc d=80 call {i + 1}: B={B} H={H} N={N} d={d} causal={causal} kv={kv}")
        inp, res, causal, scale = _run_pair(B, H, N, d, causal, kv, 700 + i)
        if i == 0:
            heads = [(0, 1)]
            compare_all(res, oracle_ref(inp, causal, scale, heads), "bf16", heads)


def test_noalloc_rejects_beyond_scratch():
    require_gpu()
    B, H, N, d = 1, 1, 16384, 128
    assert attn.bwd_workspace_bytes(B, H, N, d, torch.bfloat16) > attn.binding.NOALLOC_SCRATCH_BYTES
    t = torch.zeros(B, H, N, d, dtype=torch.bfloat16, device="cuda")
    L = torch.zeros(B, H, N, dtype=torch.float32, device="cuda")
    outs = (torch.empty_like(t), torch.empty_like(t), torch.empty_like(t), torch.empty_like(L))
    with pytest.raises(attn.AttnError) as e:
        attn.bwd_noalloc(t, t.clone(), t.clone(), t.clone(), t.clone(), L, outs)
    assert e.value.status == -9
