"""Block-sparse attention ("Notes on flashattention", section Block-sparse Flashattention) on the
GPU against the float64 oracle: random 64 x 64 block masks (with a query block left without any
key, which must give O = 0, L = -inf and dQ = 0) combined with the causal and key-padding masks,
every head dim, both dtypes, and each backward launch layout; an all-ones mask must reproduce the
dense kernels bit for bit."""

import math

import numpy as np
import pytest
import torch

import oracle.attention as ref
from causal_self_attention_flashattention_amd import binding as attn
from causal_self_attention_flashattention_amd.inputs import make_inputs

from attn_testutil import d_slack

pytestmark = pytest.mark.gpu


def _mask(N, density, seed, empty_row=True):
    tb = attn.mask_blocks(N)
    r = np.random.default_rng(seed)
    m = (r.random((tb, tb)) < density).astype(np.uint8)
    np.fill_diagonal(m, 1)
    if empty_row and tb > 2:
        m[1, :] = 0  # query block 1 sees no key at all
    return m


def _close(name, got, want, dtype, slack=0.0):
    a, r = (1e-4, 0.0) if dtype == "f32" else (2e-2, 1e-2)
    slack = np.broadcast_to(slack, want.shape)[~np.isinf(want)]
    got = got.detach().double().cpu().numpy()
    inf = np.isinf(want)
    assert np.array_equal(np.isinf(got), inf), f"{name}: -inf pattern differs"
    got, want = got[~inf], want[~inf]
    err = np.abs(got - want)
    bound = a + r * np.abs(want) + slack
    assert np.all(err <= bound), f"{name}: max err {err.max():.3g}, worst ratio {(err / bound).max():.3g}"


CASES = [
    # B, H, N, d, dtype, causal, kv_len, density, heads checked (None = all)
    (1, 2, 300, 64, "bf16", True, None, 0.5, None),
    (2, 1, 257, 128, "bf16", False, [200, 257], 0.4, None),
    (1, 2, 200, 80, "f32", True, None, 0.6, None),
    (2, 2, 130, 16, "f32", False, None, 0.5, None),
    (1, 1, 640, 32, "bf16", True, [600], 0.3, None),
    (1, 2, 512, 64, "bf16", True, None, 0.4, None),               # one merged backward launch
    (2, 20, 1024, 64, "bf16", True, None, 0.3, [(0, 0), (1, 19)]),  # dQ then dK/dV launches
    (1, 128, 1024, 128, "bf16", True, None, 0.3, [(0, 5), (0, 127)]),  # 8-wave dK/dV tiles
    (1, 2, 2048, 80, "bf16", False, [1900], 0.25, None),
    (2, 2, 300, 16, "bf16", True, [280, 300], 0.4, None),         # all of d = 16 on 16-wide products
]


@pytest.mark.parametrize("B,H,N,d,dtype,causal,kv,density,heads", CASES)
def test_blocksparse_matches_oracle(B, H, N, d, dtype, causal, kv, density, heads):
    inp = make_inputs(B, H, N, d, dtype, seed=N + d, kv_len=kv)
    q, k, v, do = (inp[n].cuda() for n in ("q", "k", "v", "do"))
    kvd = None if inp["kv_len"] is None else inp["kv_len"].cuda()
    bm = _mask(N, density, seed=N)
    scale = 1.0 / math.sqrt(d)
    o, L = attn.fwd(q, k, v, causal=causal, scale=scale, kv_len=kvd, block_mask=bm)
    dq, dk, dv, D = attn.bwd(q, k, v, o, do, L, causal=causal, scale=scale, kv_len=kvd, block_mask=bm)
    torch.cuda.synchronize()
    kw = dict(causal=causal, scale=scale, kv_len=kv, heads=heads, block_mask=bm, block=64)
    ro, rl = ref.attention_forward(inp["q"], inp["k"], inp["v"], **kw)
    rq, rk, rv, rd = ref.attention_backward(inp["q"], inp["k"], inp["v"], inp["do"], **kw)
    sel = heads or [(b, h) for b in range(B) for h in range(H)]
    for b, h in sel:
        tag = f"(b={b}, h={h})"
        _close("O" + tag, o[b, h], ro[b, h], dtype)
        _close("L" + tag, L[b, h], rl[b, h], dtype)
        _close("dQ" + tag, dq[b, h], rq[b, h], dtype)
        _close("dK" + tag, dk[b, h], rk[b, h], dtype)
        _close("dV" + tag, dv[b, h], rv[b, h], dtype)
        _close("D" + tag, D[b, h], rd[b, h], dtype, d_slack(ro[b, h], inp["do"][b, h], dtype))
    if N > 128:  # the empty query block: exact zeros and -inf
        assert torch.all(o[:, :, 64:128] == 0) and torch.all(dq[:, :, 64:128] == 0)
        assert torch.all(torch.isneginf(L[:, :, 64:128]))


# Shapes whose dense kernels run the same tiling as the block-sparse ones: one key or query group
# per workgroup (small bf16 grids use two for dense masks, which add the two halves of every sum in
# another order).
@pytest.mark.parametrize("N,d,dtype,causal,BH", [(300, 64, "bf16", True, 100), (257, 128, "f32", False, 2),
                                                  (1024, 64, "bf16", True, 40), (1024, 128, "bf16", True, 128),
                                                  (1024, 128, "bf16", False, 64), (1024, 80, "bf16", True, 64)])
def test_all_ones_mask_equals_dense_bitwise(N, d, dtype, causal, BH):
    inp = make_inputs(1, BH, N, d, dtype, seed=3)
    q, k, v, do = (inp[n].cuda() for n in ("q", "k", "v", "do"))
    ones = np.ones((attn.mask_blocks(N),) * 2, dtype=np.uint8)
    o1, l1 = attn.fwd(q, k, v, causal=causal)
    o2, l2 = attn.fwd(q, k, v, causal=causal, block_mask=ones)
    g1 = attn.bwd(q, k, v, o1, do, l1, causal=causal)
    g2 = attn.bwd(q, k, v, o2, do, l2, causal=causal, block_mask=ones)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    for a, b in zip(g1, g2):
        assert torch.equal(a, b)


def test_blocksparse_rejects_bad_mask_shape_and_long_sequences():
    inp = make_inputs(1, 1, 100, 32, "bf16", seed=1)
    q, k, v = (inp[n].cuda() for n in ("q", "k", "v"))
    with pytest.raises(ValueError):
        attn.fwd(q, k, v, block_mask=np.ones((3, 3)))
    big = torch.zeros((1, 1, 65600, 16), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(attn.AttnError):
        attn.fwd(big, big, big, block_mask=np.ones((attn.mask_blocks(65600),) * 2))
