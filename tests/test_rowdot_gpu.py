"""GPU parity of the stand-alone D pass (attn_bwd_rowdot): D_i = sum_c O_ic dO_ic ([A2] §4.2.2, the
D vector of the backward pass with recomputation) against the oracle's rowsum_o_do on the same
seeded O and dO, for every head dim and both dtypes, with row counts that leave a partial last
block of rows, and with guard bands around D.  D is defined for any O, so O here is a seeded
random tensor rather than a forward output."""

import numpy as np
import pytest
import torch

import causal_self_attention_flashattention_amd as attn
import oracle.attention as O
from causal_self_attention_flashattention_amd.inputs import make_inputs

from attn_testutil import announce, require_gpu

pytestmark = pytest.mark.gpu

CASES = [(dt, d, H, N) for dt in ("bf16", "f32") for d in (16, 32, 64, 80, 128) for (H, N) in ((3, 173), (1, 5))]


@pytest.mark.parametrize("dtype,d,H,N", CASES, ids=lambda x: str(x))
def test_rowdot_matches_oracle(dtype, d, H, N):
    require_gpu()
    B = 2
    seed = 4000 + d + N
    announce(f"rowdot dtype={dtype} B={B} H={H} N={N} d={d} seed={seed}")
    inp = make_inputs(B, H, N, d, dtype, seed)
    o, do = inp["v"], inp["do"]
    pad = 1024
    buf = torch.full((B * H * N + 2 * pad,), 12345.0, dtype=torch.float32, device="cuda")
    D = buf[pad: pad + B * H * N].view(B, H, N)
    attn.rowdot(o.cuda(), do.cuda(), out=D)
    torch.cuda.synchronize()
    assert torch.all(buf[:pad] == 12345.0) and torch.all(buf[pad + B * H * N:] == 12345.0), "wrote outside D"
    ref = O.rowsum_o_do(o, do)
    got = D.double().cpu().numpy()
    # a chain of d float32 fused multiply-adds (bf16 products are exact in float32) errs by at most
    # about d units of 2^-24 of the sum of the terms' magnitudes
    mag = np.abs(O._f64(o) * O._f64(do)).sum(-1)
    bound = d * 2.0 ** -24 * mag + 1e-7
    err = np.abs(got - ref)
    assert np.all(err <= bound), f"max err {err.max():.3g} (bound {float(bound.max()):.3g})"
