"""Systematic-bias check of the bfloat16 path against the oracle.

The elementwise bf16 tolerance (2e-2 + 1e-2 |ref|) would let a consistent scale error of a few
tenths of a percent through -- the size of the error that rounding P or dS toward zero without
compensation leaves in O, dQ, dK and dV.  Here each output X is fitted as X_gpu ~ (1 + b) X_ref
by least squares, b = sum((X_gpu - X_ref) X_ref) / sum(X_ref^2), over every element of a few
hundred thousand; random rounding errors average out of b (they leave |b| ~ 1e-5 at these
sizes), a scale bias does not.  The bound 5e-4 is a sixth of the uncompensated truncation bias
(2^-8 / (2 ln 2) = 2.8e-3).
"""

import math

import numpy as np
import pytest

from causal_self_attention_flashattention_amd.inputs import make_inputs

from attn_testutil import announce, oracle_ref, require_gpu, run_gpu, to_dev

pytestmark = pytest.mark.gpu

BIAS_BOUND = 5e-4


def scale_bias(gpu, ref) -> float:
    g = gpu.double().cpu().numpy() if hasattr(gpu, "detach") else np.asarray(gpu, dtype=np.float64)
    return float(((g - ref) * ref).sum() / (ref * ref).sum())


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal,N", [(True, 700), (False, 513)])
def test_bf16_outputs_carry_no_scale_bias(d, causal, N):
    require_gpu()
    B, H = 1, 8
    announce(f"scale-bias bf16 B={B} H={H} N={N} d={d} causal={causal}")
    inp = make_inputs(B, H, N, d, "bf16", seed=101 + d + N)
    scale = 1.0 / math.sqrt(d)
    got = run_gpu(to_dev(inp), causal, scale)
    ref = oracle_ref(inp, causal, scale)
    for name in ("O", "dQ", "dK", "dV"):
        b = scale_bias(got[name], ref[name])
        assert abs(b) <= BIAS_BOUND, f"{name}: fitted scale bias {b:.2e}"
    # L = m + ln(sum_j exp(S_ij - m)): a bias in the row sums shows up as an offset.
    off = float((got["L"].double().cpu().numpy() - ref["L"]).mean())
    assert abs(off) <= BIAS_BOUND, f"L: mean offset {off:.2e}"
