"""The drop-in autograd function (CS336 Assignment 2, §4.2.2 Problems (flash_forward) and
(flash_backward)) against the float64 oracle: gradients through ``loss.backward()`` for the
hand-out's [batch, N, d] layout and for [B, H, N, d], and parameter gradients of a small
Transformer (the end-to-end model of §2.1.3) whose attention is either the HIP kernels on the GPU
or the oracle on the CPU."""

import math

import numpy as np
import pytest
import torch

import oracle.attention as ref
from causal_self_attention_flashattention_amd.e2e import TransformerLM
from causal_self_attention_flashattention_amd.function import FlashAttention, flash_attention
from causal_self_attention_flashattention_amd.inputs import make_inputs

pytestmark = pytest.mark.gpu


def _tol(dtype):
    return (1e-4, 0.0) if dtype == "f32" else (2e-2, 1e-2)


def _check(name, got, want, dtype):
    a, r = _tol(dtype)
    got = got.detach().double().cpu().numpy()
    err = np.abs(got - want)
    bound = a + r * np.abs(want)
    assert np.all(err <= bound), f"{name}: max err {err.max():.3g}, worst ratio {(err / bound).max():.3g}"


@pytest.mark.parametrize("layout,B,H,N,d,dtype,causal,kv", [
    ("3d", 3, 1, 200, 64, "bf16", True, None),
    ("4d", 2, 3, 130, 80, "f32", False, None),
    ("4d", 2, 2, 257, 128, "bf16", True, [200, 257]),
    ("3d", 2, 1, 96, 16, "f32", True, [90, 40]),
])
def test_autograd_matches_oracle(layout, B, H, N, d, dtype, causal, kv):
    inp = make_inputs(B, H, N, d, dtype, seed=21 + N, kv_len=kv)
    scale = 1.0 / math.sqrt(d)
    q, k, v, do = (inp[n].cuda() for n in ("q", "k", "v", "do"))
    if layout == "3d":
        q, k, v, do = (t.reshape(B * H, N, d) for t in (q, k, v, do))
    q, k, v = (t.clone().requires_grad_(True) for t in (q, k, v))
    o = flash_attention(q, k, v, is_causal=causal, scale=scale, kv_len=kv)
    assert o.shape == q.shape and o.dtype == q.dtype
    (o.float() * do.float()).sum().backward()
    ro, _ = ref.attention_forward(inp["q"], inp["k"], inp["v"], causal=causal, scale=scale, kv_len=kv)
    rq, rk, rv, _ = ref.attention_backward(inp["q"], inp["k"], inp["v"], inp["do"], causal=causal, scale=scale,
                                           kv_len=kv)
    shape = (B, H, N, d)
    _check("O", o.reshape(shape), ro, dtype)
    _check("dQ", q.grad.reshape(shape), rq, dtype)
    _check("dK", k.grad.reshape(shape), rk, dtype)
    _check("dV", v.grad.reshape(shape), rv, dtype)


def test_saved_tensors_hold_logsumexp():
    # The hand-out's forward saves L (with Q, K, V, O) for the backward.
    inp = make_inputs(1, 2, 64, 32, "f32", seed=5)
    q, k, v = (inp[n].cuda().requires_grad_(True) for n in ("q", "k", "v"))
    o = FlashAttention.apply(q, k, v, True)
    saved = o.grad_fn.saved_tensors
    L = saved[4]
    _, rl = ref.attention_forward(inp["q"], inp["k"], inp["v"], causal=True, scale=1 / math.sqrt(32))
    assert L.shape == (1, 2, 64) and L.dtype == torch.float32
    assert np.abs(L.cpu().numpy() - rl).max() <= 1e-4


class _OracleAttention(torch.autograd.Function):
    """Causal attention on the CPU by the float64 oracle (forward eq. 1, backward eqs. 7-11)."""

    @staticmethod
    def forward(ctx, q, k, v, scale):
        ctx.save_for_backward(q, k, v)
        ctx.scale = scale
        o, _ = ref.attention_forward(q.detach(), k.detach(), v.detach(), causal=True, scale=scale)
        return torch.from_numpy(o)

    @staticmethod
    def backward(ctx, do):
        q, k, v = ctx.saved_tensors
        dq, dk, dv, _ = ref.attention_backward(q.detach(), k.detach(), v.detach(), do.detach(), causal=True,
                                               scale=ctx.scale)
        return torch.from_numpy(dq), torch.from_numpy(dk), torch.from_numpy(dv), None


def test_model_gradients_match_oracle_model():
    # Same weights and tokens; float32 model with the HIP attention on the GPU against a float64
    # model with the oracle's attention on the CPU.  Everything but the attention is the same torch
    # code, so the parameter gradients differ only by float32 rounding.
    torch.manual_seed(3)
    vocab, d_model, d_ff, layers, heads, n, batch = 64, 64, 128, 2, 2, 100, 2
    gpu = TransformerLM(vocab, d_model, d_ff, layers, heads, "flash").cuda()
    cpu = TransformerLM(vocab, d_model, d_ff, layers, heads, lambda q, k, v, s: _OracleAttention.apply(q, k, v, s))
    cpu.load_state_dict({k: v.detach().cpu() for k, v in gpu.state_dict().items()})
    cpu = cpu.double()
    g = torch.Generator().manual_seed(9)
    x = torch.randint(0, vocab, (batch, n), generator=g)
    y = torch.randint(0, vocab, (batch, n), generator=g)
    lg = torch.nn.functional.cross_entropy(gpu(x.cuda()).view(-1, vocab), y.cuda().view(-1))
    lc = torch.nn.functional.cross_entropy(cpu(x).view(-1, vocab), y.view(-1))
    lg.backward()
    lc.backward()
    assert abs(lg.item() - lc.item()) <= 1e-4 * abs(lc.item())
    worst = 0.0
    for (name, pg), (_, pc) in zip(gpu.named_parameters(), cpu.named_parameters()):
        a, b = pg.grad.double().cpu(), pc.grad
        err = (a - b).abs().max().item()
        scale = b.abs().max().item() + 1e-12
        worst = max(worst, err / scale)
        assert err <= 1e-3 * scale, f"{name}: max err {err:.3g} vs max |grad| {scale:.3g}"
    assert worst < 1e-3
