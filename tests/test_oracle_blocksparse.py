"""Pins for the oracle's block-sparse masking ("Notes on flashattention", section Block-sparse
Flashattention): a mask constant on ``block x block`` tiles restricts which keys each query sees.

Each pin ``bpin_*(impl)`` checks a fact that holds independently of the oracle: an all-ones mask
is dense attention; a block-diagonal mask is independent attention per diagonal segment; a zero
column block is attention over the remaining keys (and zero gradient for the dropped ones); scalar
Python loops on tiny inputs, including rows left with no key (O = 0, L = -inf); central finite
differences of the gradients.  Planted mistakes in the block expansion or the empty-row rule must
each fail at least one pin.
"""

from __future__ import annotations

import math
import types

import numpy as np
import pytest

import oracle.attention as O


def _rng(seed):
    return np.random.default_rng(seed)


def _dense(impl, q, k, v, do, *, causal, scale, kv=None):
    o, l, _ = impl.head_forward(q, k, v, causal=causal, scale=scale, kv=kv)
    g = impl.head_backward(q, k, v, do, causal=causal, scale=scale, kv=kv)
    return o, l, g


def bpin_all_ones_is_dense(impl):
    r = _rng(40)
    n, d, blk = 13, 3, 4
    q, k, v, do = r.normal(size=(4, n, d))
    ones = np.ones((4, 4), dtype=np.uint8)
    for causal, kv in ((True, None), (False, None), (True, 9), (False, 5)):
        o, l, _ = impl.head_forward(q, k, v, causal=causal, scale=0.7, kv=kv, block_mask=ones, block=blk)
        g = impl.head_backward(q, k, v, do, causal=causal, scale=0.7, kv=kv, block_mask=ones, block=blk)
        od, ld, gd = _dense(O, q, k, v, do, causal=causal, scale=0.7, kv=kv)
        np.testing.assert_allclose(o, od, atol=1e-13)
        np.testing.assert_allclose(l, ld, atol=1e-13)
        for a, b in zip(g[:3], gd[:3]):
            np.testing.assert_allclose(a, b, atol=1e-13)


def bpin_block_diagonal_is_segments(impl):
    """A block-diagonal mask splits the sequence into independent segments."""
    r = _rng(41)
    blk, seg_blocks, n, d = 3, 2, 14, 2  # segments [0, 6), [6, 12), [12, 14)
    tb = -(-n // blk)
    bm = np.zeros((tb, tb), dtype=np.uint8)
    for a in range(tb):
        for b in range(tb):
            bm[a, b] = a // seg_blocks == b // seg_blocks
    q, k, v, do = r.normal(size=(4, n, d))
    for causal in (False, True):
        o, l, _ = impl.head_forward(q, k, v, causal=causal, scale=1.1, block_mask=bm, block=blk)
        dq, dk, dv, _ = impl.head_backward(q, k, v, do, causal=causal, scale=1.1, block_mask=bm, block=blk)
        for s0 in range(0, n, blk * seg_blocks):
            sl = slice(s0, min(n, s0 + blk * seg_blocks))
            os_, ls_, (gq, gk, gv, _) = _dense(O, q[sl], k[sl], v[sl], do[sl], causal=causal, scale=1.1)
            np.testing.assert_allclose(o[sl], os_, atol=1e-13)
            np.testing.assert_allclose(l[sl], ls_, atol=1e-13)
            np.testing.assert_allclose(dq[sl], gq, atol=1e-12)
            np.testing.assert_allclose(dk[sl], gk, atol=1e-12)
            np.testing.assert_allclose(dv[sl], gv, atol=1e-12)


def bpin_dropped_key_block(impl):
    """A zero column block removes those keys: attention over the rest, zero gradient for them."""
    r = _rng(42)
    blk, n, d = 4, 16, 3
    tb = n // blk
    q, k, v, do = r.normal(size=(4, n, d))
    for c in (0, 2):
        bm = np.ones((tb, tb), dtype=np.uint8)
        bm[:, c] = 0
        bm[1, 3] = 0 if c != 3 else 1  # one more hole, not symmetric, in row block 1 only
        o, l, _ = impl.head_forward(q, k, v, causal=False, scale=0.8, block_mask=bm, block=blk)
        dq, dk, dv, _ = impl.head_backward(q, k, v, do, causal=False, scale=0.8, block_mask=bm, block=blk)
        keep = np.array([j for j in range(n) if j // blk != c])
        dropped = np.array([j for j in range(n) if j // blk == c])
        for rb in range(tb):
            rows = slice(rb * blk, (rb + 1) * blk)
            kk = np.array([j for j in keep if bm[rb, j // blk]])
            s = 0.8 * q[rows] @ k[kk].T
            p = np.exp(s - s.max(1, keepdims=True))
            lse = s.max(1) + np.log(p.sum(1))
            p /= p.sum(1, keepdims=True)
            np.testing.assert_allclose(o[rows], p @ v[kk], atol=1e-13)
            np.testing.assert_allclose(l[rows], lse, atol=1e-13)
        np.testing.assert_array_equal(dk[dropped], 0.0)
        np.testing.assert_array_equal(dv[dropped], 0.0)


def _brute(q, k, v, causal, scale, kv, bm, blk):
    """Scalar loops: visible keys of each query from the causal, padding and block rules."""
    n = len(q)
    outs, lses = [], []
    for i in range(n):
        keys = [j for j in range(n)
                if (not causal or j <= i) and (kv is None or j < kv) and bm[i // blk][j // blk]]
        if not keys:
            outs.append([0.0] * len(v[0]))
            lses.append(-math.inf)
            continue
        w = [math.exp(scale * sum(a * b for a, b in zip(q[i], k[j]))) for j in keys]
        tot = sum(w)
        outs.append([sum(wj * v[j][c] for wj, j in zip(w, keys)) / tot for c in range(len(v[0]))])
        lses.append(math.log(tot))
    return np.array(outs), np.array(lses)


def bpin_brute_force(impl):
    r = _rng(43)
    for n, blk, causal, kv in ((6, 2, False, None), (7, 2, True, None), (9, 3, True, 8), (5, 1, False, 4)):
        tb = -(-n // blk)
        bm = (r.random((tb, tb)) < 0.55).astype(np.uint8)
        bm[0, :] = 0  # row block 0 sees nothing
        bm[tb - 1, 0] = 1
        q, k, v = r.normal(size=(3, n, 2))
        o, l, _ = impl.head_forward(q, k, v, causal=causal, scale=0.9, kv=kv, block_mask=bm, block=blk)
        ob, lb = _brute(q.tolist(), k.tolist(), v.tolist(), causal, 0.9, kv, bm.tolist(), blk)
        np.testing.assert_allclose(o, ob, atol=1e-13)
        assert np.array_equal(np.isinf(l), np.isinf(lb))
        fin = np.isfinite(lb)
        np.testing.assert_allclose(l[fin], lb[fin], atol=1e-13)


def bpin_finite_differences(impl):
    """Central differences of f = sum(O o dO) match the analytic gradients under a block mask."""
    r = _rng(44)
    n, d, blk = 6, 3, 2
    bm = np.array([[1, 0, 0], [1, 1, 0], [0, 1, 1]], dtype=np.uint8)
    q, k, v, do = r.normal(size=(4, n, d))
    for causal in (False, True):
        dq, dk, dv, _ = impl.head_backward(q, k, v, do, causal=causal, scale=0.6, block_mask=bm, block=blk)

        def f(qq, kk, vv):
            o, _, _ = impl.head_forward(qq, kk, vv, causal=causal, scale=0.6, block_mask=bm, block=blk)
            return float((o * do).sum())

        h = 1e-6
        for which, grad in ((0, dq), (1, dk), (2, dv)):
            num = np.zeros_like(grad)
            for idx in np.ndindex(grad.shape):
                args_p = [q.copy(), k.copy(), v.copy()]
                args_m = [q.copy(), k.copy(), v.copy()]
                args_p[which][idx] += h
                args_m[which][idx] -= h
                num[idx] = (f(*args_p) - f(*args_m)) / (2 * h)
            np.testing.assert_allclose(grad, num, rtol=0, atol=1e-7 * max(1.0, np.abs(num).max()))


BPINS = [bpin_all_ones_is_dense, bpin_block_diagonal_is_segments, bpin_dropped_key_block, bpin_brute_force,
         bpin_finite_differences]


@pytest.mark.parametrize("pin", BPINS, ids=lambda p: p.__name__)
def test_blocksparse_pin(pin):
    pin(O)


def test_block_mask_shape_checked():
    q, k, v = _rng(45).normal(size=(3, 10, 2))
    with pytest.raises(ValueError):
        O.head_forward(q, k, v, causal=True, scale=1.0, block_mask=np.ones((2, 2)), block=4)  # needs 3 x 3


# --------------------------------------------------------------------------------------------
# planted mistakes in the block-sparse rule


def _bsp_variant(kind):
    def mask(n, causal, kv, bm, blk):
        i = np.arange(n)[:, None]
        j = np.arange(n)[None, :]
        ok = np.ones((n, n), dtype=bool)
        if causal:
            ok &= j <= i
        if kv is not None:
            ok &= j < kv
        bm = np.asarray(bm) != 0
        if kind == "transposed":
            ok &= bm[j // blk, i // blk]
        elif kind == "off_by_one":
            ok &= bm[np.minimum((i + 1) // blk, bm.shape[0] - 1), j // blk]
        elif kind != "score_zero":
            ok &= bm[i // blk, j // blk]
        return ok, bm[i // blk, j // blk] | np.zeros((n, n), dtype=bool)

    def fwd(q, k, v, *, causal, scale, kv=None, block_mask=None, block=64):
        if block_mask is None:
            return O.head_forward(q, k, v, causal=causal, scale=scale, kv=kv)
        q, k, v = (np.asarray(x, dtype=np.float64) for x in (q, k, v))
        n = q.shape[0]
        ok, inblock = mask(n, causal, kv, block_mask, block)
        s = scale * (q @ k.T)
        if kind == "score_zero":  # the literal reading: masked-out blocks keep score 0, not weight 0
            s = np.where(inblock, s, 0.0)
        live = ok.any(1)
        m = np.where(live, np.where(ok, s, -np.inf).max(1), 0.0)
        e = np.where(ok, np.exp(np.where(ok, s, 0.0) - m[:, None]), 0.0)
        den = e.sum(1)
        if kind == "empty_row_nan":
            p = e / den[:, None]
            lse = m + np.log(den)
        else:
            p = e / np.where(live, den, 1.0)[:, None]
            lse = np.where(live, m + np.log(np.where(live, den, 1.0)), -np.inf)
        return p @ v, lse, p

    def bwd(q, k, v, do, *, causal, scale, kv=None, block_mask=None, block=64):
        q, k, v, do = (np.asarray(x, dtype=np.float64) for x in (q, k, v, do))
        _, _, p = fwd(q, k, v, causal=causal, scale=scale, kv=kv, block_mask=block_mask, block=block)
        dv = p.T @ do
        dp = do @ v.T
        dref = (p * dp).sum(1)
        ds = p * dp - p * dref[:, None]
        return scale * (ds @ k), scale * (ds.T @ q), dv, dref

    return types.SimpleNamespace(head_forward=fwd, head_backward=bwd)


BSP_MUTANTS = {k: _bsp_variant(k) for k in ("transposed", "off_by_one", "score_zero", "empty_row_nan")}


@pytest.mark.parametrize("name", sorted(BSP_MUTANTS))
def test_planted_blocksparse_mistake_is_caught(name):
    failed = []
    with np.errstate(all="ignore"):
        for pin in BPINS:
            try:
                pin(BSP_MUTANTS[name])
            except (AssertionError, ValueError, IndexError, FloatingPointError):
                failed.append(pin.__name__)
    assert failed, f"planted mistake {name!r} passed every block-sparse pin"


def test_correct_variant_passes_blocksparse_pins():
    good = _bsp_variant("none")
    for pin in BPINS:
        pin(good)
