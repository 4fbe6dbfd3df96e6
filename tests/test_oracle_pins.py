"""Pins for the CPU oracle: facts fixed by the pages and by mathematics, not by the oracle itself.

Each pin is a function ``pin_*(impl) -> None`` that raises AssertionError when ``impl`` (an
object with ``head_forward`` / ``head_backward`` like ``oracle.attention``) breaks the fact.
The real oracle must pass every pin; each planted mistake in ``MUTANTS`` (a dropped term, a
wrong sign or index, a transposed operand, a misplaced scale, an off-by-one mask) must fail
at least one of them, which shows the pins would catch that mistake in the oracle.
"""

from __future__ import annotations

import json
import math
import os
import types

import numpy as np
import pytest

import oracle.attention as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_example_n2_d1.json")


def _rng(seed):
    return np.random.default_rng(seed)


# --------------------------------------------------------------------------------------------
# pins


def pin_golden_hand_example(impl):
    """Closed-form 2x1 example derived from eqs. (1), (4)-(12) of the handout (tests/golden)."""
    g = json.load(open(GOLDEN))
    inp = g["inputs"]
    q, k, v, do = (np.array(inp[n], dtype=np.float64) for n in ("q", "k", "v", "do"))
    for name, c in g["cases"].items():
        o, lse, _ = impl.head_forward(q, k, v, causal=c["causal"], scale=inp["scale"], kv=c["kv"])
        dq, dk, dv, dref = impl.head_backward(q, k, v, do, causal=c["causal"], scale=inp["scale"], kv=c["kv"])
        for got, key in ((o, "O"), (lse, "L"), (dref, "D"), (dq, "dQ"), (dk, "dK"), (dv, "dV")):
            np.testing.assert_allclose(got, np.array(c[key]), rtol=0, atol=1e-14, err_msg=f"{name}:{key}")


def pin_rows_sum_to_one(impl):
    """Softmax rows sum to 1 and masked entries get weight exactly 0 (eq. (5) + the mask)."""
    r = _rng(1)
    n, d = 37, 8
    q, k, v = r.normal(size=(3, n, d))
    for causal in (False, True):
        for kv in (None, 29):
            _, _, p = impl.head_forward(q, k, v, causal=causal, scale=0.3, kv=kv)
            np.testing.assert_allclose(p.sum(1), 1.0, atol=1e-12)
            ok = O.valid_mask(n, causal, kv)
            assert np.all(p[~ok] == 0.0)
            assert np.all(p[ok] > 0.0)


def pin_zero_query_prefix_mean(impl):
    """Q = 0 makes S = 0: O_i is the mean of the visible V rows and L_i = ln(#visible)."""
    r = _rng(2)
    n, d = 23, 5
    k, v = r.normal(size=(2, n, d))
    q = np.zeros((n, d))
    for causal, kv in ((True, None), (True, 17), (False, 9), (False, None)):
        o, lse, _ = impl.head_forward(q, k, v, causal=causal, scale=0.7, kv=kv)
        for i in range(n):
            hi = n if kv is None else kv
            if causal:
                hi = min(hi, i + 1)
            np.testing.assert_allclose(o[i], v[:hi].mean(0), atol=1e-13)
            np.testing.assert_allclose(lse[i], math.log(hi), atol=1e-13)


def pin_single_token(impl):
    """N = 1: P = [1], so O = V, L = scale q.k, dV = dO and dQ = dK = 0."""
    r = _rng(3)
    q, k, v, do = r.normal(size=(4, 1, 6))
    o, lse, _ = impl.head_forward(q, k, v, causal=True, scale=0.4, kv=None)
    dq, dk, dv, _ = impl.head_backward(q, k, v, do, causal=True, scale=0.4, kv=None)
    np.testing.assert_allclose(o, v, atol=1e-15)
    np.testing.assert_allclose(lse, 0.4 * (q @ k.T).ravel(), atol=1e-14)
    np.testing.assert_allclose(dv, do, atol=1e-15)
    assert np.abs(dq).max() < 1e-15 and np.abs(dk).max() < 1e-15


def pin_constant_values(impl):
    """Identical V rows c: O = c, dP_ij = dO_i.c = D_i so dS = 0, dQ = dK = 0; dV = P^T dO."""
    r = _rng(4)
    n, d = 19, 7
    q, k, do = r.normal(size=(3, n, d))
    c = r.normal(size=d)
    v = np.tile(c, (n, 1))
    o, _, p = impl.head_forward(q, k, v, causal=True, scale=0.5, kv=None)
    dq, dk, dv, _ = impl.head_backward(q, k, v, do, causal=True, scale=0.5, kv=None)
    np.testing.assert_allclose(o, v, atol=1e-13)
    assert np.abs(dq).max() < 1e-12 and np.abs(dk).max() < 1e-12
    np.testing.assert_allclose(dv, p.T @ do, atol=1e-12)


def pin_gradient_invariants(impl):
    """Shift invariance of softmax gives sum_j dK_j = 0; rows of P summing to 1 give
    sum_j dV_j = sum_i dO_i; masked keys (j >= kv) get dK_j = dV_j = 0 exactly."""
    r = _rng(5)
    n, d = 29, 6
    q, k, v, do = r.normal(size=(4, n, d))
    for causal, kv in ((True, None), (False, None), (True, 21), (False, 11)):
        dq, dk, dv, _ = impl.head_backward(q, k, v, do, causal=causal, scale=0.35, kv=kv)
        np.testing.assert_allclose(dk.sum(0), 0.0, atol=1e-12)
        np.testing.assert_allclose(dv.sum(0), do.sum(0), atol=1e-12)
        if kv is not None:
            assert np.all(dk[kv:] == 0.0) and np.all(dv[kv:] == 0.0)


def pin_key_shift(impl):
    """Adding u to every key adds scale*q_i.u to row i of S: O unchanged, L_i shifts by it."""
    r = _rng(6)
    n, d = 17, 4
    q, k, v = r.normal(size=(3, n, d))
    u = r.normal(size=d)
    for causal, kv in ((True, None), (False, 13)):
        o1, l1, _ = impl.head_forward(q, k, v, causal=causal, scale=0.6, kv=kv)
        o2, l2, _ = impl.head_forward(q, k + u, v, causal=causal, scale=0.6, kv=kv)
        np.testing.assert_allclose(o2, o1, atol=1e-12)
        np.testing.assert_allclose(l2 - l1, 0.6 * q @ u, atol=1e-12)


def pin_causality(impl):
    """Changing K_j, V_j for j > i leaves rows <= i of O and L unchanged (causal mask)."""
    r = _rng(7)
    n, d, cut = 21, 5, 9
    q, k, v = r.normal(size=(3, n, d))
    k2, v2 = k.copy(), v.copy()
    k2[cut + 1:] = r.normal(size=(n - cut - 1, d))
    v2[cut + 1:] = r.normal(size=(n - cut - 1, d))
    o1, l1, _ = impl.head_forward(q, k, v, causal=True, scale=0.5, kv=None)
    o2, l2, _ = impl.head_forward(q, k2, v2, causal=True, scale=0.5, kv=None)
    np.testing.assert_array_equal(o1[: cut + 1], o2[: cut + 1])
    np.testing.assert_array_equal(l1[: cut + 1], l2[: cut + 1])
    assert np.abs(o1[cut + 1:] - o2[cut + 1:]).max() > 1e-3


def pin_d_identity(impl):
    """Handout §4.2.2: rowsum(P o dP) = rowsum(O o dO), since P dP^T = O dO^T."""
    r = _rng(8)
    n, d = 31, 9
    q, k, v, do = r.normal(size=(4, n, d))
    for causal, kv in ((True, None), (False, 20)):
        o, _, _ = impl.head_forward(q, k, v, causal=causal, scale=0.4, kv=kv)
        *_, dref = impl.head_backward(q, k, v, do, causal=causal, scale=0.4, kv=kv)
        np.testing.assert_allclose(dref, O.rowsum_o_do(o, do), atol=1e-12)


def pin_finite_differences(impl):
    """Central differences of f = sum(O o dO) match the analytic dQ, dK, dV (relative 1e-7)."""
    r = _rng(9)
    h = 1e-6
    for n, d in ((1, 2), (3, 2), (8, 4)):
        for causal, kv in ((False, None), (True, None), (True, max(1, n - 2)), (False, max(1, n // 2))):
            q, k, v, do = r.normal(size=(4, n, d))
            dq, dk, dv, _ = impl.head_backward(q, k, v, do, causal=causal, scale=0.7, kv=kv)

            def f(q_, k_, v_):
                return float((impl.head_forward(q_, k_, v_, causal=causal, scale=0.7, kv=kv)[0] * do).sum())

            for which, grad in ((0, dq), (1, dk), (2, dv)):
                num = np.zeros_like(grad)
                for idx in np.ndindex(*grad.shape):
                    args_p = [q.copy(), k.copy(), v.copy()]
                    args_m = [q.copy(), k.copy(), v.copy()]
                    args_p[which][idx] += h
                    args_m[which][idx] -= h
                    num[idx] = (f(*args_p) - f(*args_m)) / (2 * h)
                scale_ = max(1.0, np.abs(num).max())
                np.testing.assert_allclose(grad, num, rtol=0, atol=1e-7 * scale_,
                                           err_msg=f"n={n} d={d} causal={causal} kv={kv} arg={which}")


def _brute_force_forward(q, k, v, causal, scale, kv):
    """Scalar Python loops: for each query, visible keys, exp of scores, weighted average of V."""
    n, d = len(q), len(q[0])
    outs, lses = [], []
    for i in range(n):
        keys = [j for j in range(n) if (not causal or j <= i) and (kv is None or j < kv)]
        scores = [scale * sum(q[i][c] * k[j][c] for c in range(d)) for j in keys]
        weights = [math.exp(s) for s in scores]
        tot = sum(weights)
        outs.append([sum(w * v[j][c] for w, j in zip(weights, keys)) / tot for c in range(len(v[0]))])
        lses.append(math.log(tot))
    return np.array(outs), np.array(lses)


def pin_brute_force(impl):
    """Tiny shapes against scalar Python loops straight from eq. (1) and eq. (12)."""
    r = _rng(10)
    for n, d in ((1, 1), (4, 3), (7, 2)):
        for causal, kv in ((True, None), (False, None), (True, max(1, n - 1)), (False, 1)):
            q, k, v = r.normal(size=(3, n, d))
            o, lse, _ = impl.head_forward(q, k, v, causal=causal, scale=0.9, kv=kv)
            ob, lb = _brute_force_forward(q.tolist(), k.tolist(), v.tolist(), causal, 0.9, kv)
            np.testing.assert_allclose(o, ob, atol=1e-13)
            np.testing.assert_allclose(lse, lb, atol=1e-13)


PINS = [
    pin_golden_hand_example,
    pin_rows_sum_to_one,
    pin_zero_query_prefix_mean,
    pin_single_token,
    pin_constant_values,
    pin_gradient_invariants,
    pin_key_shift,
    pin_causality,
    pin_d_identity,
    pin_finite_differences,
    pin_brute_force,
]


@pytest.mark.parametrize("pin", PINS, ids=lambda p: p.__name__)
def test_oracle_pin(pin):
    pin(O)


# --------------------------------------------------------------------------------------------
# library cross-check: torch's own attention in float64 on the CPU (an independent
# implementation of eq. (1)), forward and autograd backward.


@pytest.mark.parametrize("causal,kv", [(True, None), (False, None), (True, 40), (False, 17)])
def test_oracle_matches_torch_sdpa_float64(causal, kv):
    torch = pytest.importorskip("torch")
    g = torch.Generator().manual_seed(11)
    B, H, n, d = 2, 3, 53, 16
    q, k, v, do = (torch.randn(B, H, n, d, generator=g, dtype=torch.float64) for _ in range(4))
    scale = 0.25
    kv_len = None if kv is None else [kv] * B
    ok = torch.from_numpy(O.valid_mask(n, causal, kv))
    qq, kk, vv = (t.clone().requires_grad_(True) for t in (q, k, v))
    ref = torch.nn.functional.scaled_dot_product_attention(qq, kk, vv, attn_mask=ok, scale=scale)
    ref.backward(do)
    o, _ = O.attention_forward(q, k, v, causal=causal, scale=scale, kv_len=kv_len)
    dq, dk, dv, _ = O.attention_backward(q, k, v, do, causal=causal, scale=scale, kv_len=kv_len)
    np.testing.assert_allclose(o, ref.detach().numpy(), atol=1e-12)
    np.testing.assert_allclose(dq, qq.grad.numpy(), atol=1e-11)
    np.testing.assert_allclose(dk, kk.grad.numpy(), atol=1e-11)
    np.testing.assert_allclose(dv, vv.grad.numpy(), atol=1e-11)


def test_batched_heads_and_subset():
    """The batched wrappers equal the per-head functions; a head subset leaves NaN elsewhere."""
    r = _rng(12)
    B, H, n, d = 2, 2, 9, 3
    q, k, v, do = r.normal(size=(4, B, H, n, d))
    o, lse = O.attention_forward(q, k, v, causal=True, scale=0.5, kv_len=[9, 5])
    for b in range(B):
        for h in range(H):
            o1, l1, _ = O.head_forward(q[b, h], k[b, h], v[b, h], causal=True, scale=0.5, kv=[9, 5][b])
            np.testing.assert_array_equal(o[b, h], o1)
            np.testing.assert_array_equal(lse[b, h], l1)
    o2, _ = O.attention_forward(q, k, v, causal=True, scale=0.5, kv_len=[9, 5], heads=[(1, 0)])
    np.testing.assert_array_equal(o2[1, 0], o[1, 0])
    assert np.isnan(o2[0, 0]).all()


def test_fully_masked_row_rejected():
    r = _rng(13)
    q, k, v = r.normal(size=(3, 4, 2))
    with pytest.raises(ValueError):
        O.head_forward(q, k, v, causal=False, scale=1.0, kv=0)


# --------------------------------------------------------------------------------------------
# planted mistakes: each mutant copies the oracle with one plausible error; some pin must fail.


def _mutant(fwd=None, bwd=None):
    m = types.SimpleNamespace(head_forward=O.head_forward, head_backward=O.head_backward)
    if fwd is not None:
        m.head_forward = fwd
    if bwd is not None:
        m.head_backward = bwd
    return m


def _fwd_variant(kind):
    def fwd(q, k, v, *, causal, scale, kv=None):
        q, k, v = (np.asarray(x, dtype=np.float64) for x in (q, k, v))
        n = q.shape[0]
        i = np.arange(n)[:, None]
        j = np.arange(n)[None, :]
        ok = np.ones((n, n), dtype=bool)
        if causal:
            ok &= (j < i) | (i == 0) & (j == 0) if kind == "strict_causal" else j <= i
        if kv is not None:
            ok &= j <= kv if kind == "kv_off_by_one" else j < kv
        s = (q @ k.T) if kind == "no_scale" else scale * (q @ k.T)
        m = np.where(ok, s, -np.inf).max(axis=1)
        e = np.where(ok, np.exp(np.where(ok, s, 0.0) - m[:, None]), 0.0)
        den = e.sum(1)
        p = e / den[:, None]
        lse = np.log(den) if kind == "lse_without_max" else m + np.log(den)
        o = (e @ v) if kind == "unnormalised" else p @ v
        return o, lse, p

    return fwd


def _bwd_variant(kind):
    def bwd(q, k, v, do, *, causal, scale, kv=None):
        q, k, v, do = (np.asarray(x, dtype=np.float64) for x in (q, k, v, do))
        _, _, p = O.head_forward(q, k, v, causal=causal, scale=scale, kv=kv)
        dv = (p @ do) if kind == "dv_untransposed" else p.T @ do
        dp = do @ v.T
        dref = (p * dp).sum(1)
        if kind == "drop_D":
            ds = p * dp
        elif kind == "sign_D":
            ds = p * dp + p * dref[:, None]
        else:
            ds = p * dp - p * dref[:, None]
        dq = (ds @ k) if kind == "dq_no_scale" else scale * (ds @ k)
        dk = scale * (ds @ q) if kind == "dk_transposed" else scale * (ds.T @ q)
        if kind == "dq_uses_q":
            dq = scale * (ds @ q)
        return dq, dk, dv, dref

    return bwd


MUTANTS = {
    "strict_causal_mask": _mutant(fwd=_fwd_variant("strict_causal")),
    "kv_off_by_one": _mutant(fwd=_fwd_variant("kv_off_by_one")),
    "scale_dropped": _mutant(fwd=_fwd_variant("no_scale")),
    "lse_missing_max": _mutant(fwd=_fwd_variant("lse_without_max")),
    "output_unnormalised": _mutant(fwd=_fwd_variant("unnormalised")),
    "dV_untransposed": _mutant(bwd=_bwd_variant("dv_untransposed")),
    "dS_drops_D_term": _mutant(bwd=_bwd_variant("drop_D")),
    "dS_wrong_sign": _mutant(bwd=_bwd_variant("sign_D")),
    "dQ_scale_dropped": _mutant(bwd=_bwd_variant("dq_no_scale")),
    "dK_transposed": _mutant(bwd=_bwd_variant("dk_transposed")),
    "dQ_uses_Q": _mutant(bwd=_bwd_variant("dq_uses_q")),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(name):
    impl = MUTANTS[name]
    failed = []
    for pin in PINS:
        try:
            pin(impl)
        except (AssertionError, ValueError, IndexError, FloatingPointError):
            failed.append(pin.__name__)
    assert failed, f"planted mistake {name!r} passed every pin"


# --------------------------------------------------------------------------------------------
# Row-wise oracle (head_rows, head_tail_keys): used at sequence lengths whose N x N matrices do not
# fit.  Pinned against the full oracle above (itself pinned by closed forms, finite differences,
# brute force and torch) and against closed forms; planted mistakes must fail a pin.


def rpin_rows_match_full(impl):
    """Every row from head_rows equals the same row of the materialised definition."""
    r = _rng(21)
    n, d = 45, 7
    q, k, v, do = r.normal(size=(4, n, d))
    for causal, kv in ((True, None), (False, None), (True, 30), (False, 12), (True, 1)):
        o, lse, _ = O.head_forward(q, k, v, causal=causal, scale=0.45, kv=kv)
        dq, _, _, dref = O.head_backward(q, k, v, do, causal=causal, scale=0.45, kv=kv)
        rows = [0, 1, 13, 29, 30, 44]
        ro, rl, rdq, rd = impl.head_rows(q, k, v, do, rows, causal=causal, scale=0.45, kv=kv)
        np.testing.assert_allclose(ro, o[rows], atol=1e-13)
        np.testing.assert_allclose(rl, lse[rows], atol=1e-13)
        np.testing.assert_allclose(rdq, dq[rows], atol=1e-13)
        np.testing.assert_allclose(rd, dref[rows], atol=1e-13)


def rpin_rows_zero_query(impl):
    """Q = 0: each row's output is the mean of its visible V rows, L_i = ln(#visible)."""
    r = _rng(22)
    n, d = 33, 4
    k, v, do = r.normal(size=(3, n, d))
    q = np.zeros((n, d))
    for causal, kv in ((True, None), (True, 20), (False, 7)):
        rows = list(range(n))
        o, lse, _, _ = impl.head_rows(q, k, v, do, rows, causal=causal, scale=0.8, kv=kv)
        for i in rows:
            hi = n if kv is None else kv
            if causal:
                hi = min(hi, i + 1)
            np.testing.assert_allclose(o[i], v[:hi].mean(0), atol=1e-13)
            np.testing.assert_allclose(lse[i], math.log(hi), atol=1e-13)


def rpin_tail_keys_match_full(impl):
    """dK, dV of the last keys from their few query rows equal the materialised backward."""
    r = _rng(23)
    n, d = 38, 6
    q, k, v, do = r.normal(size=(4, n, d))
    _, dk, dv, _ = O.head_backward(q, k, v, do, causal=True, scale=0.55, kv=None)
    for nt in (1, 5, 17):
        tk, tv = impl.head_tail_keys(q, k, v, do, nt, scale=0.55)
        np.testing.assert_allclose(tk, dk[n - nt:], atol=1e-13)
        np.testing.assert_allclose(tv, dv[n - nt:], atol=1e-13)


def rpin_tail_keys_padded_match_full(impl):
    """With key padding kv < N, the last visible keys' dK, dV (from rows j0 .. N - 1, the rows past kv
    included) equal the materialised backward; keys past kv have no gradient at all."""
    r = _rng(24)
    n, d = 41, 5
    q, k, v, do = r.normal(size=(4, n, d))
    for kv, nt in ((30, 1), (30, 6), (12, 12), (40, 9)):
        _, dk, dv, _ = O.head_backward(q, k, v, do, causal=True, scale=0.6, kv=kv)
        tk, tv = impl.head_tail_keys(q, k, v, do, nt, scale=0.6, kv=kv)
        np.testing.assert_allclose(tk, dk[kv - nt:kv], atol=1e-13)
        np.testing.assert_allclose(tv, dv[kv - nt:kv], atol=1e-13)
        assert not dk[kv:].any() and not dv[kv:].any()


RPINS = [rpin_rows_match_full, rpin_rows_zero_query, rpin_tail_keys_match_full, rpin_tail_keys_padded_match_full]


@pytest.mark.parametrize("pin", RPINS, ids=lambda p: p.__name__)
def test_row_oracle_pin(pin):
    pin(O)


def _rows_variant(kind):
    def rows_fn(q, k, v, do, rows, *, causal, scale, kv=None):
        q, k, v, do = (np.asarray(x, dtype=np.float64) for x in (q, k, v, do))
        n = k.shape[0]
        out = ([], [], [], [])
        for i in rows:
            hi = n if kv is None else kv
            if causal:
                hi = min(hi, i if kind == "causal_excludes_diagonal" and i > 0 else i + 1)
            s = scale * (k[:hi] @ q[i])
            e = np.exp(s - s.max())
            p = e / e.sum()
            dp = v[:hi] @ do[i]
            d_i = p @ dp
            ds = p * dp if kind == "drop_D" else p * dp - p * d_i
            out[0].append(p @ v[:hi])
            out[1].append(s.max() + np.log(e.sum()))
            out[2].append((ds @ k[:hi]) if kind == "dq_no_scale" else scale * (ds @ k[:hi]))
            out[3].append(d_i)
        return tuple(np.array(x) for x in out)

    return rows_fn


def _tail_variant(kind):
    def tail_fn(q, k, v, do, ntail, *, scale, kv=None):
        q, k, v, do = (np.asarray(x, dtype=np.float64) for x in (q, k, v, do))
        n = k.shape[0]
        hi = n if kv is None else kv
        j0 = hi - ntail
        dk = np.zeros((ntail, k.shape[1]))
        dv = np.zeros((ntail, v.shape[1]))
        first = j0 + 1 if kind == "skip_first_row" else j0
        last = hi if kind == "rows_stop_at_kv" else n
        for i in range(first, last):
            vis = min(i + 1, hi)
            s = scale * (k[:vis] @ q[i])
            e = np.exp(s - s.max())
            p = e / e.sum()
            dp = v[:vis] @ do[i]
            ds = p * dp - p * (p @ dp)
            for j in range(j0, vis):
                dv[j - j0] += p[j] * do[i]
                dk[j - j0] += (ds[j] * k[j]) * scale if kind == "dk_uses_k" else scale * ds[j] * q[i]
        return dk, dv

    return tail_fn


ROW_MUTANTS = {
    "rows_causal_excludes_diagonal": types.SimpleNamespace(head_rows=_rows_variant("causal_excludes_diagonal"),
                                                           head_tail_keys=O.head_tail_keys),
    "rows_drop_D": types.SimpleNamespace(head_rows=_rows_variant("drop_D"), head_tail_keys=O.head_tail_keys),
    "rows_dq_no_scale": types.SimpleNamespace(head_rows=_rows_variant("dq_no_scale"), head_tail_keys=O.head_tail_keys),
    "tail_skips_first_row": types.SimpleNamespace(head_rows=O.head_rows, head_tail_keys=_tail_variant("skip_first_row")),
    "tail_dk_uses_k": types.SimpleNamespace(head_rows=O.head_rows, head_tail_keys=_tail_variant("dk_uses_k")),
    "tail_rows_stop_at_kv": types.SimpleNamespace(head_rows=O.head_rows,
                                                  head_tail_keys=_tail_variant("rows_stop_at_kv")),
}


@pytest.mark.parametrize("name", sorted(ROW_MUTANTS))
def test_planted_row_mistake_is_caught(name):
    impl = ROW_MUTANTS[name]
    failed = []
    for pin in RPINS:
        try:
            pin(impl)
        except (AssertionError, ValueError, IndexError, FloatingPointError):
            failed.append(pin.__name__)
    assert failed, f"planted mistake {name!r} passed every row pin"


def test_correct_variants_pass_row_pins():
    """The mutant builders without a planted mistake pass every row pin (so failures above are
    due to the planted mistake, not to the builders)."""
    ok = types.SimpleNamespace(head_rows=_rows_variant("none"), head_tail_keys=_tail_variant("none"))
    for pin in RPINS:
        pin(ok)
