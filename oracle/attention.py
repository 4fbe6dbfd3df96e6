"""CPU oracle for causal / key-padded scaled dot-product attention, forward and backward.

TEST INFRASTRUCTURE ONLY. Nothing on the product path may import, call or execute this
module: only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` use it. It shares no code with the HIP library (no kernels, headers, tables or
helpers) and never receives a value produced by the GPU path.

What it computes, and where that is defined:

* Forward: eq. (1) of the CS336 Assignment 2 (systems) handout (§4.1 "Optimizing Attention
  with FlashAttention-2") and eqs. (4)-(6) of its §4.2.2 "FlashAttention-2 forward pass":
  ``S = scale * Q K^T``, masked entries removed, row softmax ``P``, ``O = P V``.  The logsumexp
  ``L_i = log sum_j exp(S_ij)`` is eq. (12), natural log, over the unmasked entries of row i.
* Masking: Problem (flash_forward)(c) of the same handout builds a square causal mask from
  query and key index vectors and pushes masked scores to a large negative value so they get
  no weight. Here the weight of a masked entry is exactly 0 (``np.where``), which is what the
  large negative constant achieves after ``exp`` underflows. A key-padding length ``kv``
  additionally removes keys ``j >= kv`` for every query of that batch row.
* Backward: the *textbook* form, eqs. (7)-(11): ``dV = P^T dO``, ``dP = dO V^T``,
  ``dS_i = (diag(P_i) - P_i P_i^T) dP_i``, ``dQ = scale * dS K``, ``dK = scale * dS^T Q``.
  It deliberately does not use the ``D = rowsum(O o dO)`` shortcut of eqs. (13)-(19); the
  row dot product ``P_i . dP_i`` is taken from P and dP, so the oracle is independent of the
  pre-pass it is used to check.  ``rowsum_p_dp`` returns that dot product as ``D_ref``.
* Block-sparse masking: the "Block-sparse Flashattention" section of "Notes on flashattention"
  restricts the scores to the support of a mask M that is constant on blocks: entry (i, j) is
  kept iff ``block_mask[i // block, j // block]`` is non-zero.  The page writes the masked score
  as 0; read literally that would give masked keys weight exp(0), which contradicts the same
  section's point that zero blocks need no work at all, so here (as for the causal mask) a
  masked entry has weight exactly 0.  A row left with no key at all has no softmax; for it the
  oracle returns O = 0, L = -inf and zero gradients (a block mask can produce such rows; causal
  and key-padding masks with kv >= 1 cannot).
* Theorem 1 of "Notes on flashattention" (section Analysis / Correctness) shows the tiled
  online-softmax forward returns exactly ``softmax(S) V``; that is why an untiled, materialised
  reference is the right thing to compare a tiled kernel against.

Everything is float64 numpy, one (batch, head) at a time, materialising the full N x N
matrices. The only library primitive used as a step is the matrix product.
"""

from __future__ import annotations

import numpy as np

__all__ = [
    "valid_mask",
    "head_rows",
    "head_tail_keys",
    "head_forward",
    "head_backward",
    "attention_forward",
    "attention_backward",
    "rowsum_p_dp",
    "rowsum_o_do",
]


def _f64(x) -> np.ndarray:
    """Upcast to float64 (exact for bf16 and fp32 inputs). Accepts numpy arrays or CPU torch tensors."""
    if hasattr(x, "detach"):  # a CPU torch tensor: go through float32/float64 on the torch side
        import torch

        x = x.detach().to(dtype=torch.float64, device="cpu").numpy()
    return np.asarray(x, dtype=np.float64)


def valid_mask(n: int, causal: bool, kv: int | None, block_mask=None, block: int = 64) -> np.ndarray:
    """Boolean ``[n, n]`` matrix, True where query i may attend key j.

    Causal (handout Problem (flash_forward)(c)): key j is masked for query i when j > i; the
    diagonal is kept (square mask, equal query and key lengths).  Key padding: keys j >= kv are
    masked for every query.  ``kv=None`` means no padding.  Block-sparse ("Notes on
    flashattention", Block-sparse Flashattention): ``block_mask`` is a ``[ceil(n/block)]^2``
    array and (i, j) is kept only where ``block_mask[i // block, j // block]`` is non-zero.
    """
    i = np.arange(n)[:, None]
    j = np.arange(n)[None, :]
    ok = np.ones((n, n), dtype=bool)
    if causal:
        ok &= j <= i
    if kv is not None:
        ok &= j < kv
    if block_mask is not None:
        bm = np.asarray(block_mask) != 0
        tb = -(-n // block)
        if bm.shape != (tb, tb):
            raise ValueError(f"block_mask must be [{tb}, {tb}] for n={n}, block={block}")
        ok &= bm[i // block, j // block]
    return ok


def head_forward(q, k, v, *, causal: bool, scale: float, kv: int | None = None, block_mask=None,
                 block: int = 64):
    """One head. q, k, v: ``[N, d]``. Returns ``(O [N, d], L [N], P [N, N])`` in float64.

    Eq. (4): S = scale * q k^T.  Eq. (5): row softmax over the unmasked entries (shifted by the
    row maximum for stability; the shift cancels).  Eq. (6): O = P v.  Eq. (12): L = log of the
    row sum of exp(S) over unmasked entries, written as m + log(sum exp(S - m)).
    Without a block mask every row must keep at least one key (kv >= 1) and a fully masked row is
    rejected; with one, a row left without keys gets P = 0, O = 0 and L = -inf.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    n = q.shape[0]
    ok = valid_mask(n, causal, kv, block_mask, block)
    live = ok.any(axis=1)
    if block_mask is None and not live.all():
        raise ValueError("a query row has no unmasked key (kv_len must be >= 1)")
    s = scale * (q @ k.T)
    m = np.where(live, np.where(ok, s, -np.inf).max(axis=1), 0.0)
    e = np.where(ok, np.exp(np.where(ok, s, 0.0) - m[:, None]), 0.0)
    denom = e.sum(axis=1)
    p = e / np.where(live, denom, 1.0)[:, None]
    lse = np.where(live, m + np.log(np.where(live, denom, 1.0)), -np.inf)
    o = p @ v
    return o, lse, p


def head_backward(q, k, v, do, *, causal: bool, scale: float, kv: int | None = None, block_mask=None,
                  block: int = 64):
    """One head. Returns ``(dQ, dK, dV, D_ref)`` in float64 via the textbook eqs. (7)-(11).

    dV = P^T dO (7); dP = dO v^T (8); dS_i = P_i o dP_i - P_i (P_i . dP_i) which is eq. (9)'s
    (diag(P_i) - P_i P_i^T) dP_i written row by row; dQ = scale dS k (10); dK = scale dS^T q (11).
    D_ref is the row dot product P_i . dP_i taken on the way.
    """
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(do)
    _, _, p = head_forward(q, k, v, causal=causal, scale=scale, kv=kv, block_mask=block_mask, block=block)
    dv = p.T @ do
    dp = do @ v.T
    d_ref = (p * dp).sum(axis=1)
    ds = p * dp - p * d_ref[:, None]
    dq = scale * (ds @ k)
    dk = scale * (ds.T @ q)
    return dq, dk, dv, d_ref


def _row_terms(q, k, v, do, i, causal, scale, kv):
    """Row i of the definition as vectors over its visible keys (no N x N matrix): returns the key
    indices, p (eq. 5 row), L_i (eq. 12), and, when do is given, ds_i (eq. 9 row form) and D_i."""
    n = k.shape[0]
    hi = n if kv is None else kv
    if causal:
        hi = min(hi, i + 1)
    if hi < 1:
        raise ValueError("a query row has no unmasked key (kv_len must be >= 1)")
    keys = np.arange(hi)
    s = scale * (k[:hi] @ q[i])
    m = s.max()
    e = np.exp(s - m)
    tot = e.sum()
    p = e / tot
    lse = m + np.log(tot)
    if do is None:
        return keys, p, lse, None, None
    dp = v[:hi] @ do[i]  # dP_ij = do_i . v_j (eq. 8)
    d_i = float(p @ dp)
    ds = p * dp - p * d_i  # eq. 9, row form
    return keys, p, lse, ds, d_i


def head_rows(q, k, v, do, rows, *, causal: bool, scale: float, kv: int | None = None):
    """Selected query rows of one head, each evaluated from its own row of the definition.

    For row i: scores s_j = scale q_i . k_j over the visible keys, p = softmax(s) (eq. 5),
    o_i = p V (eq. 6), L_i = log sum_j exp(s_j) (eq. 12); with do, the row form of eqs. (8)-(10):
    dP_ij = do_i . v_j, D_i = p . dP_i, dS_i = p o dP_i - p D_i, dq_i = scale dS_i K.
    Costs O(N d) per row, so it serves sequence lengths whose N x N matrices do not fit.
    Returns ``(O [r, d], L [r], dQ [r, d] or None, D [r] or None)`` in float64.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    do = None if do is None else _f64(do)
    rows = [int(i) for i in rows]
    o = np.zeros((len(rows), v.shape[1]))
    lse = np.zeros(len(rows))
    dq = None if do is None else np.zeros((len(rows), q.shape[1]))
    dd = None if do is None else np.zeros(len(rows))
    for r, i in enumerate(rows):
        keys, p, l_i, ds, d_i = _row_terms(q, k, v, do, i, causal, scale, kv)
        o[r] = p @ v[keys]
        lse[r] = l_i
        if do is not None:
            dq[r] = scale * (ds @ k[keys])
            dd[r] = d_i
    return o, lse, dq, dd


def head_tail_keys(q, k, v, do, ntail: int, *, scale: float, kv: int | None = None):
    """dK_j, dV_j (eqs. 7 and 11) for the last ``ntail`` visible keys of one causal head.

    Under the causal mask key j is seen only by queries i >= j, so for the keys
    j0 = kv' - ntail .. kv' - 1 (kv' = kv with key padding, else N) the sums over i run over
    rows j0 .. N - 1 alone: dV_j = sum_i P_ij do_i, dK_j = scale sum_i dS_ij q_i, with each row's
    P_i and dS_i from that row of the definition.  With padding, the rows past kv still see these
    keys (queries are never masked), so they are part of the sums.
    Returns ``(dK [ntail, d], dV [ntail, d])`` in float64, keys kv' - ntail .. kv' - 1.
    """
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(do)
    n = k.shape[0]
    hi = n if kv is None else kv
    if not 1 <= ntail <= hi:
        raise ValueError("ntail must be in [1, number of visible keys]")
    j0 = hi - ntail
    dk = np.zeros((ntail, k.shape[1]))
    dv = np.zeros((ntail, v.shape[1]))
    for i in range(j0, n):
        keys, p, _, ds, _ = _row_terms(q, k, v, do, i, True, scale, kv)
        sel = keys >= j0
        dv[keys[sel] - j0] += p[sel, None] * do[i][None, :]
        dk[keys[sel] - j0] += scale * ds[sel, None] * q[i][None, :]
    return dk, dv


def _kv_of(kv_len, b: int):
    if kv_len is None:
        return None
    return int(np.asarray(kv_len).reshape(-1)[b])


def attention_forward(q, k, v, *, causal: bool, scale: float, kv_len=None, heads=None, block_mask=None,
                      block: int = 64):
    """Batched forward over ``[B, H, N, d]``. Returns ``(O [B,H,N,d], L [B,H,N])`` float64.

    ``kv_len``: per-batch key lengths ``[B]`` or None. ``heads``: optional list of ``(b, h)``
    pairs; when given only those heads are computed and the result arrays hold NaN elsewhere.
    ``block_mask``: optional ``[ceil(N/block)]^2`` block-sparse mask shared by every head.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, H, N, d = q.shape
    o = np.full((B, H, N, v.shape[-1]), np.nan)
    lse = np.full((B, H, N), np.nan)
    for b, h in heads if heads is not None else [(b, h) for b in range(B) for h in range(H)]:
        o[b, h], lse[b, h], _ = head_forward(
            q[b, h], k[b, h], v[b, h], causal=causal, scale=scale, kv=_kv_of(kv_len, b), block_mask=block_mask,
            block=block
        )
    return o, lse


def attention_backward(q, k, v, do, *, causal: bool, scale: float, kv_len=None, heads=None, block_mask=None,
                       block: int = 64):
    """Batched backward. Returns ``(dQ, dK, dV, D_ref)`` float64 (NaN outside ``heads`` if given)."""
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(do)
    B, H, N, d = q.shape
    dq = np.full(q.shape, np.nan)
    dk = np.full(k.shape, np.nan)
    dv = np.full(v.shape, np.nan)
    dref = np.full((B, H, N), np.nan)
    for b, h in heads if heads is not None else [(b, h) for b in range(B) for h in range(H)]:
        dq[b, h], dk[b, h], dv[b, h], dref[b, h] = head_backward(
            q[b, h], k[b, h], v[b, h], do[b, h], causal=causal, scale=scale, kv=_kv_of(kv_len, b),
            block_mask=block_mask, block=block
        )
    return dq, dk, dv, dref


def rowsum_p_dp(q, k, v, do, *, causal: bool, scale: float, kv_len=None, heads=None):
    """``D_i = P_i . dP_i`` from the materialised P and dP (the quantity eq. (9) needs)."""
    return attention_backward(q, k, v, do, causal=causal, scale=scale, kv_len=kv_len, heads=heads)[3]


def rowsum_o_do(o, do):
    """``D = rowsum(O o dO)`` (handout §4.2.2, "backward pass with recomputation"), float64."""
    return (_f64(o) * _f64(do)).sum(axis=-1)
