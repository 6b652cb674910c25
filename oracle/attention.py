"""CPU fp64 reference for exact attention, forward and backward (test infrastructure).

This is the plain definition written out, S and P materialised, so that a
reader can check it against the pages by eye:

* lecture summary (page 3), part 2 "standard attention", section 2.1:
  Attention(Q, K, V) = softmax(Q K^T / sqrt(d_k)) V; section 2.2 lists the
  three steps S = Q K^T, P = softmax(S), O = P V.
* "why attention is slow" (page 2), section on time complexity: the
  three-pass safe softmax (row max m, denominator sum of e^(x - m), then
  e^(x - m) / denominator).
* overview article (page 1), FlashAttention-2 "main operations", backward
  pass: the backward keeps only the row logsumexp, LSE = m + ln l.
* The backward itself is the chain rule through the softmax Jacobian (page 3,
  part 4.1 names it without printing it): with dP = dO V^T,
  D_i = sum_j P_ij dP_ij, dS = P o (dP - D), dQ = scale dS K,
  dK = scale dS^T Q, dV = P^T dO.

Readings taken where the pages are silent (each listed in the design notes):
* scale multiplies the scores inside the softmax: S = scale Q K^T;
* LSE uses the natural log and is of the scaled scores;
* causal means key j is allowed for query i iff j <= i (top-left aligned);
* a block mask is an [N/block, N/block] 0/1 grid, one per call, keep = 1;
  masked pairs have P = 0 and receive no gradient;
* a query row with no allowed key gets O = 0, LSE = -inf, zero gradients.

Nothing in the product (the HIP library and its binding) imports this module;
only tests, the smoke check and the benchmark's CPU-baseline leg call it.
Work is split over independent chunks of query rows only, to bound memory:
each row's S, P, O, LSE and dQ are computed exactly as in the unchunked
definition, and dK, dV sum the per-chunk terms.
"""
from __future__ import annotations

import numpy as np


def allowed(rows: np.ndarray, n_k: int, causal: bool, block_mask, block: int) -> np.ndarray:
    """Boolean [len(rows), n_k]: may query row i attend key j."""
    cols = np.arange(n_k)
    a = np.ones((rows.shape[0], n_k), dtype=bool)
    if causal:
        a &= cols[None, :] <= rows[:, None]
    if block_mask is not None:
        bm = np.asarray(block_mask).astype(bool)
        a &= bm[(rows // block)[:, None], (cols // block)[None, :]]
    return a


def softmax_rows(q_rows, k, rows, *, scale: float, causal: bool, block_mask, block: int):
    """P and LSE for the query rows `rows` (q_rows = Q[rows]) against all keys.

    S = scale * Q K^T with disallowed pairs at -inf, then the safe softmax in
    its three passes. Returns (p [len(rows), Nk], lse [len(rows)]).
    """
    ok = allowed(rows, k.shape[0], causal, block_mask, block)
    s = np.where(ok, scale * (q_rows @ k.T), -np.inf)
    # pass 1: row max
    m = s.max(axis=1)
    empty = ~ok.any(axis=1)
    m_safe = np.where(empty, 0.0, m)
    # pass 2: denominator l = sum_j e^(s - m)   (e^-inf = 0)
    e = np.exp(s - m_safe[:, None])
    l = e.sum(axis=1)
    # pass 3: P = e^(s - m) / l
    p = e / np.where(empty, 1.0, l)[:, None]
    lse = np.where(empty, -np.inf, m_safe + np.log(np.where(empty, 1.0, l)))
    return p, lse


def attention_head(q, k, v, do=None, *, scale: float, causal: bool = False,
                   block_mask=None, block: int = 128, chunk: int = 1024):
    """One (batch, head): q [N, d], k [Nk, d], v [Nk, dv], do [N, dv] (float64).

    Returns dict(o, lse, and if do is given: dq, dk, dv, D).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    n = q.shape[0]
    out = {
        "o": np.zeros((n, v.shape[1])),
        "lse": np.full(n, -np.inf),
    }
    grads = do is not None
    if grads:
        do = np.asarray(do, dtype=np.float64)
        out["dq"] = np.zeros_like(q)
        out["dk"] = np.zeros_like(k)
        out["dv"] = np.zeros_like(v)
        out["D"] = np.zeros(n)
    for r0 in range(0, n, chunk):
        rows = np.arange(r0, min(n, r0 + chunk))
        p, lse = softmax_rows(q[rows], k, rows, scale=scale, causal=causal,
                              block_mask=block_mask, block=block)
        out["o"][rows] = p @ v
        out["lse"][rows] = lse
        if grads:
            dor = do[rows]
            out["dv"] += p.T @ dor
            dp = dor @ v.T
            dvec = (p * dp).sum(axis=1)
            ds = p * (dp - dvec[:, None])
            out["dq"][rows] = scale * (ds @ k)
            out["dk"] += scale * (ds.T @ q[rows])
            out["D"][rows] = dvec
    return out


def attention(q, k, v, do=None, *, scale: float, causal: bool = False, block_mask=None,
              block: int = 128, chunk: int = 1024, heads=None):
    """Batched [B, H, N, d] arrays (anything np.asarray accepts; bf16 torch tensors
    should be converted with .double().numpy() first).

    heads: optional iterable of (b, h) pairs; only those heads are computed and
    the result arrays hold NaN elsewhere (for sampled checks at full size).
    block_mask: None, one [nb, nb] grid shared by every head, or [B, H, nb, nb].
    Returns dict of float64 arrays: o, lse (and dq, dk, dv, D when do is given).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, H, n, _ = q.shape
    if do is not None:
        do = np.asarray(do, dtype=np.float64)
    bm = None if block_mask is None else np.asarray(block_mask)
    keys = ["o", "lse"] + (["dq", "dk", "dv", "D"] if do is not None else [])
    shapes = {"o": (B, H, n, v.shape[3]), "lse": (B, H, n), "dq": q.shape,
              "dk": k.shape, "dv": v.shape, "D": (B, H, n)}
    res = {key: np.full(shapes[key], np.nan) for key in keys}
    todo = [(b, h) for b in range(B) for h in range(H)] if heads is None else list(heads)
    for b, h in todo:
        mask_bh = None if bm is None else (bm if bm.ndim == 2 else bm[b, h])
        r = attention_head(q[b, h], k[b, h], v[b, h], None if do is None else do[b, h],
                           scale=scale, causal=causal, block_mask=mask_bh, block=block,
                           chunk=chunk)
        for key in keys:
            res[key][b, h] = r[key]
    return res


def attention_rows(q, k, v, rows, *, scale: float, causal: bool = False, block_mask=None,
                   block: int = 128):
    """Forward outputs (o [len(rows), dv], lse [len(rows)]) for selected query rows of one head.

    Each row of the definition depends only on that query row and all of K, V,
    so sampled rows of a large problem cost O(len(rows) * Nk * d).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    rows = np.asarray(rows)
    p, lse = softmax_rows(q[rows], k, rows, scale=scale, causal=causal,
                          block_mask=block_mask, block=block)
    return p @ v, lse


def attention_dq_rows(q, k, v, do, rows, *, scale: float, causal: bool = False,
                      block_mask=None, block: int = 128):
    """dQ for selected query rows of one head: dQ_i needs only row i of P and dP."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    do = np.asarray(do, dtype=np.float64)
    rows = np.asarray(rows)
    p, _ = softmax_rows(q[rows], k, rows, scale=scale, causal=causal,
                        block_mask=block_mask, block=block)
    dp = do[rows] @ v.T
    dvec = (p * dp).sum(axis=1)
    ds = p * (dp - dvec[:, None])
    return scale * (ds @ k)
