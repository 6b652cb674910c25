"""CPU fp64 reference for decoding against a key/value cache (test infrastructure).

The pages mention inference with a KV cache and FlashDecoding (lecture summary,
remark after section 3.1 and the conclusion) without defining them. The reading
taken: the Nq queries are the newest Nq positions of a sequence whose Nk keys and
values are cached, so query i sits at position Nk - Nq + i; under the causal
mask it sees key j iff j <= Nk - Nq + i (aligned at the bottom right, which is
the top-left rule of the training-time oracle when Nq = Nk). What is computed is
the plain definition of attention over those pairs (lecture summary, section
2.1; three-pass safe softmax of the "why attention is slow" page):
O_i = sum_j softmax_j(scale q_i . k_j) v_j and LSE_i = ln sum_j e^(scale q_i . k_j)
over the visible keys; a query that sees no key gets O = 0 and LSE = -inf.

Only tests, the smoke check and the benchmark's CPU-baseline leg use this module.
"""
from __future__ import annotations

import numpy as np


def decode_head(q, k, v, *, scale: float, causal: bool):
    """One (batch, head): q [Nq, d], k [Nk, d], v [Nk, dv] -> (o [Nq, dv], lse [Nq])."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    nq, nk = q.shape[0], k.shape[0]
    s = scale * (q @ k.T)
    if causal:
        pos = nk - nq + np.arange(nq)
        s = np.where(np.arange(nk)[None, :] <= pos[:, None], s, -np.inf)
    m = s.max(axis=1) if nk else np.full(nq, -np.inf)
    empty = ~np.isfinite(m)
    ms = np.where(empty, 0.0, m)
    e = np.exp(s - ms[:, None])                       # pass 2: e^(s - m), masked entries 0
    l = e.sum(axis=1)
    p = e / np.where(empty, 1.0, l)[:, None]          # pass 3
    o = p @ v
    lse = np.where(empty, -np.inf, ms + np.log(np.where(empty, 1.0, l)))
    return o, lse


def decode(q, k, v, *, scale: float, causal: bool, heads=None):
    """Batched: q [B, H, Nq, d], k and v [B, H, Nk, d] -> dict(o, lse), float64.

    heads: optional iterable of (b, h); other heads hold NaN.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, H, nq, _ = q.shape
    o = np.full((B, H, nq, v.shape[3]), np.nan)
    lse = np.full((B, H, nq), np.nan)
    for b, h in (heads if heads is not None else [(b, h) for b in range(B) for h in range(H)]):
        o[b, h], lse[b, h] = decode_head(q[b, h], k[b, h], v[b, h], scale=scale, causal=causal)
    return {"o": o, "lse": lse}
