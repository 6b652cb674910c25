"""Brute-force attention in pure Python loops, for tiny inputs only (test infrastructure).

A second, independent spelling of the same definition, used to pin the NumPy
oracle: no arrays, no max subtraction (fine for the small scores used here),
math.fsum for every sum, and the backward through the explicit softmax Jacobian
dP_a/dS_b = P_a (delta_ab - P_b) (lecture summary, page 3, part 4.1 mentions
the Jacobian) instead of the rowsum shortcut the NumPy oracle uses.

Forward: softmax(scale Q K^T) V with the same mask readings as the oracle
(lecture summary, section 2.1, for the formula; causal = key j <= query i;
block mask = keep[i // block][j // block]).
"""
from __future__ import annotations

import math


def _ok(i, j, causal, block_mask, block):
    if causal and j > i:
        return False
    if block_mask is not None and not block_mask[i // block][j // block]:
        return False
    return True


def attention_brute(q, k, v, do, scale, causal=False, block_mask=None, block=4):
    """q, k: N x d nested lists; v, do: N x dv. Returns dict(o, lse, dq, dk, dv)."""
    n, nk = len(q), len(k)
    d, dv_ = len(q[0]), len(v[0])
    P = [[0.0] * nk for _ in range(n)]
    o = [[0.0] * dv_ for _ in range(n)]
    lse = [-math.inf] * n
    for i in range(n):
        keys = [j for j in range(nk) if _ok(i, j, causal, block_mask, block)]
        if not keys:
            continue
        ex = {j: math.exp(scale * math.fsum(q[i][c] * k[j][c] for c in range(d))) for j in keys}
        z = math.fsum(ex.values())
        for j in keys:
            P[i][j] = ex[j] / z
        lse[i] = math.log(z)
        for c in range(dv_):
            o[i][c] = math.fsum(P[i][j] * v[j][c] for j in keys)
    # backward: dV_j = sum_i P_ij dO_i ; dP_ij = dO_i . V_j
    dv = [[math.fsum(P[i][j] * do[i][c] for i in range(n)) for c in range(dv_)] for j in range(nk)]
    dP = [[math.fsum(do[i][c] * v[j][c] for c in range(dv_)) for j in range(nk)] for i in range(n)]
    # dS_ib = sum_a dP_ia * P_ia * (delta_ab - P_ib)   (softmax Jacobian, row i)
    dS = [[0.0] * nk for _ in range(n)]
    for i in range(n):
        for b in range(nk):
            dS[i][b] = math.fsum(dP[i][a] * P[i][a] * ((1.0 if a == b else 0.0) - P[i][b])
                                 for a in range(nk))
    # S = scale * Q K^T  =>  dQ_i = scale sum_j dS_ij K_j ; dK_j = scale sum_i dS_ij Q_i
    dq = [[scale * math.fsum(dS[i][j] * k[j][c] for j in range(nk)) for c in range(d)]
          for i in range(n)]
    dk = [[scale * math.fsum(dS[i][j] * q[i][c] for i in range(n)) for c in range(d)]
          for j in range(nk)]
    return {"o": o, "lse": lse, "dq": dq, "dk": dk, "dv": dv}
