"""The softmax forms the pages derive, each written out in the pages' order (test infrastructure).

All of them compute the same numbers in exact arithmetic; the tests check that
they agree in fp64 and against hand-derived values. The main attention oracle
uses only the three-pass form; the others exist so that the recurrences the
tiled kernel relies on are themselves pinned.

* row_softmax: the plain definition over every row of a matrix (the target of
  the standalone row-softmax kernel).
* three_pass: "why attention is slow" (page 2), time-complexity section -
  the safe softmax in three loops: running max, denominator scaled by the
  final max, then each probability.
* online_normalizer / two_pass: same page - the online normalizer
  (attributed there to NVIDIA, 2018), where the denominator is kept relative to
  the running max: d'_i = d'_(i-1) e^(m_(i-1) - m_i) + e^(x_i - m_i); a second
  loop then divides e^(x_i - m_N) by d'_N. A block size > 1 folds a whole block
  of x into one step of the same recurrence.
* one_pass_output: lecture summary (page 3), section 3.2 "online softmax",
  the one-pass form with an output: per block, the running max m, the running
  denominator l~ and the running normalised output o~ are updated as
      m_i  = max(m_(i-1), max of this block's scores)
      l~_i = l~_(i-1) e^(m_(i-1) - m_i) + sum_k e^(s_k - m_i)
      o~_i = o~_(i-1) l~_(i-1) e^(m_(i-1) - m_i) / l~_i + sum_k e^(s_k - m_i) V_k / l~_i
  (the printed formula is garbled; this is its reading).
* one_pass_deferred: the same recurrence with o kept unnormalised and divided
  by l once at the end - the reading taken for the FlashAttention-2 forward's
  "fewer non-matmul operations" (page 1, FlashAttention-2 main operations,
  whose figure is missing from the text).
"""
from __future__ import annotations

import math

import numpy as np


def three_pass(x) -> np.ndarray:
    """Safe softmax of a 1-D vector in three passes; -inf entries get probability 0."""
    x = np.asarray(x, dtype=np.float64)
    m = -np.inf
    for xi in x:                      # pass 1: m_i = max(m_(i-1), x_i)
        m = max(m, xi)
    d = 0.0
    for xi in x:                      # pass 2: d_i = d_(i-1) + e^(x_i - m_N)
        d = d + math.exp(xi - m)
    a = np.empty_like(x)
    for i, xi in enumerate(x):        # pass 3: a_i = e^(x_i - m_N) / d_N
        a[i] = math.exp(xi - m) / d
    return a


def row_softmax(x) -> np.ndarray:
    """Softmax of every row of a 2-D array, in fp64: the plain definition.

    Row r: e^(x_rc - m_r) / sum_c e^(x_rc - m_r) with m_r the row maximum
    (the safe softmax of the same page). Entries equal to -inf get 0. A row
    with no finite entry has no defined softmax; the reading taken here is an
    all-zero row, the same convention as a query row that sees no key.
    """
    x = np.asarray(x, dtype=np.float64)
    m = x.max(axis=1, keepdims=True)
    live = np.isfinite(m)
    e = np.where(live, np.exp(x - np.where(live, m, 0.0)), 0.0)
    tot = e.sum(axis=1, keepdims=True)
    return np.where(live, e / np.where(live, tot, 1.0), 0.0)


def online_normalizer(x, block: int = 1):
    """Running (m_i, d'_i) after each block of x; returns (list of m, list of d')."""
    x = np.asarray(x, dtype=np.float64)
    m_prev, d_prev = -np.inf, 0.0
    ms, ds = [], []
    for b0 in range(0, x.shape[0], block):
        xb = x[b0:b0 + block]
        m_new = max(m_prev, float(xb.max()))
        # e^(m_(i-1) - m_i): the first step has d' = 0, so its factor is irrelevant
        carry = 0.0 if d_prev == 0.0 else d_prev * math.exp(m_prev - m_new)
        d_new = carry + float(np.sum(np.exp(xb - m_new)))
        ms.append(m_new)
        ds.append(d_new)
        m_prev, d_prev = m_new, d_new
    return ms, ds


def two_pass(x, block: int = 1) -> np.ndarray:
    """Softmax via the online normalizer, then a_i = e^(x_i - m_N) / d'_N."""
    x = np.asarray(x, dtype=np.float64)
    ms, ds = online_normalizer(x, block)
    m_n, d_n = ms[-1], ds[-1]
    return np.exp(x - m_n) / d_n


def one_pass_output(s, V, block: int = 1):
    """One-pass softmax-weighted sum of V's rows for one query's scores s.

    Normalised running output, as in the lecture's recurrence. Returns
    (o, m_N, l_N) with o = sum_k softmax(s)_k V_k.
    """
    s = np.asarray(s, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    m, l = -np.inf, 0.0
    o = np.zeros(V.shape[1])
    for b0 in range(0, s.shape[0], block):
        sb, vb = s[b0:b0 + block], V[b0:b0 + block]
        m_new = max(m, float(sb.max()))
        w = np.exp(sb - m_new)                       # e^(s_k - m_i)
        shrink = 0.0 if l == 0.0 else math.exp(m - m_new)
        l_new = l * shrink + float(w.sum())
        o = o * (l * shrink / l_new) + (w @ vb) / l_new
        m, l = m_new, l_new
    return o, m, l


def one_pass_deferred(s, V, block: int = 1):
    """As one_pass_output, but o is kept unnormalised and divided by l once at the end."""
    s = np.asarray(s, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    m, l = -np.inf, 0.0
    acc = np.zeros(V.shape[1])
    for b0 in range(0, s.shape[0], block):
        sb, vb = s[b0:b0 + block], V[b0:b0 + block]
        m_new = max(m, float(sb.max()))
        shrink = 0.0 if l == 0.0 else math.exp(m - m_new)
        w = np.exp(sb - m_new)
        l = l * shrink + float(w.sum())
        acc = acc * shrink + w @ vb
        m = m_new
    return acc / l, m, l
