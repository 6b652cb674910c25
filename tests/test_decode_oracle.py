"""Pins of the decoding oracle (oracle/decode.py) against things other than itself.

* Nq = Nk: the training-time oracle (top-left causal rule) gives the same rows;
* the last Nq rows of a full causal attention over Nk queries are exactly the
  decoding of those Nq queries (this fixes the bottom-right alignment);
* pure-Python loops on tiny inputs;
* closed forms: a zero query averages the visible values, LSE = ln(count);
  queries positioned before the first key see nothing (O = 0, LSE = -inf).
"""
import math

import numpy as np
import pytest

from oracle import attention_head
from oracle.decode import decode, decode_head


def _rand(rng, *shape):
    return rng.standard_normal(shape)


@pytest.mark.parametrize("causal", [False, True])
def test_square_case_is_the_training_oracle(causal):
    rng = np.random.default_rng(1)
    q, k, v = _rand(rng, 9, 6), _rand(rng, 9, 6), _rand(rng, 9, 5)
    o, lse = decode_head(q, k, v, scale=0.4, causal=causal)
    ref = attention_head(q, k, v, scale=0.4, causal=causal)
    np.testing.assert_allclose(o, ref["o"], rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(lse, ref["lse"], rtol=1e-13)


@pytest.mark.parametrize("nq", [1, 3, 16])
def test_last_rows_of_full_causal_attention(nq):
    rng = np.random.default_rng(2 + nq)
    nk, d = 40, 8
    Q, k, v = _rand(rng, nk, d), _rand(rng, nk, d), _rand(rng, nk, d)
    full = attention_head(Q, k, v, scale=0.3, causal=True)
    o, lse = decode_head(Q[nk - nq:], k, v, scale=0.3, causal=True)
    np.testing.assert_allclose(o, full["o"][nk - nq:], rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(lse, full["lse"][nk - nq:], rtol=1e-13)


def test_brute_force_loops():
    rng = np.random.default_rng(3)
    nq, nk, d = 2, 5, 3
    q, k, v = _rand(rng, nq, d), _rand(rng, nk, d), _rand(rng, nk, d)
    for causal in (False, True):
        o, lse = decode_head(q, k, v, scale=0.7, causal=causal)
        for i in range(nq):
            vis = [j for j in range(nk) if not causal or j <= nk - nq + i]
            w = [math.exp(0.7 * sum(q[i, c] * k[j, c] for c in range(d))) for j in vis]
            z = sum(w)
            assert lse[i] == pytest.approx(math.log(z), rel=1e-13)
            for c in range(d):
                assert o[i, c] == pytest.approx(sum(wj * v[j, c] for wj, j in zip(w, vis)) / z,
                                                rel=1e-12, abs=1e-14)


def test_zero_query_and_queries_before_the_cache():
    rng = np.random.default_rng(4)
    nq, nk, d = 4, 6, 5
    k, v = _rand(rng, nk, d), _rand(rng, nk, d)
    o, lse = decode_head(np.zeros((nq, d)), k, v, scale=1.0, causal=True)
    for i in range(nq):
        cnt = nk - nq + i + 1
        np.testing.assert_allclose(o[i], v[:cnt].mean(axis=0), rtol=1e-13, atol=1e-15)
        assert lse[i] == pytest.approx(math.log(cnt), rel=1e-13)
    # more queries than cached keys: the first Nq - Nk queries see nothing
    o, lse = decode_head(_rand(rng, 8, d), k[:3], v[:3], scale=1.0, causal=True)
    assert np.all(o[:5] == 0.0) and np.all(lse[:5] == -np.inf)
    assert np.all(np.isfinite(lse[5:]))


def test_batched_heads_subset():
    rng = np.random.default_rng(5)
    q, k, v = _rand(rng, 2, 3, 4, 8), _rand(rng, 2, 3, 10, 8), _rand(rng, 2, 3, 10, 8)
    r = decode(q, k, v, scale=0.5, causal=True, heads=[(1, 2)])
    o, lse = decode_head(q[1, 2], k[1, 2], v[1, 2], scale=0.5, causal=True)
    np.testing.assert_array_equal(r["o"][1, 2], o)
    assert np.isnan(r["o"][0, 0]).all()
