"""Plant plausible mistakes in copies of the oracle and check that the pins catch each one.

Every mutant is the oracle's own source with one textual change, loaded as a
separate module on the CPU; the real oracle is never modified. A mutant
"survives" if all three independent pins pass on it - hand-derived values,
the pure-Python brute force, and finite differences - which would mean the
pins could not tell that mistake from the definition.
"""
import math
import os
import types

import numpy as np
import pytest

from oracle.brute import attention_brute
from tests.test_oracle import _arr, _ev, _load

SRC = os.path.join(os.path.dirname(os.path.dirname(__file__)), "oracle", "attention.py")

MUTANTS = {
    "dV uses P instead of P^T": ("out[\"dv\"] += p.T @ dor", "out[\"dv\"] += p[:, :p.shape[0]] @ dor"),
    "dropped D term": ("            ds = p * (dp - dvec[:, None])", "            ds = p * dp"),
    "wrong sign of D": ("            ds = p * (dp - dvec[:, None])",
                        "            ds = p * (dp + dvec[:, None])"),
    "dQ missing scale": ("out[\"dq\"][rows] = scale * (ds @ k)", "out[\"dq\"][rows] = ds @ k"),
    "dK uses dS not dS^T": ("out[\"dk\"] += scale * (ds.T @ q[rows])",
                            "out[\"dk\"] += scale * (ds[:, :ds.shape[0]] @ q[rows])"),
    "causal off by one": ("a &= cols[None, :] <= rows[:, None]", "a &= cols[None, :] < rows[:, None]"),
    "block mask transposed": ("a &= bm[(rows // block)[:, None], (cols // block)[None, :]]",
                              "a &= bm.T[(rows // block)[:, None], (cols // block)[None, :]]"),
    "LSE without max": ("lse = np.where(empty, -np.inf, m_safe + np.log(np.where(empty, 1.0, l)))",
                        "lse = np.where(empty, -np.inf, np.log(np.where(empty, 1.0, l)))"),
    "scale outside softmax": ("s = np.where(ok, scale * (q_rows @ k.T), -np.inf)",
                              "s = np.where(ok, q_rows @ k.T, -np.inf)"),
    "no normalisation": ("p = e / np.where(empty, 1.0, l)[:, None]", "p = e"),
}


def _mutant(old, new):
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation anchor not found exactly once: {old!r}"
    mod = types.ModuleType("oracle_mutant")
    exec(compile(src.replace(old, new), "oracle_mutant", "exec"), mod.__dict__)
    return mod


def _pins_pass(mod) -> bool:
    """True if the mutant passes every pin check below."""
    try:
        for case in _load("hand_cases.json")["cases"]:
            q, k, v, do = (_arr(case[n]) for n in ("q", "k", "v", "do"))
            bm = None if case["block_mask"] is None else np.array(case["block_mask"], np.uint8)
            r = mod.attention_head(q, k, v, do, scale=_ev(case["scale"]), causal=case["causal"],
                                   block_mask=bm, block=case["block"])
            for key, exp in case["expect"].items():
                np.testing.assert_allclose(r[key], _arr(exp), rtol=1e-12, atol=1e-12)
        rng = np.random.default_rng(5)
        for causal, use_bm in ((False, False), (True, False), (False, True)):
            n, d = 12, 4
            q, k, v, do = (rng.standard_normal((n, d)) for _ in range(4))
            bm = None
            if use_bm:
                bm = np.array([[1, 1, 0], [0, 1, 0], [1, 0, 1]], np.uint8)
            r = mod.attention_head(q, k, v, do, scale=0.5, causal=causal, block_mask=bm, block=4)
            b = attention_brute(q.tolist(), k.tolist(), v.tolist(), do.tolist(), 0.5, causal,
                                None if bm is None else bm.tolist(), 4)
            for key in ("o", "lse", "dq", "dk", "dv"):
                np.testing.assert_allclose(r[key], np.array(b[key]), rtol=1e-10, atol=1e-10)
            # finite differences against the mutant's own forward
            h = 1e-6
            for name, x in (("dq", q), ("dk", k), ("dv", v)):
                idx = (3, 1)
                orig = x[idx]
                x[idx] = orig + h
                lp = float((mod.attention_head(q, k, v, scale=0.5, causal=causal,
                                               block_mask=bm, block=4)["o"] * do).sum())
                x[idx] = orig - h
                lm = float((mod.attention_head(q, k, v, scale=0.5, causal=causal,
                                               block_mask=bm, block=4)["o"] * do).sum())
                x[idx] = orig
                g = (lp - lm) / (2 * h)
                assert math.isclose(g, r[name][idx], rel_tol=1e-5, abs_tol=1e-8)
    except AssertionError:
        return False
    return True


def test_unmutated_source_passes():
    assert _pins_pass(_mutant("import numpy as np", "import numpy as np"))


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name):
    old, new = MUTANTS[name]
    assert not _pins_pass(_mutant(old, new)), f"pins did not catch: {name}"
