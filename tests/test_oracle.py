"""Pins for the CPU oracle: it is checked against things other than itself.

Each test names the pin it implements:
  golden   hand-derived values (tests/golden/*.json)
  P1       brute force in pure-Python loops (different arithmetic path)
  P2       the pages' softmax recurrences agree with each other
  P3       softmax rows are distributions, zero where masked
  P4-P7    closed forms for special inputs
  P8       invariants (sums of gradients, shifts, permutations)
  P9       central finite differences of L = sum(O * dO)
  P10      reductions of the block mask to dense attention
  lib      library routines (torch SDPA + autograd in fp64, scipy logsumexp)
"""
import ast
import json
import math
import operator
import os

import numpy as np
import pytest

from oracle import attention, attention_dq_rows, attention_head, attention_rows, softmax_rows
from oracle import softmax_forms as sf
from oracle.brute import attention_brute

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")

# ---------------------------------------------------------------------------------------------
# hand-derived fixtures


_OPS = {ast.Add: operator.add, ast.Sub: operator.sub, ast.Mult: operator.mul,
        ast.Div: operator.truediv, ast.USub: operator.neg, ast.UAdd: operator.pos}
_FUNCS = {"log": math.log, "exp": math.exp, "sqrt": math.sqrt}


def _ev(expr: str) -> float:
    """Evaluate a fixture expression: numbers, + - * /, log/exp/sqrt calls only."""
    def walk(n):
        if isinstance(n, ast.Expression):
            return walk(n.body)
        if isinstance(n, ast.Constant) and isinstance(n.value, (int, float)):
            return float(n.value)
        if isinstance(n, ast.BinOp) and type(n.op) in _OPS:
            return _OPS[type(n.op)](walk(n.left), walk(n.right))
        if isinstance(n, ast.UnaryOp) and type(n.op) in _OPS:
            return _OPS[type(n.op)](walk(n.operand))
        if isinstance(n, ast.Call) and isinstance(n.func, ast.Name) and n.func.id in _FUNCS:
            return _FUNCS[n.func.id](*[walk(a) for a in n.args])
        raise ValueError(f"unsupported fixture expression: {expr!r}")
    return walk(ast.parse(expr, mode="eval"))


def _arr(x):
    if isinstance(x, list):
        return np.array([_arr(e) for e in x], dtype=np.float64)
    return _ev(x)


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


@pytest.mark.parametrize("case", _load("hand_cases.json")["cases"], ids=lambda c: c["name"])
def test_golden_hand_cases(case):
    """golden: oracle reproduces every hand-derived value of the 2x2 cases."""
    q, k, v, do = (_arr(case[n]) for n in ("q", "k", "v", "do"))
    bm = None if case["block_mask"] is None else np.array(case["block_mask"], np.uint8)
    r = attention_head(q, k, v, do, scale=_ev(case["scale"]), causal=case["causal"],
                       block_mask=bm, block=case["block"])
    for key, exp in case["expect"].items():
        np.testing.assert_allclose(r[key], _arr(exp), rtol=1e-14, atol=1e-14, err_msg=key)
    # the same case through the brute force
    b = attention_brute(q.tolist(), k.tolist(), v.tolist(), do.tolist(), _ev(case["scale"]),
                        case["causal"], None if bm is None else bm.tolist(), case["block"])
    for key, exp in case["expect"].items():
        np.testing.assert_allclose(np.array(b[key]), _arr(exp), rtol=1e-14, atol=1e-14,
                                   err_msg="brute " + key)


def test_golden_online_softmax():
    """golden: the softmax recurrences hit every hand-derived intermediate value."""
    g = _load("online_softmax.json")
    x = _arr(g["x"])
    np.testing.assert_allclose(sf.three_pass(x), _arr(g["three_pass"]["softmax"]), rtol=1e-15)
    for blk, key in ((1, "online_normalizer_block1"), (2, "online_normalizer_block2")):
        ms, ds = sf.online_normalizer(x, blk)
        np.testing.assert_allclose(ms, _arr(g[key]["m"]), rtol=1e-15, atol=1e-15)
        np.testing.assert_allclose(ds, _arr(g[key]["d"]), rtol=1e-15)
    np.testing.assert_allclose(sf.two_pass(x, 1), _arr(g["three_pass"]["softmax"]), rtol=1e-15)
    V = _arr(g["one_pass_output"]["V"])
    for i, (o_exp, l_exp) in enumerate(zip(g["one_pass_output"]["o_after"],
                                           g["one_pass_output"]["l_after"])):
        o, _, l = sf.one_pass_output(x[: i + 1], V[: i + 1], block=1)
        assert o[0] == pytest.approx(_ev(o_exp), rel=1e-14)
        assert l == pytest.approx(_ev(l_exp), rel=1e-14)


# ---------------------------------------------------------------------------------------------
# helpers

def _rand(rng, n, d, nk=None, dv=None):
    nk = n if nk is None else nk
    dv = d if dv is None else dv
    return (rng.standard_normal((n, d)), rng.standard_normal((nk, d)),
            rng.standard_normal((nk, dv)), rng.standard_normal((n, dv)))


MASKS = ["none", "causal", "block", "causal+block"]


def _mask_args(kind, n, rng, block):
    causal = "causal" in kind
    bm = None
    if "block" in kind:
        nb = -(-n // block)
        bm = (rng.random((nb, nb)) < 0.5).astype(np.uint8)
        np.fill_diagonal(bm, 1)
    return causal, bm


# ---------------------------------------------------------------------------------------------
# P1 brute force

@pytest.mark.parametrize("kind", MASKS)
@pytest.mark.parametrize("n,d", [(1, 1), (5, 3), (9, 8), (16, 4), (13, 7)])
def test_p1_brute_force(kind, n, d):
    rng = np.random.default_rng(100 + n * 10 + d)
    q, k, v, do = _rand(rng, n, d)
    scale = 1.0 / math.sqrt(d)
    causal, bm = _mask_args(kind, n, rng, block=4)
    r = attention_head(q, k, v, do, scale=scale, causal=causal, block_mask=bm, block=4, chunk=3)
    b = attention_brute(q.tolist(), k.tolist(), v.tolist(), do.tolist(), scale, causal,
                        None if bm is None else bm.tolist(), 4)
    for key in ("o", "lse", "dq", "dk", "dv"):
        np.testing.assert_allclose(r[key], np.array(b[key]), rtol=1e-12, atol=1e-13, err_msg=key)


# ---------------------------------------------------------------------------------------------
# P2 softmax forms

@pytest.mark.parametrize("block", [1, 2, 3, 7, 50])
def test_p2_softmax_forms_agree(block):
    rng = np.random.default_rng(7)
    x = rng.standard_normal(50) * 4.0
    x[[3, 17]] = -np.inf   # masked entries
    ref = sf.three_pass(x)
    np.testing.assert_allclose(sf.two_pass(x, block), ref, rtol=1e-13, atol=1e-300)
    V = rng.standard_normal((50, 6))
    o_ref = ref @ V
    o1, m1, l1 = sf.one_pass_output(x, V, block)
    o2, m2, l2 = sf.one_pass_deferred(x, V, block)
    np.testing.assert_allclose(o1, o_ref, rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(o2, o_ref, rtol=1e-13, atol=1e-14)
    # final statistics equal the global max and denominator: LSE = m + ln l
    lse = m1 + math.log(l1)
    assert lse == pytest.approx(m2 + math.log(l2), rel=1e-14)
    finite = x[np.isfinite(x)]
    assert lse == pytest.approx(finite.max() + math.log(np.exp(finite - finite.max()).sum()),
                                rel=1e-14)


def test_row_softmax_pins():
    """The row-softmax oracle against the pinned forms, closed forms and its conventions."""
    rng = np.random.default_rng(11)
    x = rng.standard_normal((6, 37)) * 5.0
    x[1, [0, 5, 36]] = -np.inf
    x[4, :] = -np.inf                      # no finite entry: all zeros (reading)
    y = sf.row_softmax(x)
    for r in range(x.shape[0]):
        if r == 4:
            assert np.all(y[r] == 0.0)
            continue
        np.testing.assert_allclose(y[r], sf.three_pass(x[r]), rtol=1e-13, atol=1e-300)
        np.testing.assert_allclose(y[r], sf.two_pass(x[r], block=5), rtol=1e-13, atol=1e-300)
        assert y[r].sum() == pytest.approx(1.0, abs=1e-13)
    assert np.all(y[1, [0, 5, 36]] == 0.0)
    # closed forms: a constant row is uniform; [0, ln 2] -> [1/3, 2/3]; a -inf entry is 0
    np.testing.assert_allclose(sf.row_softmax(np.full((1, 9), 3.7)), np.full((1, 9), 1 / 9),
                               rtol=1e-15)
    np.testing.assert_allclose(sf.row_softmax([[0.0, math.log(2.0)]]), [[1 / 3, 2 / 3]],
                               rtol=1e-15)
    np.testing.assert_allclose(sf.row_softmax([[5.0, 5.0 + math.log(3.0), -np.inf]]),
                               [[0.25, 0.75, 0.0]], rtol=1e-15)
    # shift invariance per row, and a huge spread does not overflow
    np.testing.assert_allclose(sf.row_softmax(x[:4] + 1000.0), y[:4], rtol=1e-12, atol=1e-300)
    big = sf.row_softmax([[1000.0, 0.0, -1000.0]])
    assert big[0, 0] == pytest.approx(1.0) and np.all(np.isfinite(big))


def test_p2_online_matches_attention_row():
    """The one-pass recurrence over key blocks gives the oracle's O row and LSE."""
    rng = np.random.default_rng(8)
    q, k, v, _ = _rand(rng, 6, 5, nk=40)
    scale = 0.37
    for i in range(6):
        s = scale * (k @ q[i])
        o_r, lse_r = attention_rows(q, k, v, [i], scale=scale)
        for blk in (1, 4, 16, 40):
            o, m, l = sf.one_pass_deferred(s, v, blk)
            np.testing.assert_allclose(o, o_r[0], rtol=1e-13, atol=1e-14)
            assert m + math.log(l) == pytest.approx(lse_r[0], rel=1e-14)


# ---------------------------------------------------------------------------------------------
# P3 softmax rows

@pytest.mark.parametrize("kind", MASKS)
def test_p3_rows_are_distributions(kind):
    rng = np.random.default_rng(9)
    n, d = 40, 8
    q, k, _, _ = _rand(rng, n, d)
    causal, bm = _mask_args(kind, n, rng, block=8)
    rows = np.arange(n)
    p, lse = softmax_rows(q * 3, k, rows, scale=0.5, causal=causal, block_mask=bm, block=8)
    assert np.all(p >= 0)
    np.testing.assert_allclose(p.sum(axis=1), 1.0, rtol=0, atol=1e-14)
    from oracle import allowed
    assert np.all(p[~allowed(rows, n, causal, bm, 8)] == 0.0)


# ---------------------------------------------------------------------------------------------
# P4 zero Q

@pytest.mark.parametrize("causal", [False, True])
def test_p4_zero_q(causal):
    rng = np.random.default_rng(10)
    n, d = 24, 6
    _, k, v, do = _rand(rng, n, d)
    q = np.zeros((n, d))
    scale = 0.4
    r = attention_head(q, k, v, do, scale=scale, causal=causal, chunk=5)
    cnt = np.arange(1, n + 1) if causal else np.full(n, n)
    vis = np.tril(np.ones((n, n))) if causal else np.ones((n, n))
    mean_v = (vis @ v) / cnt[:, None]
    np.testing.assert_allclose(r["o"], mean_v, rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(r["lse"], np.log(cnt), rtol=1e-14)
    assert np.all(r["dk"] == 0.0)
    dv_exp = vis.T @ (do / cnt[:, None])
    np.testing.assert_allclose(r["dv"], dv_exp, rtol=1e-13, atol=1e-14)
    dq_exp = np.zeros((n, d))
    for i in range(n):
        js = np.nonzero(vis[i])[0]
        coef = (v[js] - r["o"][i]) @ do[i]
        dq_exp[i] = scale / cnt[i] * (coef @ k[js])
    np.testing.assert_allclose(r["dq"], dq_exp, rtol=1e-12, atol=1e-13)


# ---------------------------------------------------------------------------------------------
# P5 all K rows equal

def test_p5_equal_keys():
    rng = np.random.default_rng(11)
    n, d = 20, 5
    q, _, v, do = _rand(rng, n, d)
    kvec = rng.standard_normal(d)
    k = np.tile(kvec, (n, 1))
    scale = 0.7
    for causal in (False, True):
        r = attention_head(q, k, v, do, scale=scale, causal=causal)
        cnt = np.arange(1, n + 1) if causal else np.full(n, n)
        vis = np.tril(np.ones((n, n))) if causal else np.ones((n, n))
        np.testing.assert_allclose(r["o"], (vis @ v) / cnt[:, None], rtol=1e-13, atol=1e-14)
        np.testing.assert_allclose(r["lse"], scale * q @ kvec + np.log(cnt), rtol=1e-13)
        np.testing.assert_allclose(r["dq"], 0.0, atol=1e-13)


# ---------------------------------------------------------------------------------------------
# P6 special V

def test_p6_identity_and_ones_v():
    rng = np.random.default_rng(12)
    n = 16
    q, k, _, _ = _rand(rng, n, n)
    scale = 0.3
    for causal in (False, True):
        p, _ = softmax_rows(q, k, np.arange(n), scale=scale, causal=causal, block_mask=None,
                            block=128)
        r = attention_head(q, k, np.eye(n), scale=scale, causal=causal)
        np.testing.assert_allclose(r["o"], p, rtol=1e-14, atol=1e-16)
        r1 = attention_head(q, k, np.ones((n, 3)), scale=scale, causal=causal)
        np.testing.assert_allclose(r1["o"], 1.0, rtol=1e-14)


# ---------------------------------------------------------------------------------------------
# P7 trivial rows

def test_p7_single_row_and_causal_row0():
    rng = np.random.default_rng(13)
    q, k, v, do = _rand(rng, 1, 4)
    r = attention_head(q, k, v, do, scale=0.5)
    np.testing.assert_array_equal(r["o"], v)
    assert r["lse"][0] == pytest.approx(0.5 * float(q[0] @ k[0]), rel=1e-15)
    assert np.all(r["dq"] == 0) and np.all(r["dk"] == 0)
    np.testing.assert_array_equal(r["dv"], do)
    q, k, v, do = _rand(rng, 10, 4)
    r = attention_head(q, k, v, do, scale=0.5, causal=True)
    np.testing.assert_array_equal(r["o"][0], v[0])
    assert r["lse"][0] == pytest.approx(0.5 * float(q[0] @ k[0]), rel=1e-15)


# ---------------------------------------------------------------------------------------------
# P8 invariants

@pytest.mark.parametrize("kind", MASKS)
def test_p8_gradient_sums(kind):
    rng = np.random.default_rng(14)
    n, d = 32, 8
    q, k, v, do = _rand(rng, n, d)
    causal, bm = _mask_args(kind, n, rng, block=8)
    r = attention_head(q, k, v, do, scale=0.35, causal=causal, block_mask=bm, block=8, chunk=7)
    # every dS row sums to zero, hence sum_j dK_j = scale * sum_i (sum_j dS_ij) Q_i = 0
    np.testing.assert_allclose(r["dk"].sum(axis=0), 0.0, atol=1e-12)
    # every P row sums to one, hence sum_j dV_j = sum_i dO_i
    np.testing.assert_allclose(r["dv"].sum(axis=0), do.sum(axis=0), rtol=1e-12, atol=1e-12)
    # D_i = sum_j P_ij dP_ij equals dO_i . O_i
    np.testing.assert_allclose(r["D"], (do * r["o"]).sum(axis=1), rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("kind", MASKS)
def test_p8_key_shift(kind):
    rng = np.random.default_rng(15)
    n, d = 24, 6
    q, k, v, do = _rand(rng, n, d)
    causal, bm = _mask_args(kind, n, rng, block=8)
    u = rng.standard_normal(d)
    scale = 0.45
    a = attention_head(q, k, v, do, scale=scale, causal=causal, block_mask=bm, block=8)
    b = attention_head(q, k + u, v, do, scale=scale, causal=causal, block_mask=bm, block=8)
    for key in ("o", "dq", "dv", "dk"):
        np.testing.assert_allclose(b[key], a[key], rtol=1e-11, atol=1e-12, err_msg=key)
    np.testing.assert_allclose(b["lse"], a["lse"] + scale * q @ u, rtol=1e-13)


def test_p8_key_permutation():
    rng = np.random.default_rng(16)
    n, d = 24, 6
    q, k, v, do = _rand(rng, n, d)
    perm = rng.permutation(n)
    a = attention_head(q, k, v, do, scale=0.4)
    b = attention_head(q, k[perm], v[perm], do, scale=0.4)
    for key in ("o", "lse", "dq"):
        np.testing.assert_allclose(b[key], a[key], rtol=1e-12, atol=1e-13, err_msg=key)
    np.testing.assert_allclose(b["dk"], a["dk"][perm], rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(b["dv"], a["dv"][perm], rtol=1e-12, atol=1e-13)


# ---------------------------------------------------------------------------------------------
# P9 finite differences

def _loss(q, k, v, do, **kw):
    return float((attention_head(q, k, v, **kw)["o"] * do).sum())


@pytest.mark.parametrize("kind", MASKS)
def test_p9_finite_differences_every_entry(kind):
    rng = np.random.default_rng(17)
    n, d = 8, 4
    q, k, v, do = _rand(rng, n, d)
    causal, bm = _mask_args(kind, n, rng, block=2)
    kw = dict(scale=0.6, causal=causal, block_mask=bm, block=2)
    r = attention_head(q, k, v, do, **kw)
    h = 1e-6
    for name, x in (("dq", q), ("dk", k), ("dv", v)):
        g = np.zeros_like(x)
        for idx in np.ndindex(*x.shape):
            orig = x[idx]
            x[idx] = orig + h
            lp = _loss(q, k, v, do, **kw)
            x[idx] = orig - h
            lm = _loss(q, k, v, do, **kw)
            x[idx] = orig
            g[idx] = (lp - lm) / (2 * h)
        err = np.linalg.norm(g - r[name]) / max(np.linalg.norm(r[name]), 1e-300)
        assert err <= 1e-6, (name, err)


def test_p9_finite_differences_sampled():
    rng = np.random.default_rng(18)
    n, d = 64, 16
    q, k, v, do = _rand(rng, n, d)
    kw = dict(scale=0.25, causal=True)
    r = attention_head(q, k, v, do, **kw)
    h = 1e-6
    for name, x in (("dq", q), ("dk", k), ("dv", v)):
        picks = [tuple(rng.integers(0, s) for s in x.shape) for _ in range(22)]
        num, ref = [], []
        for idx in picks:
            orig = x[idx]
            x[idx] = orig + h
            lp = _loss(q, k, v, do, **kw)
            x[idx] = orig - h
            lm = _loss(q, k, v, do, **kw)
            x[idx] = orig
            num.append((lp - lm) / (2 * h))
            ref.append(r[name][idx])
        num, ref = np.array(num), np.array(ref)
        assert np.linalg.norm(num - ref) / np.linalg.norm(ref) <= 1e-6, name


# ---------------------------------------------------------------------------------------------
# P10 block-mask reductions

def test_p10_all_ones_block_mask_is_dense():
    rng = np.random.default_rng(19)
    n, d = 64, 8
    q, k, v, do = _rand(rng, n, d)
    bm = np.ones((4, 4), np.uint8)
    a = attention_head(q, k, v, do, scale=0.3, block_mask=bm, block=16)
    b = attention_head(q, k, v, do, scale=0.3)
    for key in a:
        np.testing.assert_array_equal(a[key], b[key])


def test_p10_diagonal_block_mask_is_independent_sequences():
    rng = np.random.default_rng(20)
    n, d, blk = 64, 8, 16
    q, k, v, do = _rand(rng, n, d)
    bm = np.eye(n // blk, dtype=np.uint8)
    a = attention_head(q, k, v, do, scale=0.3, block_mask=bm, block=blk)
    for s in range(n // blk):
        sl = slice(s * blk, (s + 1) * blk)
        b = attention_head(q[sl], k[sl], v[sl], do[sl], scale=0.3)
        for key in ("o", "lse", "dq", "dk", "dv"):
            np.testing.assert_allclose(a[key][sl], b[key], rtol=1e-12, atol=1e-13, err_msg=key)


# ---------------------------------------------------------------------------------------------
# library routines

@pytest.mark.parametrize("kind", MASKS)
def test_lib_torch_sdpa_and_autograd(kind):
    """torch's own attention (math path, fp64, CPU) and its autograd agree with the oracle."""
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(21)
    B, H, n, d = 2, 3, 48, 16
    q = rng.standard_normal((B, H, n, d))
    k = rng.standard_normal((B, H, n, d))
    v = rng.standard_normal((B, H, n, d))
    do = rng.standard_normal((B, H, n, d))
    causal, bm = _mask_args(kind, n, rng, block=16)
    scale = 1.0 / math.sqrt(d)
    r = attention(q, k, v, do, scale=scale, causal=causal, block_mask=bm, block=16, chunk=20)
    from oracle import allowed
    ok = torch.from_numpy(allowed(np.arange(n), n, causal, bm, 16))
    tq, tk, tv = (torch.from_numpy(x.copy()).requires_grad_(True) for x in (q, k, v))
    o = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=ok, scale=scale)
    o.backward(torch.from_numpy(do))
    np.testing.assert_allclose(r["o"], o.detach().numpy(), rtol=1e-12, atol=1e-12)
    for key, t in (("dq", tq), ("dk", tk), ("dv", tv)):
        np.testing.assert_allclose(r[key], t.grad.numpy(), rtol=1e-11, atol=1e-12, err_msg=key)
    # logsumexp of the scaled, masked scores
    from scipy.special import logsumexp
    s = scale * np.einsum("bhid,bhjd->bhij", q, k)
    s = np.where(ok.numpy(), s, -np.inf)
    np.testing.assert_allclose(r["lse"], logsumexp(s, axis=-1), rtol=1e-13)


# ---------------------------------------------------------------------------------------------
# chunking, sampling helpers, edge conventions

def test_chunking_does_not_change_results():
    rng = np.random.default_rng(22)
    n, d = 37, 5
    q, k, v, do = _rand(rng, n, d)
    ref = attention_head(q, k, v, do, scale=0.5, causal=True, chunk=n)
    for chunk in (1, 6, 20):
        r = attention_head(q, k, v, do, scale=0.5, causal=True, chunk=chunk)
        for key in ref:
            np.testing.assert_allclose(r[key], ref[key], rtol=1e-13, atol=1e-14, err_msg=key)


def test_row_samplers_match_full_head():
    rng = np.random.default_rng(23)
    n, d = 50, 6
    q, k, v, do = _rand(rng, n, d)
    bm = (rng.random((5, 5)) < 0.5).astype(np.uint8)
    np.fill_diagonal(bm, 1)
    kw = dict(scale=0.5, causal=True, block_mask=bm, block=10)
    full = attention_head(q, k, v, do, **kw)
    rows = [0, 7, 19, 49]
    o, lse = attention_rows(q, k, v, rows, **kw)
    np.testing.assert_allclose(o, full["o"][rows], rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(lse, full["lse"][rows], rtol=1e-14)
    dq = attention_dq_rows(q, k, v, do, rows, **kw)
    np.testing.assert_allclose(dq, full["dq"][rows], rtol=1e-12, atol=1e-13)


def test_empty_row_convention():
    """A row with no visible key: O = 0, LSE = -inf, no gradient in or out."""
    rng = np.random.default_rng(24)
    n, d = 8, 4
    q, k, v, do = _rand(rng, n, d)
    bm = np.array([[1, 0], [0, 0]], np.uint8)   # rows 4..7 see nothing
    r = attention_head(q, k, v, do, scale=0.5, block_mask=bm, block=4)
    assert np.all(r["o"][4:] == 0) and np.all(np.isneginf(r["lse"][4:]))
    assert np.all(r["dq"][4:] == 0)
    assert np.all(r["dk"][4:] == 0) and np.all(r["dv"][4:] == 0)
    assert np.all(np.isfinite(r["dq"])) and np.all(np.isfinite(r["o"]))


def test_batched_heads_subset():
    rng = np.random.default_rng(25)
    q, k, v, do = (rng.standard_normal((2, 2, 12, 4)) for _ in range(4))
    full = attention(q, k, v, do, scale=0.5)
    part = attention(q, k, v, do, scale=0.5, heads=[(1, 0)])
    for key in full:
        np.testing.assert_array_equal(part[key][1, 0], full[key][1, 0])
        assert np.all(np.isnan(part[key][0, 0]))
