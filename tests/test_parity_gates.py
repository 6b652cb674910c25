"""CPU checks of the GPU parity gates themselves (tests/gpu_util.py).

An emulation of the kernels' roundings must pass them: O, dQ, dK, dV rounded
once to bf16, and D_i = dO_i . O_i formed from the bf16-rounded O as the
backward does. That includes peaked scores, where one key dominates most rows
and the dK rows of those keys are small differences (the case the dK rounding
floor is for). Planted structural mistakes of the kind the gates exist to
catch (a key group's half of dK dropped, a tile missing from dQ or O, a missed
scale) must fail them.
"""
import math

import numpy as np
import pytest
import torch

from exact_io_aware_61_amd.workloads import make_qkv
from oracle.attention import softmax_rows
from tests.gpu_util import assert_parity, run_oracle

B, H, N, D = 1, 2, 200, 64
SCALE = float(np.float32(1 / math.sqrt(D)))


def _inputs(peaked):
    q, k, v, do = make_qkv(B, H, N, D, seed=4242)
    if peaked:
        q = (q.float() * 4).to(torch.bfloat16)
        k = (k.float() * 4).to(torch.bfloat16)
        v = (v.float() * 0.5).to(torch.bfloat16)
    return q, k, v, do


def _emulated(q, k, v, do, causal, drop_tile=None):
    """fp64 attention with the kernels' roundings; drop_tile = (tensor, first key) leaves
    out the 64 keys starting there from that output."""
    out = {n: np.zeros((B, H, N, D)) for n in ("o", "dq", "dk", "dv")}
    out["lse"] = np.zeros((B, H, N))
    for h in range(H):
        qh, kh, vh, doh = (t.double().numpy()[0, h] for t in (q, k, v, do))
        p, lse = softmax_rows(qh, kh, np.arange(N), scale=SCALE, causal=causal, block_mask=None,
                              block=128)
        o = p @ vh
        ob = torch.tensor(o).to(torch.bfloat16).double().numpy()
        ds = p * (doh @ vh.T - (doh * ob).sum(axis=1)[:, None])
        res = {"o": o, "dq": SCALE * ds @ kh, "dk": SCALE * ds.T @ qh, "dv": p.T @ doh}
        if drop_tile is not None:
            name, j0 = drop_tile
            keep = np.ones(N, bool)
            keep[j0:j0 + 64] = False
            if name == "o":
                res["o"] = p[:, keep] @ vh[keep]
            if name == "dq":
                res["dq"] = SCALE * ds[:, keep] @ kh[keep]
        for n in ("o", "dq", "dk", "dv"):
            out[n][0, h] = res[n]
        out["lse"][0, h] = lse
    gpu = {n: torch.tensor(out[n]).to(torch.bfloat16) for n in ("o", "dq", "dk", "dv")}
    gpu["lse"] = torch.tensor(out["lse"]).float()
    return gpu


@pytest.mark.parametrize("peaked", [False, True])
@pytest.mark.parametrize("causal", [False, True])
def test_emulated_roundings_pass(peaked, causal):
    q, k, v, do = _inputs(peaked)
    ref = run_oracle(q, k, v, do, causal=causal, scale=SCALE)
    e = assert_parity(_emulated(q, k, v, do, causal), ref, label="emulated")
    if peaked:
        assert "dk_row_plain" in e   # the plain dK row figure fails here; the floor decides


@pytest.mark.parametrize("peaked", [False, True])
def test_planted_mistakes_fail(peaked):
    q, k, v, do = _inputs(peaked)
    ref = run_oracle(q, k, v, do, causal=True, scale=SCALE)
    good = _emulated(q, k, v, do, True)
    cases = {}
    half = {n: t.clone() for n, t in good.items()}
    half["dk"][0, 1, 64:96] *= 0.5          # one 32-key group's dK half missing
    cases["dk half of a key group"] = half
    cases["dq tile missing"] = _emulated(q, k, v, do, True, drop_tile=("dq", 64))
    cases["o tile missing"] = _emulated(q, k, v, do, True, drop_tile=("o", 0))
    noscale = {n: t.clone() for n, t in good.items()}
    noscale["dk"] = (noscale["dk"].double() / SCALE).to(torch.bfloat16)   # scale left out
    cases["dk scale missing"] = noscale
    for name, gpu in cases.items():
        with pytest.raises(AssertionError):
            assert_parity(gpu, ref, label=name)
