"""Helpers shared by the GPU parity tests: run the HIP path, run the oracle, compare.

Tolerances (bf16 inputs, fp32 accumulation): O max-abs <= 1e-2, LSE max-abs
<= 1e-3, dQ/dK/dV relative Frobenius error <= 2e-2, each over the whole
compared tensor.
"""
from __future__ import annotations

import json
import os

import numpy as np
import torch

import exact_io_aware_61_amd as fa
from oracle import attention as oracle_attention

TOL_O = 1e-2
TOL_LSE = 1e-3
TOL_GRAD = 2e-2


def to64(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu", torch.float64).numpy()


def run_gpu(q, k, v, do, *, causal=False, block_mask=None, scale=None, with_bwd=True):
    """Forward (+ backward) through the C ABI on cuda:0. Inputs: CPU bf16 tensors."""
    dev = torch.device("cuda:0")
    qg, kg, vg = (t.to(dev) for t in (q, k, v))
    o, lse = fa.forward(qg, kg, vg, causal=causal, block_mask=block_mask, scale=scale)
    out = {"o": o, "lse": lse}
    if with_bwd:
        dq, dk, dv = fa.backward(qg, kg, vg, o, lse, do.to(dev), causal=causal,
                                 block_mask=block_mask, scale=scale)
        out.update(dq=dq, dk=dk, dv=dv)
    torch.cuda.synchronize()
    return out


def run_oracle(q, k, v, do, *, causal=False, block_mask=None, scale, heads=None):
    return oracle_attention(to64(q), to64(k), to64(v), None if do is None else to64(do),
                            scale=scale, causal=causal, block_mask=block_mask, heads=heads)


def errors(gpu: dict, ref: dict, heads=None):
    """Error metrics of the GPU result against the oracle (optionally on some heads only)."""
    sel = (lambda x: x) if heads is None else (lambda x: np.stack([x[b, h] for b, h in heads]))
    res = {}
    o_g, o_r = sel(to64(gpu["o"])), sel(ref["o"])
    res["o_maxabs"] = float(np.abs(o_g - o_r).max()) if o_r.size else 0.0
    l_g, l_r = sel(to64(gpu["lse"])), sel(ref["lse"])
    fin = np.isfinite(l_r)
    res["lse_inf_match"] = bool(np.array_equal(np.isneginf(l_g), np.isneginf(l_r)))
    res["lse_maxabs"] = float(np.abs(l_g[fin] - l_r[fin]).max()) if fin.any() else 0.0
    for key in ("dq", "dk", "dv"):
        if key in gpu and key in ref:
            g, r = sel(to64(gpu[key])), sel(ref[key])
            nr = np.linalg.norm(r)
            res[key + "_rel"] = float(np.linalg.norm(g - r) / nr) if nr > 0 else float(
                np.linalg.norm(g))
    return res


def assert_parity(gpu: dict, ref: dict, heads=None, label=""):
    e = errors(gpu, ref, heads)
    print(f"[parity] {label} {e}", flush=True)
    log = os.environ.get("FA_PARITY_LOG")
    if log:
        with open(log, "a") as f:
            f.write(json.dumps({"case": label, **e}) + "\n")
    assert e["o_maxabs"] <= TOL_O, (label, e)
    assert e["lse_inf_match"], (label, e)
    assert e["lse_maxabs"] <= TOL_LSE, (label, e)
    for key in ("dq_rel", "dk_rel", "dv_rel"):
        if key in e:
            assert e[key] <= TOL_GRAD, (label, key, e)
    return e
