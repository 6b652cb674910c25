"""The path captured in a HIP graph and replayed.

The kernels take their stream from the caller and allocate nothing when the
caller supplies every output and the workspace, so a whole training step
(forward, then the three backward stages) or a decoding step can be recorded
once with torch.cuda.graph and replayed. Each test replays the graph several
times with new inputs copied in between (eager work and synchronisations
between the replays), and compares every replay bitwise with eager calls on the
same inputs: the kernels are deterministic, so the two must agree exactly.
"""
import ctypes
import math

import numpy as np
import pytest
import torch

import exact_io_aware_61_amd as fa
from exact_io_aware_61_amd.workloads import make_block_mask, make_qkv

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


def _capture(fn):
    """Record fn() into a graph after one warm-up call on a side stream."""
    side = torch.cuda.Stream(DEV)
    side.wait_stream(torch.cuda.current_stream(DEV))
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream(DEV).wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


@pytest.mark.parametrize("d,causal,block", [(128, True, False), (64, False, True)])
def test_training_step_replays_bitwise(d, causal, block):
    B, H, N = 2, 4, 1000   # ragged: N is no multiple of any tile
    print(f"[case] graph replay of forward+backward: B{B} H{H} N{N} d{d} causal={causal} "
          f"block={block}", flush=True)
    scale = float(np.float32(1 / math.sqrt(d)))
    q, k, v, do = (t.to(DEV) for t in make_qkv(B, H, N, d, 900))
    bm = None
    if block:   # already a device uint8 grid: the binding then copies nothing
        bm = torch.as_tensor(make_block_mask(N, 0.5, 901)).to(DEV, torch.uint8).contiguous()
    o, dq, dk, dv = (torch.empty_like(q) for _ in range(4))
    lse = torch.empty((B, H, N), device=DEV, dtype=torch.float32)
    ws = fa.workspace(q)

    def step():
        fa.forward(q, k, v, causal=causal, block_mask=bm, scale=scale, out=o, lse=lse)
        fa.backward(q, k, v, o, lse, do, causal=causal, block_mask=bm, scale=scale, ws=ws,
                    dq=dq, dk=dk, dv=dv)

    g = _capture(step)
    for rep in range(3):
        nq, nk, nv, ndo = (t.to(DEV) for t in make_qkv(B, H, N, d, 910 + rep))
        q.copy_(nq)
        k.copy_(nk)
        v.copy_(nv)
        do.copy_(ndo)
        g.replay()
        torch.cuda.synchronize()
        got = {"o": o.clone(), "lse": lse.clone(), "dq": dq.clone(), "dk": dk.clone(),
               "dv": dv.clone()}
        eo, e_lse = fa.forward(q, k, v, causal=causal, block_mask=bm, scale=scale)
        edq, edk, edv = fa.backward(q, k, v, eo, e_lse, do, causal=causal, block_mask=bm,
                                    scale=scale)
        torch.cuda.synchronize()
        ref = {"o": eo, "lse": e_lse, "dq": edq, "dk": edk, "dv": edv}
        for name in ref:
            assert torch.equal(got[name], ref[name]), (rep, name)
        # the inputs changed between replays, so the outputs must too
        if rep > 0:
            assert not torch.equal(got["o"], prev_o)
        prev_o = got["o"]


def test_decoding_step_replays_bitwise():
    B, H, Nq, Nk, d = 2, 8, 4, 3000, 128
    print(f"[case] graph replay of decoding: B{B} H{H} Nq{Nq} Nk{Nk} d{d} causal", flush=True)
    g0 = torch.Generator().manual_seed(920)
    mk = lambda n: torch.randn((B, H, n, d), generator=g0).to(torch.bfloat16).to(DEV)  # noqa: E731
    q, k, v = mk(Nq), mk(Nk), mk(Nk)
    n = ctypes.c_size_t()
    assert fa.load().fa_decode_workspace_size(B, H, Nq, Nk, d, ctypes.byref(n)) == 0
    ws = torch.empty(max(n.value, 16), device=DEV, dtype=torch.uint8)
    out = {}

    def step():
        out["o"], out["lse"] = fa.decode(q, k, v, causal=True, ws=ws)

    g = _capture(step)
    for rep in range(3):
        q.copy_(mk(Nq))
        k.copy_(mk(Nk))
        v.copy_(mk(Nk))
        g.replay()
        torch.cuda.synchronize()
        got_o, got_lse = out["o"].clone(), out["lse"].clone()
        eo, e_lse = fa.decode(q, k, v, causal=True)
        torch.cuda.synchronize()
        assert torch.equal(got_o, eo), rep
        assert torch.equal(got_lse, e_lse), rep
