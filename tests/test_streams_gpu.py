"""Independent calls on two streams at once.

The library keeps no state between calls (fa_bwd_noalloc's fixed array aside,
whose overlapping calls are documented to race and are not made here), so a
forward and backward on one stream must not disturb another running on a
second stream at the same time. Two problems of different shapes are
enqueued alternately on two streams of default priority, several times over,
and each result is compared bitwise with the same call made alone.
"""
import math

import numpy as np
import pytest
import torch

import exact_io_aware_61_amd as fa
from exact_io_aware_61_amd.workloads import make_qkv

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


def _problem(B, H, N, d, seed):
    return [t.to(DEV) for t in make_qkv(B, H, N, d, seed)]


def _step(q, k, v, do, causal):
    scale = float(np.float32(1 / math.sqrt(q.shape[-1])))
    o, lse = fa.forward(q, k, v, causal=causal, scale=scale)
    dq, dk, dv = fa.backward(q, k, v, o, lse, do, causal=causal, scale=scale)
    return o, lse, dq, dk, dv


def test_two_streams_match_serial_calls():
    print("[case] two streams: B2 H8 N1500 d128 causal and B4 H4 N777 d64", flush=True)
    a = _problem(2, 8, 1500, 128, 1200)
    b = _problem(4, 4, 777, 64, 1201)
    ref_a = _step(*a, causal=True)
    ref_b = _step(*b, causal=False)
    torch.cuda.synchronize()
    s1, s2 = torch.cuda.Stream(DEV), torch.cuda.Stream(DEV)
    for t in a + b:
        t.record_stream(s1)
        t.record_stream(s2)
    outs = []
    for _ in range(3):
        with torch.cuda.stream(s1):
            ra = _step(*a, causal=True)
        with torch.cuda.stream(s2):
            rb = _step(*b, causal=False)
        outs.append((ra, rb))
    torch.cuda.synchronize()
    for ra, rb in outs:
        for x, y in zip(ra, ref_a):
            assert torch.equal(x, y)
        for x, y in zip(rb, ref_b):
            assert torch.equal(x, y)
