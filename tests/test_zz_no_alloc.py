"""fa_bwd_noalloc: the backward with its workspace in the library's fixed device array.

Called through the C ABI (ctypes) and compared with fa_bwd, which takes a
caller-allocated workspace and runs the same kernels: the outputs must be
bitwise equal. Two calls in a row, the second on a smaller problem, so the
second call runs over what the first left in the shared array. Sizes beyond
the array are refused on the host before anything is enqueued.
"""
import ctypes
import math

import numpy as np
import pytest
import torch

import exact_io_aware_61_amd as fa
from exact_io_aware_61_amd.workloads import make_block_mask, make_qkv

pytestmark = pytest.mark.gpu

FA_ERR_SCRATCH = -9


def _call_both(B, H, N, d, causal, block, seed):
    lib = fa.load()
    dev = torch.device("cuda:0")
    q, k, v, do = (t.to(dev) for t in make_qkv(B, H, N, d, seed))
    scale = float(np.float32(1 / math.sqrt(d)))
    bm = make_block_mask(N, 0.5, seed + 1) if block else None
    o, lse = fa.forward(q, k, v, causal=causal, block_mask=bm, scale=scale)
    ref = fa.backward(q, k, v, o, lse, do, causal=causal, block_mask=bm, scale=scale)
    got = [torch.full_like(q, float("nan")) for _ in range(3)]
    mptr, keep = fa._binding._mask(causal, bm, B, H, N, dev)
    P = lambda t: ctypes.c_void_p(t.data_ptr())  # noqa: E731
    stream = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
    rc = lib.fa_bwd_noalloc(P(q), P(k), P(v), P(o), P(do), P(lse), P(got[0]), P(got[1]),
                            P(got[2]), B, H, N, d, ctypes.c_float(scale), mptr, stream)
    torch.cuda.synchronize()
    del keep
    assert rc == 0, fa.strerror(rc)
    for name, a, b in zip(("dq", "dk", "dv"), got, ref):
        assert torch.equal(a, b), name


@pytest.mark.parametrize("causal,block", [(True, False), (False, True)])
def test_noalloc_matches_fa_bwd_twice_second_smaller(causal, block):
    print(f"[case] no-alloc backward causal={causal} block={block}: B2 H8 N1000 d128, "
          f"then B1 H3 N333 d64", flush=True)
    _call_both(2, 8, 1000, 128, causal, block, seed=77)
    _call_both(1, 3, 333, 64, causal, block, seed=78)


def test_noalloc_refuses_problems_beyond_its_scratch():
    lib = fa.load()
    # B*H*ceil(N/128)*128 = 2^21 + 128 rows: one row block too many. Rejected on the
    # host from the sizes alone (the pointers are never used).
    p = ctypes.c_void_p(256)
    rc = lib.fa_bwd_noalloc(p, p, p, p, p, p, p, p, p, 1, 1, (1 << 21) + 1, 64,
                            ctypes.c_float(0.125), None, None)
    assert rc == FA_ERR_SCRATCH
    assert "scratch" in fa.strerror(rc)
