"""GPU parity at the tile edges of every kernel, against the CPU fp64 oracle.

The kernels cut the sequence into 64-key tiles (forward, dQ at d=128 or with a
block mask), 32-key tiles (dQ at d=64 without a mask), 128- and 256-row
workgroups (forward, dQ), 128-key workgroups (dK/dV) and 64-row blocks (dK/dV).
Each length below sits on or next to one of those edges, so a tail that is one
row, one key or one block long, or a tile that is exactly full, is compared
element by element with the oracle on every head. A second set does the same
with a block mask, and a third with peaked scores (Q and K scaled by 4, exact in
bf16), where most rows are dominated by a single key. There O is close to one V
row, so V is halved (exact) to keep |O| below 4: at |O| >= 4 half a bf16 unit in
the last place is 2^-6, above the 1e-2 max-abs bar, and even the correctly
rounded O would fail it.
"""
import math

import numpy as np
import pytest
import torch

import exact_io_aware_61_amd as fa
from exact_io_aware_61_amd.workloads import make_block_mask, make_qkv
from tests.gpu_util import assert_parity, run_gpu, run_oracle

pytestmark = pytest.mark.gpu

EDGE_N = [31, 32, 33, 63, 64, 127, 128, 255, 257, 383, 511, 512, 767, 769]


@pytest.fixture(scope="module", autouse=True)
def _lib():
    fa.load()
    torch.cuda.init()


def _scale(d):
    return float(np.float32(1 / math.sqrt(d)))


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N", EDGE_N)
def test_tile_edges(N, causal, d):
    q, k, v, do = make_qkv(1, 2, N, d, seed=9500 + N + d)
    print(f"[case] tile edge N={N} d={d} causal={causal}", flush=True)
    gpu = run_gpu(q, k, v, do, causal=causal, scale=_scale(d))
    ref = run_oracle(q, k, v, do, causal=causal, scale=_scale(d))
    assert_parity(gpu, ref, label=f"edge N={N} d={d} causal={causal}")


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("N", [127, 129, 255, 257, 383, 640])
def test_tile_edges_block_mask(N, d):
    causal = N % 2 == 1
    q, k, v, do = make_qkv(2, 2, N, d, seed=9700 + N + d)
    bm = make_block_mask(N, 0.5, seed=9800 + N)
    print(f"[case] tile edge with block mask N={N} d={d} causal={causal}", flush=True)
    gpu = run_gpu(q, k, v, do, causal=causal, block_mask=bm, scale=_scale(d))
    ref = run_oracle(q, k, v, do, causal=causal, block_mask=bm, scale=_scale(d))
    assert_parity(gpu, ref, label=f"edge+block N={N} d={d}")


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_peaked_scores(d, causal):
    N = 500
    q, k, v, do = make_qkv(1, 3, N, d, seed=9900 + d)
    q = (q.float() * 4).to(torch.bfloat16)   # exact: a power of two
    k = (k.float() * 4).to(torch.bfloat16)
    v = (v.float() * 0.5).to(torch.bfloat16)
    print(f"[case] peaked scores N={N} d={d} causal={causal}", flush=True)
    gpu = run_gpu(q, k, v, do, causal=causal, scale=_scale(d))
    ref = run_oracle(q, k, v, do, causal=causal, scale=_scale(d))
    assert_parity(gpu, ref, label=f"peaked d={d} causal={causal}")


@pytest.mark.parametrize("B,H,N,d,causal,masked", [(16, 64, 96, 64, True, False),
                                                    (8, 128, 130, 128, False, True),
                                                    (7, 9, 300, 128, True, True),
                                                    (9, 7, 257, 64, False, True)])
def test_many_heads_and_head_orders(B, H, N, d, causal, masked):
    """Many heads with few row blocks each (1024 heads), and B*H = 63, which is not a
    multiple of 8, so masked launches keep the interleaved workgroup order instead of
    the head-major one; block masks are per head. Every head is compared in full."""
    q, k, v, do = make_qkv(B, H, N, d, seed=9950 + B * H + N)
    bm = None
    if masked:
        nb = -(-N // 128)
        rng = np.random.default_rng(9960 + N)
        bm = (rng.random((B, H, nb, nb)) < 0.6).astype(np.uint8)
        for b in range(B):
            for h in range(H):
                np.fill_diagonal(bm[b, h], 1)
    print(f"[case] many heads B={B} H={H} N={N} d={d} causal={causal} masked={masked}", flush=True)
    gpu = run_gpu(q, k, v, do, causal=causal, block_mask=bm, scale=_scale(d))
    ref = run_oracle(q, k, v, do, causal=causal, block_mask=bm, scale=_scale(d))
    assert_parity(gpu, ref, label=f"many heads B={B} H={H} N={N} d={d}")
