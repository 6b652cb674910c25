"""GPU parity: the HIP path (through the C ABI) against the CPU fp64 oracle.

Small cases run the oracle on every head; they span several tiles in both
dimensions and end in a ragged tail (N not a multiple of 64 or 128). The five
named workloads run whole on the GPU, in the launch configuration the
benchmark times, and are compared with the oracle on sampled (batch, head)
pairs, which the oracle computes completely.
"""
import math

import numpy as np
import pytest
import torch

import exact_io_aware_61_amd as fa
from exact_io_aware_61_amd.workloads import (WORKLOADS, make_block_mask, make_inputs, make_qkv,
                                             variant)
from tests.gpu_util import assert_parity, run_gpu, run_oracle, to64

pytestmark = pytest.mark.gpu

MASKS = ["none", "causal", "block", "causal+block"]


def _mask(kind, N, seed):
    causal = "causal" in kind
    bm = make_block_mask(N, 0.5, seed) if "block" in kind else None
    return causal, bm


@pytest.fixture(scope="module", autouse=True)
def _lib():
    fa.load()
    torch.cuda.init()


# -------------------------------------------------------------------------------------------------
# full comparison on small shapes

@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("kind", MASKS)
@pytest.mark.parametrize("N", [256, 333, 513])
def test_small_parity(N, kind, d):
    B, H = 1, 2
    q, k, v, do = make_qkv(B, H, N, d, seed=7000 + N + d)
    causal, bm = _mask(kind, N, seed=N)
    scale = float(np.float32(1 / math.sqrt(d)))
    print(f"[case] small N={N} d={d} mask={kind}", flush=True)
    gpu = run_gpu(q, k, v, do, causal=causal, block_mask=bm, scale=scale)
    ref = run_oracle(q, k, v, do, causal=causal, block_mask=bm, scale=scale)
    assert_parity(gpu, ref, label=f"N={N} d={d} {kind}")


@pytest.mark.parametrize("keep", [0.05, 0.1, 0.25, 0.5, 1.0])
@pytest.mark.parametrize("causal", [False, True])
def test_block_density_sweep(keep, causal):
    """The densities of the block-sparse sweep, alone and combined with the causal mask."""
    B, H, N, d = 1, 2, 1152, 64   # 9 x 9 mask blocks
    q, k, v, do = make_qkv(B, H, N, d, seed=8100)
    bm = make_block_mask(N, keep, seed=8200 + int(keep * 100))
    scale = float(np.float32(1 / math.sqrt(d)))
    print(f"[case] density keep={keep} causal={causal}", flush=True)
    gpu = run_gpu(q, k, v, do, causal=causal, block_mask=bm, scale=scale)
    ref = run_oracle(q, k, v, do, causal=causal, block_mask=bm, scale=scale)
    assert_parity(gpu, ref, label=f"keep={keep} causal={causal}")


@pytest.mark.parametrize("N,d,B,H", [(1, 64, 1, 1), (17, 128, 2, 1), (65, 64, 1, 3),
                                      (129, 128, 1, 2), (200, 64, 3, 2)])
@pytest.mark.parametrize("causal", [False, True])
def test_ragged_and_tiny_shapes(N, d, B, H, causal):
    q, k, v, do = make_qkv(B, H, N, d, seed=9000 + N)
    scale = float(np.float32(1 / math.sqrt(d)))
    print(f"[case] ragged N={N} d={d} B={B} H={H} causal={causal}", flush=True)
    gpu = run_gpu(q, k, v, do, causal=causal, scale=scale)
    ref = run_oracle(q, k, v, do, causal=causal, scale=scale)
    assert_parity(gpu, ref, label=f"ragged N={N} d={d}")


def test_custom_scale():
    q, k, v, do = make_qkv(1, 2, 300, 64, seed=31)
    print("[case] scale=0.3", flush=True)
    gpu = run_gpu(q, k, v, do, causal=True, scale=0.3)
    ref = run_oracle(q, k, v, do, causal=True, scale=0.3)
    assert_parity(gpu, ref, label="scale=0.3")


def test_per_head_block_masks():
    B, H, N, d = 2, 2, 384, 64
    q, k, v, do = make_qkv(B, H, N, d, seed=32)
    nb = 3
    rng = np.random.default_rng(5)
    grids = (rng.random((B, H, nb, nb)) < 0.5).astype(np.uint8)
    for b in range(B):
        for h in range(H):
            np.fill_diagonal(grids[b, h], 1)
    scale = 0.125
    print("[case] per-head block masks", flush=True)
    gpu = run_gpu(q, k, v, do, block_mask=grids, scale=scale)
    ref = run_oracle(q, k, v, do, block_mask=grids, scale=scale)
    assert_parity(gpu, ref, label="per-head masks")


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_block_mask_head_major_order(d, causal):
    """B*H a multiple of 8 with a block mask: the launches take the head-major
    workgroup order (each XCD works through whole heads); every head, with a
    grid of its own, is compared in full, on a ragged N."""
    B, H, N = 2, 8, 600
    q, k, v, do = make_qkv(B, H, N, d, seed=34 + d)
    nb = -(-N // 128)
    rng = np.random.default_rng(35 + d)
    grids = (rng.random((B, H, nb, nb)) < 0.5).astype(np.uint8)
    for b in range(B):
        for h in range(H):
            np.fill_diagonal(grids[b, h], 1)
    scale = float(np.float32(1 / math.sqrt(d)))
    print(f"[case] head-major block order d={d} causal={causal}", flush=True)
    gpu = run_gpu(q, k, v, do, causal=causal, block_mask=grids, scale=scale)
    ref = run_oracle(q, k, v, do, causal=causal, block_mask=grids, scale=scale)
    assert_parity(gpu, ref, label=f"head-major d={d} causal={causal}")


def test_empty_rows_from_block_mask():
    """Rows whose every block is dropped: O = 0, LSE = -inf, zero gradients."""
    N, d = 256, 64
    q, k, v, do = make_qkv(1, 1, N, d, seed=33)
    bm = np.array([[1, 0], [0, 0]], np.uint8)   # rows 128..255 see nothing
    scale = 0.125
    print("[case] empty rows", flush=True)
    gpu = run_gpu(q, k, v, do, block_mask=bm, scale=scale)
    ref = run_oracle(q, k, v, do, block_mask=bm, scale=scale)
    assert_parity(gpu, ref, label="empty rows")
    o = to64(gpu["o"])[0, 0]
    assert np.all(o[128:] == 0)
    assert np.all(np.isneginf(to64(gpu["lse"])[0, 0, 128:]))
    assert np.all(to64(gpu["dq"])[0, 0, 128:] == 0)
    assert np.all(to64(gpu["dk"])[0, 0, 128:] == 0) and np.all(to64(gpu["dv"])[0, 0, 128:] == 0)


def test_zero_extent_is_noop():
    dev = torch.device("cuda:0")
    for shape in [(0, 2, 64, 64), (1, 0, 64, 64), (1, 2, 0, 64)]:
        q = torch.empty(shape, dtype=torch.bfloat16, device=dev)
        o, lse = fa.forward(q, q.clone(), q.clone())
        assert o.shape == shape and lse.shape == shape[:3]


# -------------------------------------------------------------------------------------------------
# closed forms and invariants on the GPU (pins of the kernels themselves)

def test_zero_q_gives_mean_of_v():
    B, H, N, d = 1, 2, 300, 128
    _, k, v, do = make_qkv(B, H, N, d, seed=40)
    q = torch.zeros_like(k)
    gpu = run_gpu(q, k, v, do, causal=True, scale=0.1)
    cnt = np.arange(1, N + 1)
    mean = np.cumsum(to64(v), axis=2) / cnt[None, None, :, None]
    assert np.abs(to64(gpu["o"]) - mean).max() <= 1e-2
    np.testing.assert_allclose(to64(gpu["lse"]), np.broadcast_to(np.log(cnt), (B, H, N)),
                               atol=1e-4)
    assert np.abs(to64(gpu["dk"])).max() <= 1e-6


def test_ones_v_and_causal_row0():
    B, H, N, d = 1, 2, 257, 64
    q, k, _, do = make_qkv(B, H, N, d, seed=41)
    v = torch.ones_like(q)
    gpu = run_gpu(q, k, v, do, causal=True, scale=0.125, with_bwd=False)
    assert np.all(to64(gpu["o"]) == 1.0)
    q2, k2, v2, _ = make_qkv(B, H, N, d, seed=42)
    g2 = run_gpu(q2, k2, v2, None, causal=True, scale=0.125, with_bwd=False)
    np.testing.assert_array_equal(to64(g2["o"])[:, :, 0], to64(v2)[:, :, 0])
    s00 = 0.125 * (to64(q2)[:, :, 0] * to64(k2)[:, :, 0]).sum(-1)
    np.testing.assert_allclose(to64(g2["lse"])[:, :, 0], s00, atol=1e-5)


def test_identity_v_exposes_p():
    """N = d = 128 and V = I: O = P, so the kernel's probability tile is compared directly."""
    N = d = 128
    q, k, _, _ = make_qkv(1, 1, N, d, seed=43)
    v = torch.eye(N, dtype=torch.bfloat16).reshape(1, 1, N, N)
    gpu = run_gpu(q, k, v, None, scale=0.088, with_bwd=False)
    from oracle import softmax_rows
    p, _ = softmax_rows(to64(q)[0, 0], to64(k)[0, 0], np.arange(N), scale=0.088, causal=False,
                        block_mask=None, block=128)
    assert np.abs(to64(gpu["o"])[0, 0] - p).max() <= 2e-3


def test_all_ones_block_mask_is_bitwise_dense():
    q, k, v, do = make_qkv(1, 2, 384, 64, seed=44)
    a = run_gpu(q, k, v, do, scale=0.125)
    b = run_gpu(q, k, v, do, block_mask=np.ones((3, 3), np.uint8), scale=0.125)
    for key in ("o", "lse", "dk", "dv"):
        assert torch.equal(a[key], b[key]), key


def test_gradient_sums():
    """sum_j dK_j = 0 and sum_j dV_j = sum_i dO_i per head (no empty rows)."""
    q, k, v, do = make_qkv(2, 2, 512, 128, seed=45)
    gpu = run_gpu(q, k, v, do, causal=True, scale=0.088)
    dk, dv, dof = to64(gpu["dk"]), to64(gpu["dv"]), to64(do)
    assert np.abs(dk.sum(axis=2)).max() <= 2e-2 * np.abs(dk).sum(axis=2).max()
    np.testing.assert_allclose(dv.sum(axis=2), dof.sum(axis=2), atol=0.05 * np.sqrt(512))


@pytest.mark.parametrize("d", [64, 128])
def test_every_output_bitwise_reproducible(d):
    """No atomics anywhere: repeated calls give identical bits for every output."""
    q, k, v, do = make_qkv(2, 4, 1024, d, seed=46)
    a = run_gpu(q, k, v, do, causal=True, scale=0.088)
    b = run_gpu(q, k, v, do, causal=True, scale=0.088)
    for key in ("o", "lse", "dq", "dk", "dv"):
        assert torch.equal(a[key], b[key]), key


def test_autograd_wrapper_matches_backward():
    dev = torch.device("cuda:0")
    q, k, v, do = (t.to(dev) for t in make_qkv(1, 2, 256, 64, seed=47))
    qr, kr, vr = (t.clone().requires_grad_(True) for t in (q, k, v))
    o = fa.attention(qr, kr, vr, causal=True)
    o.backward(do)
    o2, lse = fa.forward(q, k, v, causal=True)
    dq, dk, dv = fa.backward(q, k, v, o2, lse, do, causal=True)
    assert torch.equal(o, o2)
    assert torch.equal(kr.grad, dk) and torch.equal(vr.grad, dv) and torch.equal(qr.grad, dq)


# -------------------------------------------------------------------------------------------------
# the named workloads at full size: whole problem on the GPU, oracle on sampled heads

def _sampled(w, heads):
    q, k, v, do, bm = make_inputs(w)
    print(f"[case] workload {w.name} B={w.B} H={w.H} N={w.N} d={w.d} heads={heads}", flush=True)
    gpu = run_gpu(q, k, v, do, causal=w.causal, block_mask=bm, scale=w.scale)
    ref = run_oracle(q, k, v, do, causal=w.causal, block_mask=bm, scale=w.scale, heads=heads)
    return assert_parity(gpu, ref, heads=heads, label=w.name)


def test_workload_tiny_full():
    w = WORKLOADS["tiny"]
    q, k, v, do, bm = make_inputs(w)
    gpu = run_gpu(q, k, v, do, causal=w.causal, block_mask=bm, scale=w.scale)
    ref = run_oracle(q, k, v, do, causal=w.causal, block_mask=bm, scale=w.scale)
    assert_parity(gpu, ref, label="tiny (all heads)")


def test_workload_dense2k_sampled():
    _sampled(WORKLOADS["dense2k"], heads=[(0, 0), (3, 7), (7, 15)])


def test_workload_causal8k_sampled():
    _sampled(WORKLOADS["causal8k"], heads=[(0, 0), (1, 15)])


@pytest.mark.timeout(300)
def test_workload_causal32k_sampled():
    _sampled(WORKLOADS["causal32k"], heads=[(0, 5)])


@pytest.mark.timeout(300)
def test_workload_sparse16k_sampled():
    _sampled(WORKLOADS["sparse16k"], heads=[(0, 0), (3, 15)])


@pytest.mark.timeout(300)
def test_workload_sparse16k_sparsest_causal_sampled():
    """The sparsest density of the sweep, combined with the causal mask, at full size."""
    _sampled(variant(WORKLOADS["sparse16k"], block_keep=0.05, causal=True), heads=[(2, 9)])
