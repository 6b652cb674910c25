"""The online-softmax rescale under test: inputs whose row maxima keep growing.

The forward keeps a running row maximum m and, when a tile raises it, rescales
the row's denominator and its unnormalised output by 2^(m_old - m_new) (the
one-pass recurrence of the lecture summary on FlashAttention v1, section 3.2;
the FlashAttention-2 overview's deferred normalisation). fa_fwd moves its
reference maximum lazily, only when some row of a wave outgrows it by more than
2^8, which N(0,1) inputs never do after a row's first tile. These inputs
(workloads.make_rising_scores) make the scores of most rows grow steadily with
the key index, so the rescale runs several times per row sweep with factors in
(0, 1). A host replay of the kernel's rule (per wave of 32 query rows, 64-key
tiles in sweep order) counts those events from the inputs alone and each case
asserts at least one; outputs are then compared element-wise with the fp64
oracle, and the same inputs go through the decoding and K/V-outer kernels,
which rescale on every tile.
"""
import math

import numpy as np
import pytest
import torch

import exact_io_aware_61_amd as fa
from exact_io_aware_61_amd.workloads import make_block_mask, make_qkv, make_rising_scores
from tests.gpu_util import assert_parity, run_gpu, run_oracle, to64

LOG2E = 1.4426950408889634
THRESHOLD = 8.0     # log2 units by which a row must outgrow the reference max
WAVE_ROWS = 32
TILE_KEYS = 64
MASK_BLOCK = 128


def rescale_events(q, k, scale, causal, block_mask):
    """Rescale events after a wave's first visible tile, replaying the forward's rule.

    q, k: [N, d] arrays of one head. Per wave of 32 consecutive query rows, the
    visible 64-key tiles are swept in order; a tile whose row maxima (log2 units)
    exceed some row's reference by more than THRESHOLD moves every row's reference
    to max(reference, tile max). Counted: moves in which at least one row had a
    finite reference that went up, i.e. a rescale by a factor in (0, 1).
    """
    q = np.asarray(q, np.float32)
    k = np.asarray(k, np.float32)
    N = q.shape[0]
    s = (q @ k.T) * np.float32(scale * LOG2E)
    rows = np.arange(N)
    if causal:
        s = np.where(rows[None, :] <= rows[:, None], s, -np.inf)
    if block_mask is not None:
        bm = np.asarray(block_mask).astype(bool)
        s = np.where(bm[rows[:, None] // MASK_BLOCK, rows[None, :] // MASK_BLOCK], s, -np.inf)
    events = 0
    for w0 in range(0, N, WAVE_ROWS):
        ref = np.full(min(WAVE_ROWS, N - w0), -np.inf, np.float32)
        for kb in range(0, N, TILE_KEYS):
            if causal and kb > w0 + WAVE_ROWS - 1:
                break
            if block_mask is not None and not bm[w0 // MASK_BLOCK, kb // MASK_BLOCK]:
                continue
            mx = s[w0:w0 + WAVE_ROWS, kb:kb + TILE_KEYS].max(axis=1)
            if np.any(mx > ref + THRESHOLD):
                new = np.maximum(ref, mx)
                if np.any(np.isfinite(ref) & (new > ref)):
                    events += 1
                ref = new
    return events


def _events_all_heads(q, k, scale, causal, bm):
    B, H = q.shape[:2]
    return [rescale_events(to64(q)[b, h], to64(k)[b, h], scale, causal, bm)
            for b in range(B) for h in range(H)]


MASKS = ["none", "causal", "block", "causal+block"]


def _case(kind, N, d, seed, **kw):
    q, k, v, do = make_rising_scores(1, 2, N, d, seed, **kw)
    causal = "causal" in kind
    bm = make_block_mask(N, 0.5, seed + 1) if "block" in kind else None
    scale = float(np.float32(1 / math.sqrt(d)))
    return q, k, v, do, causal, bm, scale


# ------------------------------------------------------------------------------------------------
# CPU: the inputs do what the GPU cases rely on


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("kind", MASKS)
def test_rising_inputs_trigger_rescales(kind, d):
    q, k, _, _, causal, bm, scale = _case(kind, 333, d, seed=300 + d)
    ev = _events_all_heads(q, k, scale, causal, bm)
    assert min(ev) >= 1, ev


def test_normal_inputs_never_rescale_after_the_first_tile():
    """Why the rising inputs are needed: N(0,1) draws never move the lazy reference."""
    q, k, _, _ = make_qkv(1, 2, 513, 128, seed=7000 + 513 + 128, with_do=False)
    assert _events_all_heads(q, k, float(np.float32(1 / math.sqrt(128))), True, None) == [0, 0]


# ------------------------------------------------------------------------------------------------
# GPU parity on those inputs


@pytest.fixture(scope="module")
def _lib():
    fa.load()
    torch.cuda.init()


@pytest.mark.gpu
@pytest.mark.parametrize("N", [333, 1000])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("kind", MASKS)
def test_rescale_parity(_lib, kind, d, N):
    q, k, v, do, causal, bm, scale = _case(kind, N, d, seed=300 + d + N)
    ev = _events_all_heads(q, k, scale, causal, bm)
    print(f"[case] rescale N={N} d={d} mask={kind} events={ev}", flush=True)
    assert min(ev) >= 1, ev
    gpu = run_gpu(q, k, v, do, causal=causal, block_mask=bm, scale=scale)
    ref = run_oracle(q, k, v, do, causal=causal, block_mask=bm, scale=scale)
    assert_parity(gpu, ref, label=f"rescale N={N} d={d} {kind} events={ev}")


@pytest.mark.gpu
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_rescale_late_outliers(_lib, d, causal):
    """The last keys jump far above every earlier score: the maximum moves on the last tile.

    The outlier keys then dominate their rows, so O is close to a mean of a few V
    rows; V is halved (exact in bf16) to keep |O| below 2, where one bf16 unit in
    the last place stays under the 1e-2 O bar and the case measures the rescale
    rather than the resolution of bf16 at |O| >= 2."""
    N = 600
    q, k, v, do = make_rising_scores(1, 2, N, d, 900 + d, late_outliers=5)
    v = (v.float() * 0.5).to(torch.bfloat16)
    scale = float(np.float32(1 / math.sqrt(d)))
    ev = _events_all_heads(q, k, scale, causal, None)
    print(f"[case] late outliers d={d} causal={causal} events={ev}", flush=True)
    assert min(ev) >= 1, ev
    gpu = run_gpu(q, k, v, do, causal=causal, scale=scale)
    ref = run_oracle(q, k, v, do, causal=causal, scale=scale)
    assert_parity(gpu, ref, label=f"late outliers d={d} causal={causal} events={ev}")


@pytest.mark.gpu
@pytest.mark.timeout(300)
def test_rescale_full_size_causal8k_shape(_lib):
    """The causal8k shape (B=2, H=16, N=8192, d=128, causal) with rising scores; the whole
    problem runs on the GPU in the benchmark's launch configuration, and the oracle checks
    one head in full."""
    B, H, N, d = 2, 16, 8192, 128
    q, k, v, do = make_rising_scores(B, H, N, d, 1303)
    scale = float(np.float32(1 / math.sqrt(d)))
    heads = [(1, 9)]
    ev = [rescale_events(to64(q)[b, h], to64(k)[b, h], scale, True, None) for b, h in heads]
    print(f"[case] rescale causal8k shape heads={heads} events={ev}", flush=True)
    assert min(ev) >= 1, ev
    gpu = run_gpu(q, k, v, do, causal=True, scale=scale)
    ref = run_oracle(q, k, v, do, causal=True, scale=scale, heads=heads)
    assert_parity(gpu, ref, heads=heads, label=f"rescale causal8k shape events={ev}")


@pytest.mark.gpu
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_rescale_inputs_through_kv_outer(_lib, d, causal):
    N = 333
    q, k, v, _ = make_rising_scores(1, 2, N, d, 500 + d)
    scale = float(np.float32(1 / math.sqrt(d)))
    print(f"[case] rescale kv-outer d={d} causal={causal}", flush=True)
    o, lse = fa.forward_kv_outer(q.cuda(), k.cuda(), v.cuda(), causal=causal, scale=scale)
    torch.cuda.synchronize()
    ref = run_oracle(q, k, v, None, causal=causal, scale=scale)
    assert_parity({"o": o, "lse": lse}, ref, label=f"rescale kv-outer d={d} causal={causal}")


@pytest.mark.gpu
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_rescale_inputs_through_decode(_lib, d, causal):
    """The newest 16 queries of a rising-score sequence against its whole cache."""
    from oracle.decode import decode as decode_ref
    N, Nq = 2000, 16
    q, k, v, _ = make_rising_scores(1, 2, N, d, 600 + d)
    qn = q[:, :, N - Nq:].contiguous()
    scale = float(np.float32(1 / math.sqrt(d)))
    print(f"[case] rescale decode d={d} causal={causal}", flush=True)
    o, lse = fa.decode(qn.cuda(), k.cuda(), v.cuda(), causal=causal, scale=scale)
    torch.cuda.synchronize()
    ref = decode_ref(to64(qn), to64(k), to64(v), scale=scale, causal=causal)
    assert_parity({"o": o, "lse": lse}, ref, label=f"rescale decode d={d} causal={causal}")
