"""Host checks of the input generators and of the attended-pair count used for FLOP figures.

kept_fraction is checked against a brute-force count of the mask definitions
(causal: key j visible to query i iff j <= i; block: iff the 128 x 128 block
holding (i, j) is kept), so the FLOP numerators of the benchmark rest on the
definitions, not on the closed forms inside kept_fraction.
"""
import numpy as np
import pytest
import torch

from exact_io_aware_61_amd.workloads import (BLOCK, WORKLOADS, kept_fraction, make_block_mask,
                                             make_inputs, variant)


def _brute_rho(N, causal, bm):
    i = np.arange(N)[:, None]
    j = np.arange(N)[None, :]
    vis = np.ones((N, N), dtype=bool)
    if causal:
        vis &= j <= i
    if bm is not None:
        vis &= bm[i // BLOCK, j // BLOCK].astype(bool)
    return vis.sum() / (N * N)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("keep", [None, 0.05, 0.5, 1.0])
def test_kept_fraction_matches_brute_force(causal, keep):
    N = 640
    bm = None if keep is None else make_block_mask(N, keep, seed=31)
    assert kept_fraction(N, causal, bm) == pytest.approx(_brute_rho(N, causal, bm), abs=1e-12)


def test_block_mask_shape_and_diagonal():
    m = make_block_mask(1000, 0.0, seed=5)
    assert m.shape == (8, 8) and m.dtype == np.uint8
    assert np.array_equal(m, np.eye(8, dtype=np.uint8))          # keep 0: diagonal only
    assert make_block_mask(1000, 1.0, seed=5).all()               # keep 1: everything
    dens = make_block_mask(16384, 0.25, seed=1006).mean()
    assert abs(dens - (0.25 + 0.75 / 128)) < 0.01                 # expected kept fraction


def test_variant_keeps_the_draws():
    w = WORKLOADS["tiny"]
    v = variant(w, block_keep=0.1, causal=True)
    assert v.name == "tiny:keep=0.1+causal" and v.causal and v.block_keep == 0.1
    q0, k0, v0, d0, m0 = make_inputs(w)
    q1, k1, v1, d1, m1 = make_inputs(v)
    assert m0 is None and m1.shape == (2, 2)
    for a, b in ((q0, q1), (k0, k1), (v0, v1), (d0, d1)):
        assert torch.equal(a, b)
    assert variant(w) == w   # no change, same name


def test_sparse16k_mask_draw_is_seeded():
    w = WORKLOADS["sparse16k"]
    a = make_block_mask(w.N, w.block_keep, w.seed + 1)
    b = make_block_mask(w.N, w.block_keep, w.seed + 1)
    assert np.array_equal(a, b)
    c = make_block_mask(w.N, 0.05, w.seed + 1)
    assert c.sum() < a.sum()
