"""Host-side arithmetic of bench.py (CPU only): the IO models it reports, the
traffic records it reads from profiles/, and its one-GPU guard.

* kv_outer_io_model is checked against a brute-force walk of the K/V-outer
  loops (every (K/V block, Q block) pair tested for a visible key, the bytes of
  each visit added one by one), not against its own closed form.
* naive_io_model is checked against the bytes of standard attention counted by
  hand, pass by pass, at the causal8k shape (the figure quoted in the profiles).
* Each committed traffic record must be consistent with its own raw counter
  values and calibration factors.
* The CPU oracle timing reports both the algorithmic and the executed rate.
* pass_io_models' tile visits are checked against a walk over every (query, key)
  pair of small ragged shapes.
"""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def kv_outer_bytes_by_walk(N, d, causal, BM=128, BN=64):
    Tr, Tc = -(-N // BM), -(-N // BN)
    total = 4 * N * d                      # K and V, read once
    started = set()
    for j in range(Tc):
        for i in range(Tr):
            if causal and i * BM + BM - 1 < j * BN:
                continue                   # every row of block i precedes every key of block j
            total += 2 * BM * d            # the Q block
            if i in started:
                total += 4 * BM * d + 8 * BM   # O (float32), m, l read back
            total += 4 * BM * d + 8 * BM       # ... and written
            started.add(i)
    total += 4 * N * d + 8 * N             # last sweep: O, m, l read
    total += 2 * N * d + 4 * N             # O (bf16) and LSE written
    return total


@pytest.mark.parametrize("N,d,causal", [(256, 64, False), (256, 64, True), (1000, 128, True),
                                        (2048, 64, False), (8192, 128, True)])
def test_kv_outer_io_model_matches_loop_walk(N, d, causal):
    heads = 3
    assert bench.kv_outer_io_model(N, d, causal, heads) == heads * kv_outer_bytes_by_walk(N, d, causal)


def test_naive_io_model_causal8k_by_hand():
    N, d, heads = 8192, 128, 32
    nd, nn = 2 * N * d, 2 * N * N          # bytes of one [N, d] and one [N, N] bf16 matrix
    passes = [
        2 * nd,            # K^T made contiguous: read K, write K^T
        2 * nd,            # Q scaled: read Q, write it
        2 * nd + nn,       # S = Q K^T: read both, write S
        2 * nn,            # mask: read S, write S
        2 * nn,            # softmax: read S, write P
        nn + 2 * nd,       # O = P V: read P and V, write O
    ]
    got = bench.naive_io_model(N, d, True, heads)
    assert got["naive_model"] == heads * sum(passes)
    assert got["naive_s_p_bytes"] == heads * 5 * nn
    assert abs(got["naive_model"] / 1e9 - 26.31) < 0.01   # the figure quoted in the profiles
    unmasked = bench.naive_io_model(N, d, False, heads)
    assert got["naive_model"] - unmasked["naive_model"] == heads * 2 * nn


def _records():
    out = []
    prof = os.path.join(ROOT, "profiles")
    for name in sorted(os.listdir(prof)):
        if not name.startswith("traffic_"):
            continue
        with open(os.path.join(prof, name)) as f:
            for line in f:
                if line.startswith("traffic-record:"):
                    out.append((name, json.loads(line.split(":", 1)[1])))
    return out


def test_traffic_records_are_self_consistent():
    recs = _records()
    assert recs, "no traffic records under profiles/"
    for name, rec in recs:
        if "fetch_kib_raw" not in rec:
            continue
        bytes_ = (rec["fetch_kib_raw"] * rec["fetch_factor"] + rec["write_kib_raw"] * rec["write_factor"]) * 1024
        # the stored factors are rounded (e.g. 1 GiB / 524300 KiB = 1.99995 shown as
        # 2.0); the bytes were computed with the unrounded ones
        assert abs(bytes_ - rec["bytes_per_launch"]) <= 1e-4 * rec["bytes_per_launch"], name
        if "algorithmic_bytes" in rec and "ratio_to_algorithmic" in rec:
            assert abs(rec["bytes_per_launch"] / rec["algorithmic_bytes"]
                       - rec["ratio_to_algorithmic"]) < 2e-3, name


def test_dominant_kernel_traffic_record_matches_current_sources():
    # bench.py's roofline reads this record for the dK/dV kernel at causal8k; it
    # must have been taken on the sources as they are.
    digest = bench.kernel_digest("fa_bwd_dkdv_kernel")
    rec = bench.traffic_record("fa_bwd_dkdv_kernel", "causal8k", digest)
    assert rec is not None, f"profiles/ has no traffic record for dK/dV at source digest {digest}"
    assert rec["bytes_per_launch"] > 0


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_cpu_baseline_reports_algorithmic_and_executed_rates():
    """The oracle timing on the tiny causal shape: algorithmic TFLOP/s counts
    3.5 x 4 N^2 d rho per head, executed TFLOP/s the 12 N^2 d the materialising
    oracle runs; their ratio is fixed by the shape."""
    from exact_io_aware_61_amd.workloads import WORKLOADS, kept_fraction, make_inputs, variant
    w = variant(WORKLOADS["tiny"], causal=True)
    q, k, v, do, bm = make_inputs(w)
    cb = bench.cpu_baseline(w, q, k, v, do, bm, seconds=0.05)
    assert cb["kind"] == "oracle" and cb["unit"] == "TFLOP/s" and cb["cores"] >= 1
    rho = kept_fraction(w.N, w.causal, bm)
    assert cb["executed_tflops"] / cb["value"] == pytest.approx(12.0 / (14.0 * rho))
    assert cb["fwd"]["executed_tflops"] / cb["fwd"]["value"] == pytest.approx(1.0 / rho)


def _visits_by_pairs(N, rows, keys, causal, keep):
    """Blocks of `rows` query rows x `keys` keys holding at least one attended pair,
    found by testing the pairs one by one."""
    import numpy as np
    i = np.arange(N)[:, None]
    j = np.arange(N)[None, :]
    att = keep[i // 128, j // 128] & ((j <= i) if causal else True)
    total = 0
    for r0 in range(0, N, rows):
        for k0 in range(0, N, keys):
            total += bool(att[r0:r0 + rows, k0:k0 + keys].any())
    return total


@pytest.mark.parametrize("N,d,causal,masked", [(300, 64, True, False), (300, 128, False, False),
                                               (640, 64, False, True), (640, 128, True, True),
                                               (1, 64, True, False)])
def test_pass_io_models_match_pair_walk(N, d, causal, masked):
    import numpy as np
    nb = -(-N // 128)
    rng = np.random.default_rng(N + d)
    mask = (rng.random((nb, nb)) < 0.4) | np.eye(nb, dtype=bool) if masked else None
    keep = np.ones((nb, nb), bool) if mask is None else mask
    io = bench.pass_io_models(N, d, causal, mask, heads=3)
    bm_fwd = bench.fwd_rows_per_workgroup(d, masked)
    bm_dq = 128 if (masked or d == 64) else 256
    bn_dq = 32 if (d == 64 and not masked) else 64
    nd = N * d
    assert io["tile_model_fwd"] == 3 * (4 * nd + 4 * N
                                        + _visits_by_pairs(N, bm_fwd, 64, causal, keep) * 64 * d * 4)
    assert io["tile_model_dq"] == 3 * (6 * nd + 8 * N
                                       + _visits_by_pairs(N, bm_dq, bn_dq, causal, keep) * bn_dq * d * 4)
    assert io["tile_model_dkdv"] == 3 * (8 * nd
                                         + _visits_by_pairs(N, 64, 128, causal, keep) * (64 * d * 4 + 512))
    assert io["compulsory_fwd"] == 3 * (8 * nd + 4 * N)
    assert io["compulsory_dkdv"] == 3 * (12 * nd + 8 * N)
    assert io["compulsory_dq"] == 3 * (10 * nd + 8 * N)
