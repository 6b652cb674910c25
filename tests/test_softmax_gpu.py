"""GPU parity of the row-softmax kernel (fa_softmax_rows) against the fp64 oracle.

Tolerance, derived from float32 arithmetic: each output is e^(x - m) (one
v_exp_f32 of (x - m) log2 e, whose argument carries a relative rounding of
2^-24 on |x - m| <= ~100 here, i.e. <= 1e-5 relative) times a rescale factor
and 1/sum, the sum being float32 accumulation over at most 2^18 terms in
per-lane runs plus a tree (a few 1e-6 relative). So each element must match
within 3e-5 relative, plus 1e-37 absolute for values that float32 flushes to 0.
"""
import numpy as np
import pytest
import torch

import exact_io_aware_61_amd as fa
from oracle.softmax_forms import row_softmax

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib():
    fa.load()
    torch.cuda.init()


def _check(y, x64):
    ref = row_softmax(x64)
    got = y.double().cpu().numpy()
    err = np.abs(got - ref)
    bad = err > 3e-5 * ref + 1e-37
    assert not bad.any(), f"max rel err {np.max(err / np.maximum(ref, 1e-300)):.3g} at {np.argwhere(bad)[:3]}"
    live = np.isfinite(x64).any(axis=1)
    np.testing.assert_allclose(got[live].sum(axis=1), 1.0, atol=3e-5)
    assert np.all(got[~live] == 0.0)


def _inputs(rows, cols, sigma, seed, holes=True):
    rng = np.random.default_rng(seed)
    x = (rng.standard_normal((rows, cols)) * sigma).astype(np.float32)
    if holes and rows > 2 and cols > 1:
        x[1, rng.integers(0, cols, size=max(1, cols // 7))] = -np.inf   # masked entries
        x[2, :] = -np.inf                                               # no finite entry
    return x


@pytest.mark.parametrize("rows,cols", [(1, 1), (3, 3), (5, 63), (7, 64), (9, 65), (4, 256),
                                       (6, 1000), (33, 4096), (5, 4097), (3, 100003),
                                       (2, 262144)])
@pytest.mark.parametrize("sigma", [1.0, 8.0])
def test_softmax_rows_parity(rows, cols, sigma):
    x = _inputs(rows, cols, sigma, seed=rows * 1000 + cols)
    print(f"[case] softmax rows={rows} cols={cols} sigma={sigma}", flush=True)
    y = fa.softmax_rows(torch.from_numpy(x).cuda())
    torch.cuda.synchronize()
    _check(y, x.astype(np.float64))


@pytest.mark.parametrize("cols", [252, 256, 258, 260, 512, 516, 1024, 1028, 2048, 2052, 4092])
def test_softmax_rows_kernel_switch_points(cols):
    """Rows of 16-byte-aligned floats up to 4096 run the register kernel, one wave per row
    holding 4, 8, 16, 32 or 64 floats per lane (row lengths up to 256, 512, 1024, 2048,
    4096); other lengths run the streaming kernel. Lengths on and next to each switch point,
    one that is not a multiple of four (258) among them."""
    x = _inputs(11, cols, 4.0, seed=5000 + cols)
    print(f"[case] softmax switch point cols={cols}", flush=True)
    y = fa.softmax_rows(torch.from_numpy(x).cuda())
    torch.cuda.synchronize()
    _check(y, x.astype(np.float64))


def test_softmax_rows_in_place_and_unaligned():
    x = _inputs(17, 2048, 4.0, seed=3)
    print("[case] softmax in place", flush=True)
    t = torch.from_numpy(x).cuda()
    fa.softmax_rows(t, out=t)
    torch.cuda.synchronize()
    _check(t, x.astype(np.float64))
    # rows 4-byte but not 16-byte aligned: the scalar kernel
    print("[case] softmax unaligned", flush=True)
    buf = torch.zeros(17 * 2048 + 4, device="cuda", dtype=torch.float32)
    xin = buf[1:1 + 17 * 2048].view(17, 2048)
    xin.copy_(torch.from_numpy(x))
    out = torch.empty(17 * 2048 + 4, device="cuda", dtype=torch.float32)[1:1 + 17 * 2048].view(17, 2048)
    fa.softmax_rows(xin, out=out)
    torch.cuda.synchronize()
    _check(out, x.astype(np.float64))


def test_softmax_rows_large_shape_sampled():
    """The benchmark's shape (65536 x 4096) on the GPU, oracle on sampled rows."""
    rows, cols = 65536, 4096
    g = torch.Generator(device="cpu").manual_seed(77)
    x = torch.randn((rows, cols), generator=g, dtype=torch.float32) * 4.0
    print("[case] softmax 65536x4096 sampled", flush=True)
    y = fa.softmax_rows(x.cuda())
    torch.cuda.synchronize()
    idx = torch.tensor([0, 1, 4095, 32768, 65535])
    _check(y[idx.cuda()], x[idx].double().numpy())


def test_softmax_rows_errors():
    x = torch.zeros((4, 8), device="cuda")
    lib = fa.load()
    import ctypes
    P = lambda t: ctypes.c_void_p(t.data_ptr())  # noqa: E731
    assert lib.fa_softmax_rows(P(x), P(x), -1, 8, None) == -2
    assert lib.fa_softmax_rows(None, P(x), 4, 8, None) == -1
    assert lib.fa_softmax_rows(P(x), ctypes.c_void_p(x.data_ptr() + 2), 4, 8, None) == -4
    assert lib.fa_softmax_rows(P(x), ctypes.c_void_p(x.data_ptr() + 16), 4, 8, None) == -8
    assert lib.fa_softmax_rows(P(x), P(x), 0, 8, None) == 0
