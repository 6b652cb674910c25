"""The Python binding rejects caller-supplied buffers it cannot hand to the C ABI.

Output tensors, the lse input and workspaces given by the caller are checked
for shape, dtype, device and contiguity before any launch, and a workspace's
size is its byte count whatever its dtype. The CPU tests drive the checks with
host tensors; the GPU tests call the public entry points with bad buffers and
expect ValueError (nothing is launched: the check precedes the call).
"""
import pytest
import torch

import exact_io_aware_61_amd as fa
from exact_io_aware_61_amd import _binding as b

FAKE_GPU = torch.device("cuda:0")


def test_like_rejects_wrong_shape_dtype_layout_and_device():
    t = torch.empty(2, 3, 4, dtype=torch.float32)
    with pytest.raises(ValueError, match="shape"):
        b._like(t, (2, 3, 5), torch.float32, FAKE_GPU, "lse")
    with pytest.raises(ValueError, match="shape"):
        b._like(t, (2, 3, 4), torch.bfloat16, FAKE_GPU, "out")
    with pytest.raises(ValueError, match="non-contiguous"):
        b._like(t.transpose(0, 1), (3, 2, 4), torch.float32, FAKE_GPU, "lse")
    with pytest.raises(ValueError, match="live on"):
        b._like(t, (2, 3, 4), torch.float32, FAKE_GPU, "lse")   # a host tensor
    with pytest.raises(ValueError, match="torch tensor"):
        b._like([1, 2], (2,), torch.float32, FAKE_GPU, "lse")


def test_workspace_must_be_a_device_tensor():
    with pytest.raises(ValueError, match="workspace"):
        b._ws_bytes(torch.empty(64, dtype=torch.uint8), FAKE_GPU)
    with pytest.raises(ValueError, match="workspace"):
        b._ws_bytes(None, FAKE_GPU)


@pytest.mark.gpu
def test_entry_points_reject_bad_buffers():
    fa.load()
    dev = torch.device("cuda:0")
    q = torch.randn(1, 2, 128, 64, device=dev).to(torch.bfloat16)
    k, v, do = q.clone(), q.clone(), q.clone()
    o, lse = fa.forward(q, k, v)
    with pytest.raises(ValueError):
        fa.forward(q, k, v, lse=torch.empty(1, 2, device=dev))            # [B, H] lse
    with pytest.raises(ValueError):
        fa.forward(q, k, v, lse=torch.empty(1, 2, 128))                   # host lse
    with pytest.raises(ValueError):
        fa.forward(q, k, v, out=torch.empty(1, 2, 128, 64, device=dev))   # float32 out
    with pytest.raises(ValueError):
        fa.backward(q, k, v, o, lse[:, :, :64], do)                       # short lse
    with pytest.raises(ValueError):
        fa.backward(q, k, v, o, lse, do, ws=torch.empty(1 << 16, dtype=torch.uint8))  # host ws
    with pytest.raises(ValueError):
        fa.backward(q, k, v, o, lse, do, dq=torch.empty_like(q)[:, :, :, :32])
    # a workspace of another dtype counts in bytes: 4-byte elements suffice at a quarter count
    n = fa.bwd_workspace_size(1, 2, 128, 64)
    ws = torch.empty(-(-n // 4), dtype=torch.float32, device=dev)
    dq, dk, dv = fa.backward(q, k, v, o, lse, do, ws=ws)
    ref = fa.backward(q, k, v, o, lse, do)
    torch.cuda.synchronize()
    assert torch.equal(dq, ref[0]) and torch.equal(dk, ref[1]) and torch.equal(dv, ref[2])
    # too small by one byte's worth: the C ABI refuses it
    with pytest.raises(fa.FaError):
        fa.backward(q, k, v, o, lse, do, ws=torch.empty(n - 1, dtype=torch.uint8, device=dev))
