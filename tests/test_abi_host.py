"""CPU-only checks of the C ABI: the library loads, exports every declared symbol,
and rejects bad arguments on the host before anything reaches a GPU.

Only argument combinations that fail validation are passed here (with
placeholder pointer values), so no call ever enqueues device work.
"""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa.h")
LIB = os.path.join(ROOT, "exact_io_aware_61_amd", "libfa.so")

OK, NULL, SHAPE, MASK, ALIGN, WS, HIP, SCALE, ALIAS, SCRATCH = 0, -1, -2, -3, -4, -5, -6, -7, -8, -9


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):
        from exact_io_aware_61_amd.build import build
        build()
    from exact_io_aware_61_amd import _binding
    return _binding.load()


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^(?:int|const char\s*\*)\s*(fa_\w+)\s*\(", text, re.M)))


def test_header_declares_the_abi():
    names = declared_functions()
    assert names == sorted(["fa_fwd", "fa_bwd", "fa_bwd_workspace_size", "fa_bwd_preprocess",
                            "fa_bwd_dkdv", "fa_bwd_dq", "fa_decode_workspace_size", "fa_decode",
                            "fa_fwd_kv_outer_workspace_size", "fa_fwd_kv_outer",
                            "fa_softmax_rows", "fa_bwd_noalloc", "fa_strerror"])


def test_every_declared_symbol_is_exported(lib):
    from exact_io_aware_61_amd import EXPORTS
    for name in declared_functions():
        assert hasattr(lib, name), name
    assert sorted(EXPORTS) == declared_functions()


def test_strerror_covers_every_status(lib):
    msgs = {s: lib.fa_strerror(s).decode() for s in (OK, NULL, SHAPE, MASK, ALIGN, WS, HIP, SCALE,
                                                     ALIAS, SCRATCH)}
    assert len(set(msgs.values())) == len(msgs)
    assert lib.fa_strerror(12345).decode() == "unknown status"


def test_workspace_size_arithmetic(lib):
    n = ctypes.c_size_t()
    for B, H, N, d in [(2, 16, 8192, 128), (1, 1, 1, 64), (4, 16, 16384, 64), (3, 5, 1000, 128)]:
        assert lib.fa_bwd_workspace_size(B, H, N, d, ctypes.byref(n)) == OK
        r256 = lambda x: (x + 255) // 256 * 256
        Np = (N + 127) // 128 * 128
        assert n.value == 2 * r256(B * H * Np * 4)   # D_i and LSE_i log2(e), per padded row
    assert lib.fa_bwd_workspace_size(1, 1, 1, 96, ctypes.byref(n)) == SHAPE
    assert lib.fa_bwd_workspace_size(-1, 1, 1, 64, ctypes.byref(n)) == SHAPE
    assert lib.fa_bwd_workspace_size(1, 1, 1, 64, None) == NULL


P = [ctypes.c_void_p(0x10000 * (i + 1)) for i in range(12)]   # placeholder device addresses
STREAM = ctypes.c_void_p(0)


def fwd(lib, q=P[0], k=P[1], v=P[2], o=P[3], lse=P[4], B=1, H=2, N=256, d=64, scale=0.125,
        mask=None):
    return lib.fa_fwd(q, k, v, o, lse, B, H, N, d, scale, mask, STREAM)


def test_fwd_rejects_bad_arguments(lib):
    from exact_io_aware_61_amd._binding import FaMask
    assert fwd(lib, q=None) == NULL
    assert fwd(lib, lse=None) == NULL
    assert fwd(lib, d=96) == SHAPE
    assert fwd(lib, d=256) == SHAPE
    assert fwd(lib, N=-1) == SHAPE
    assert fwd(lib, B=1 << 20, H=1 << 20, N=1 << 10, d=64) == SHAPE   # > 2^40 elements
    # under 2^40 elements, but 4*B*H*ceil(N/256)*256 work-items reach 2^32
    assert fwd(lib, B=1, H=1 << 21, N=512, d=64) == SHAPE
    assert fwd(lib, B=1, H=1 << 21, N=257, d=64) == SHAPE
    assert fwd(lib, q=None, B=1, H=(1 << 21) - 1, N=512, d=64) == NULL   # just inside
    assert fwd(lib, scale=0.0) == SCALE
    assert fwd(lib, scale=float("nan")) == SCALE
    assert fwd(lib, scale=float("inf")) == SCALE
    assert fwd(lib, scale=-0.5) == SCALE
    assert fwd(lib, q=ctypes.c_void_p(0x10008)) == ALIGN
    assert fwd(lib, lse=ctypes.c_void_p(0x50002)) == ALIGN
    # o overlaps k: 1*2*256*64*2 bytes = 64 KiB per tensor
    assert fwd(lib, o=ctypes.c_void_p(0x20000 + 4096)) == ALIAS
    bad_kind = FaMask(4, 128, None, 0)
    assert fwd(lib, mask=ctypes.byref(bad_kind)) == MASK
    no_grid = FaMask(2, 128, None, 0)
    assert fwd(lib, mask=ctypes.byref(no_grid)) == MASK
    bad_block = FaMask(2, 64, 0x90000, 0)
    assert fwd(lib, mask=ctypes.byref(bad_block)) == MASK
    neg_stride = FaMask(2, 128, 0x90000, -1)
    assert fwd(lib, mask=ctypes.byref(neg_stride)) == MASK
    # a block mask covers at most 16384 blocks of 128: N <= 2^21
    grid = FaMask(2, 128, 0x90000, 0)
    assert fwd(lib, mask=ctypes.byref(grid), N=(1 << 21) + 1, B=1, H=1) == MASK


def test_zero_extent_returns_ok_without_pointers(lib):
    # nothing to compute: no pointer is dereferenced and nothing is launched
    assert fwd(lib, q=None, k=None, v=None, o=None, lse=None, N=0) == OK
    assert fwd(lib, q=None, k=None, v=None, o=None, lse=None, B=0) == OK


def test_bwd_rejects_bad_arguments(lib):
    n = ctypes.c_size_t()
    lib.fa_bwd_workspace_size(1, 2, 256, 64, ctypes.byref(n))
    ws, need = P[9], n.value

    def bwd(q=P[0], dq=P[5], ws_ptr=ws, ws_bytes=need, d=64, scale=0.125):
        return lib.fa_bwd(q, P[1], P[2], P[3], P[4], P[8], dq, P[6], P[7], 1, 2, 256, d, scale,
                          None, ws_ptr, ws_bytes, STREAM)

    assert bwd(q=None) == NULL
    assert bwd(d=80) == SHAPE
    assert bwd(scale=0.0) == SCALE
    assert bwd(ws_ptr=None) == WS
    assert bwd(ws_bytes=need - 1) == WS
    assert bwd(ws_ptr=ctypes.c_void_p(0x90004)) == ALIGN
    assert bwd(dq=ctypes.c_void_p(0x10000 + 64)) == ALIAS   # dq overlaps q
    assert lib.fa_bwd_preprocess(None, P[4], P[8], 1, 2, 256, 64, ws, need, STREAM) == NULL
    assert lib.fa_bwd_preprocess(P[3], P[4], None, 1, 2, 256, 64, ws, need, STREAM) == NULL
    assert lib.fa_bwd_preprocess(P[3], P[4], P[8], 1, 2, 256, 64, ws, need - 1, STREAM) == WS
    assert lib.fa_bwd_preprocess(P[3], P[4], P[8], 1, 2, 256, 64, P[4], need, STREAM) == ALIAS
    assert lib.fa_bwd_dkdv(P[0], P[1], P[2], P[4], P[6], P[7], 1, 2, 256, 64, 0.125, None,
                           ws, 16, STREAM) == WS
    assert lib.fa_bwd_dkdv(P[0], P[1], P[2], P[4], None, P[7], 1, 2, 256, 64, 0.125, None,
                           ws, need, STREAM) == NULL
    assert lib.fa_bwd_dkdv(P[0], P[1], P[2], P[4], P[0], P[7], 1, 2, 256, 64, 0.125, None,
                           ws, need, STREAM) == ALIAS   # dk overlaps q
    assert lib.fa_bwd_dkdv(P[0], P[1], P[2], P[4], ws, P[7], 1, 2, 256, 64, 0.125, None,
                           ws, need, STREAM) == ALIAS   # dk overlaps the workspace
    assert lib.fa_bwd_dq(P[0], P[1], P[2], P[4], P[5], 1, 2, 256, 64, 0.125, None, None,
                         need, STREAM) == WS
    assert lib.fa_bwd_dq(P[0], P[1], P[2], P[4], P[5], 1, 2, 256, 64, -1.0, None, ws, need,
                         STREAM) == SCALE
    assert lib.fa_bwd_dq(P[0], P[1], P[2], P[4], ctypes.c_void_p(0x60008), 1, 2, 256, 64,
                         0.125, None, ws, need, STREAM) == ALIGN


def test_binding_refuses_cpu_tensors():
    """The Python layer has no CPU path: CPU tensors are an error, not a fallback."""
    import torch
    import exact_io_aware_61_amd as fa
    q = torch.zeros(1, 1, 64, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        fa.forward(q, q, q)


def test_softmax_rows_rejects_bad_arguments(lib):
    x, y = P[0], P[1]
    assert lib.fa_softmax_rows(x, y, -1, 8, STREAM) == SHAPE
    assert lib.fa_softmax_rows(x, y, 8, 1 << 31, STREAM) == SHAPE
    assert lib.fa_softmax_rows(x, y, 1 << 20, 1 << 20, STREAM) == SHAPE   # rows * cols >= 2^40
    assert lib.fa_softmax_rows(None, y, 4, 8, STREAM) == NULL
    assert lib.fa_softmax_rows(x, ctypes.c_void_p(0x20002), 4, 8, STREAM) == ALIGN
    assert lib.fa_softmax_rows(x, ctypes.c_void_p(0x10010), 4, 8, STREAM) == ALIAS   # overlaps x
    assert lib.fa_softmax_rows(None, None, 0, 8, STREAM) == OK                      # empty: no-op


def test_decode_rejects_bad_arguments(lib):
    n = ctypes.c_size_t()
    assert lib.fa_decode_workspace_size(2, 4, 16, 4096, 128, ctypes.byref(n)) == OK
    assert n.value > 0 and n.value % 256 == 0
    assert lib.fa_decode_workspace_size(1, 1, 16, 64, 128, ctypes.byref(n)) == OK
    need = n.value   # placeholder buffers 64 KiB apart: keep the shapes below that size
    assert lib.fa_decode_workspace_size(2, 4, 33, 4096, 128, ctypes.byref(n)) == SHAPE
    assert lib.fa_decode_workspace_size(2, 4, 8, 4096, 96, ctypes.byref(n)) == SHAPE
    # work-items per launch stay below 2^32: the merge runs B*H*Nq*d of them,
    # the key split 64 per chunk with up to B*H + 1024 chunks
    assert lib.fa_decode_workspace_size(1, 1 << 20, 32, 1, 128, ctypes.byref(n)) == SHAPE
    assert lib.fa_decode_workspace_size(1, (1 << 20) - 1, 32, 1, 128, ctypes.byref(n)) == OK
    assert lib.fa_decode_workspace_size(1, (1 << 26) - 1024, 1, 1, 64, ctypes.byref(n)) == SHAPE
    assert lib.fa_decode_workspace_size(1, (1 << 26) - 1025, 1, 1, 64, ctypes.byref(n)) == OK
    ws = P[11]

    def dec(q=P[0], k=P[1], v=P[2], o=P[3], lse=P[4], Nq=16, Nk=64, d=128, scale=0.1,
            causal=1, w=ws, wb=need):
        return lib.fa_decode(q, k, v, o, lse, 1, 1, Nq, Nk, d, scale, causal, w, wb, STREAM)

    assert dec(Nq=33) == SHAPE
    assert dec(scale=float("nan")) == SCALE
    assert dec(causal=2) == MASK
    assert dec(q=None) == NULL
    assert dec(k=None) == NULL
    assert dec(o=ctypes.c_void_p(0x40008)) == ALIGN
    assert dec(w=None) == WS
    assert dec(wb=need - 1) == WS
    assert dec(o=ctypes.c_void_p(0x10000 + 32)) == ALIAS          # o inside q
    assert dec(Nq=0) == OK and dec(q=None, Nq=0) == OK              # nothing to do


def test_kv_outer_rejects_bad_arguments(lib):
    n = ctypes.c_size_t()
    assert lib.fa_fwd_kv_outer_workspace_size(1, 2, 100, 64, ctypes.byref(n)) == OK
    r256 = lambda x: (x + 255) // 256 * 256  # noqa: E731
    assert n.value == r256(2 * 100 * 64 * 4) + 2 * r256(2 * 100 * 4)
    need = n.value

    def kvo(q=P[0], o=P[3], causal=1, w=P[10], wb=need, d=64):
        return lib.fa_fwd_kv_outer(q, P[1], P[2], o, P[4], 1, 2, 100, d, 0.125, causal, w, wb,
                                   STREAM)

    assert kvo(d=80) == SHAPE
    assert kvo(causal=3) == MASK
    assert kvo(q=None) == NULL
    assert kvo(w=None) == WS and kvo(wb=need - 4) == WS
    assert kvo(o=ctypes.c_void_p(0x10000 + 16)) == ALIAS
