"""ctypes binding of libfa.so (include/fa.h). Argument marshalling only.

Every computation runs in the library's HIP kernels; PyTorch provides device
memory (output and workspace tensors) and the current stream. There is no
fallback: if the library is missing or the device is not a GPU, calls raise.
"""
from __future__ import annotations

import ctypes
import math
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libfa.so")

FA_MASK_CAUSAL = 1
FA_MASK_BLOCK = 2
MASK_BLOCK_SIZE = 128

EXPORTS = ("fa_fwd", "fa_bwd", "fa_bwd_workspace_size", "fa_bwd_preprocess", "fa_bwd_dkdv",
           "fa_bwd_dq", "fa_decode_workspace_size", "fa_decode", "fa_fwd_kv_outer_workspace_size",
           "fa_fwd_kv_outer", "fa_softmax_rows", "fa_bwd_noalloc", "fa_strerror")


class FaError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"fa status {status}: {msg}")
        self.status = status


class FaMask(ctypes.Structure):
    _fields_ = [("kind", ctypes.c_int32), ("block", ctypes.c_int32),
                ("blocks", ctypes.c_void_p), ("bh_stride", ctypes.c_int64)]


_lib = None


def load() -> ctypes.CDLL:
    """Load libfa.so once; raise if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m exact_io_aware_61_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i32, f32, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    mp = ctypes.POINTER(FaMask)
    lib.fa_fwd.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, f32, mp, vp]
    lib.fa_bwd_workspace_size.argtypes = [i32, i32, i32, i32, ctypes.POINTER(sz)]
    lib.fa_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, f32, mp, vp,
                           sz, vp]
    lib.fa_bwd_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, f32,
                                   mp, vp]
    lib.fa_bwd_preprocess.argtypes = [vp, vp, vp, i32, i32, i32, i32, vp, sz, vp]
    lib.fa_bwd_dkdv.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, f32, mp, vp, sz, vp]
    lib.fa_bwd_dq.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, f32, mp, vp, sz, vp]
    lib.fa_softmax_rows.argtypes = [vp, vp, ctypes.c_int64, ctypes.c_int64, vp]
    lib.fa_decode_workspace_size.argtypes = [i32, i32, i32, i32, i32, ctypes.POINTER(sz)]
    lib.fa_decode.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, f32, i32, vp, sz, vp]
    lib.fa_fwd_kv_outer_workspace_size.argtypes = [i32, i32, i32, i32, ctypes.POINTER(sz)]
    lib.fa_fwd_kv_outer.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, f32, i32, vp, sz, vp]
    for name in EXPORTS[:-1]:
        getattr(lib, name).restype = ctypes.c_int
    lib.fa_strerror.argtypes = [ctypes.c_int]
    lib.fa_strerror.restype = ctypes.c_char_p
    _lib = lib
    return lib


def strerror(status: int) -> str:
    return load().fa_strerror(status).decode()


def _check(status: int):
    if status != 0:
        raise FaError(status, strerror(status))


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(t: torch.Tensor):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _shape(q: torch.Tensor, *others):
    if q.dim() != 4:
        raise ValueError("expected [B, H, N, d] tensors")
    for t in (q,) + others:
        if t.shape != q.shape or t.dtype != torch.bfloat16 or not t.is_contiguous():
            raise ValueError("q, k, v (and o, dO) must be contiguous bf16 tensors of one shape")
        if not t.is_cuda or t.device != q.device:
            raise ValueError("tensors must live on the same GPU")
    return tuple(int(x) for x in q.shape)


def _like(t, shape, dtype, device, name: str):
    """A caller-supplied output (or the lse input): contiguous, of this shape and dtype,
    on this GPU. Checked before anything is launched: a wrong pointer here would
    reach the kernels as an out-of-bounds or host address."""
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name} must be a torch tensor")
    if tuple(t.shape) != tuple(shape) or t.dtype != dtype or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous {dtype} tensor of shape {tuple(shape)}, "
                         f"got {t.dtype} {tuple(t.shape)}"
                         f"{'' if t.is_contiguous() else ' (non-contiguous)'}")
    if not t.is_cuda or t.device != device:
        raise ValueError(f"{name} must live on {device}, got {t.device}")
    return t


def _ws_bytes(ws, device) -> int:
    """Size in bytes of a caller-supplied workspace tensor (any dtype), on this GPU."""
    if not isinstance(ws, torch.Tensor) or not ws.is_cuda or ws.device != device:
        raise ValueError(f"the workspace must be a tensor on {device}")
    if not ws.is_contiguous():
        raise ValueError("the workspace must be contiguous")
    return int(ws.numel()) * int(ws.element_size())


def _mask(causal: bool, block_mask, B: int, H: int, N: int, device):
    """Build the fa_mask_t (or None) and keep the grid tensor alive alongside it."""
    kind = FA_MASK_CAUSAL if causal else 0
    grid = None
    stride = 0
    if block_mask is not None:
        nb = -(-N // MASK_BLOCK_SIZE)
        grid = torch.as_tensor(block_mask).to(device=device, dtype=torch.uint8).contiguous()
        if grid.shape == (nb, nb):
            stride = 0
        elif grid.shape == (B, H, nb, nb):
            stride = nb * nb
        else:
            raise ValueError(f"block_mask must be [{nb}, {nb}] or [B, H, {nb}, {nb}]")
        kind |= FA_MASK_BLOCK
    if kind == 0:
        return None, None
    m = FaMask(kind, MASK_BLOCK_SIZE, None if grid is None else grid.data_ptr(), stride)
    return ctypes.byref(m), (m, grid)


def default_scale(d: int) -> float:
    return 1.0 / math.sqrt(d)


def forward(q, k, v, *, causal: bool = False, block_mask=None, scale: float | None = None,
            out=None, lse=None):
    """(o, lse) = attention forward. q, k, v: [B, H, N, d] bf16 on one GPU."""
    B, H, N, d = _shape(q, k, v)
    scale = default_scale(d) if scale is None else float(scale)
    o = torch.empty_like(q) if out is None else _like(out, q.shape, torch.bfloat16, q.device,
                                                         "out")
    lse = (torch.empty((B, H, N), device=q.device, dtype=torch.float32) if lse is None
           else _like(lse, (B, H, N), torch.float32, q.device, "lse"))
    mptr, keep = _mask(causal, block_mask, B, H, N, q.device)
    _check(load().fa_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H, N, d, scale, mptr,
                         _stream(q)))
    del keep
    return o, lse


def bwd_workspace_size(B: int, H: int, N: int, d: int) -> int:
    n = ctypes.c_size_t(0)
    _check(load().fa_bwd_workspace_size(B, H, N, d, ctypes.byref(n)))
    return int(n.value)


def workspace(q: torch.Tensor) -> torch.Tensor:
    B, H, N, d = (int(x) for x in q.shape)
    return torch.empty(max(bwd_workspace_size(B, H, N, d), 16), device=q.device, dtype=torch.uint8)


def backward(q, k, v, o, lse, do, *, causal: bool = False, block_mask=None,
             scale: float | None = None, ws=None, dq=None, dk=None, dv=None):
    """(dq, dk, dv) for upstream gradient do, recomputing P from lse."""
    B, H, N, d = _shape(q, k, v, o, do)
    scale = default_scale(d) if scale is None else float(scale)
    _like(lse, (B, H, N), torch.float32, q.device, "lse")
    ws = workspace(q) if ws is None else ws
    ws_bytes = _ws_bytes(ws, q.device)
    outs = []
    for name, t in (("dq", dq), ("dk", dk), ("dv", dv)):
        outs.append(torch.empty_like(q) if t is None
                    else _like(t, q.shape, torch.bfloat16, q.device, name))
    dq, dk, dv = outs
    mptr, keep = _mask(causal, block_mask, B, H, N, q.device)
    _check(load().fa_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(do), _ptr(lse), _ptr(dq),
                         _ptr(dk), _ptr(dv), B, H, N, d, scale, mptr, _ptr(ws), ws_bytes,
                         _stream(q)))
    del keep
    return dq, dk, dv


def bwd_preprocess(o, do, lse, ws):
    B, H, N, d = _shape(o, do)
    _like(lse, (B, H, N), torch.float32, o.device, "lse")
    _check(load().fa_bwd_preprocess(_ptr(o), _ptr(do), _ptr(lse), B, H, N, d, _ptr(ws),
                                    _ws_bytes(ws, o.device), _stream(o)))


def bwd_dkdv(q, k, v, do, dk, dv, ws, *, causal=False, block_mask=None, scale=None):
    B, H, N, d = _shape(q, k, v, do)
    scale = default_scale(d) if scale is None else float(scale)
    _like(dk, q.shape, torch.bfloat16, q.device, "dk")
    _like(dv, q.shape, torch.bfloat16, q.device, "dv")
    ws_bytes = _ws_bytes(ws, q.device)
    mptr, keep = _mask(causal, block_mask, B, H, N, q.device)
    _check(load().fa_bwd_dkdv(_ptr(q), _ptr(k), _ptr(v), _ptr(do), _ptr(dk), _ptr(dv),
                              B, H, N, d, scale, mptr, _ptr(ws), ws_bytes, _stream(q)))
    del keep


def bwd_dq(q, k, v, do, dq, ws, *, causal=False, block_mask=None, scale=None):
    B, H, N, d = _shape(q, k, v, do)
    scale = default_scale(d) if scale is None else float(scale)
    _like(dq, q.shape, torch.bfloat16, q.device, "dq")
    ws_bytes = _ws_bytes(ws, q.device)
    mptr, keep = _mask(causal, block_mask, B, H, N, q.device)
    _check(load().fa_bwd_dq(_ptr(q), _ptr(k), _ptr(v), _ptr(do), _ptr(dq),
                            B, H, N, d, scale, mptr, _ptr(ws), ws_bytes, _stream(q)))
    del keep


def forward_kv_outer(q, k, v, *, causal: bool = False, scale: float | None = None):
    """The forward in the K/V-outer loop order (fa_fwd_kv_outer): same (o, lse) as forward()."""
    B, H, N, d = _shape(q, k, v)
    scale = default_scale(d) if scale is None else float(scale)
    n = ctypes.c_size_t()
    _check(load().fa_fwd_kv_outer_workspace_size(B, H, N, d, ctypes.byref(n)))
    ws = torch.empty(max(n.value, 16), device=q.device, dtype=torch.uint8)
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), device=q.device, dtype=torch.float32)
    _check(load().fa_fwd_kv_outer(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H, N, d, scale,
                                  1 if causal else 0, _ptr(ws), ws.numel(), _stream(q)))
    return o, lse


def decode(q, k, v, *, causal: bool = False, scale: float | None = None, ws=None):
    """Attention of the newest Nq queries q [B, H, Nq, d] over a cache k, v [B, H, Nk, d]
    (fa_decode). Returns (o [B, H, Nq, d] bf16, lse [B, H, Nq] float32)."""
    for t in (q, k, v):
        if t.dim() != 4 or t.dtype != torch.bfloat16 or not t.is_contiguous() or not t.is_cuda:
            raise ValueError("q, k, v must be contiguous 4-D bf16 GPU tensors")
    B, H, Nq, d = (int(x) for x in q.shape)
    if k.shape != v.shape or tuple(k.shape[:2]) != (B, H) or int(k.shape[3]) != d:
        raise ValueError("k and v must be [B, H, Nk, d] matching q")
    Nk = int(k.shape[2])
    scale = default_scale(d) if scale is None else float(scale)
    n = ctypes.c_size_t()
    _check(load().fa_decode_workspace_size(B, H, Nq, Nk, d, ctypes.byref(n)))
    if ws is None:
        ws = torch.empty(max(n.value, 16), device=q.device, dtype=torch.uint8)
    ws_bytes = _ws_bytes(ws, q.device)
    if k.device != q.device or v.device != q.device:
        raise ValueError("q, k, v must live on the same GPU")
    o = torch.empty_like(q)
    lse = torch.empty((B, H, Nq), device=q.device, dtype=torch.float32)
    _check(load().fa_decode(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H, Nq, Nk, d, scale,
                            1 if causal else 0, _ptr(ws), ws_bytes, _stream(q)))
    return o, lse


def softmax_rows(x: torch.Tensor, out: torch.Tensor | None = None) -> torch.Tensor:
    """Softmax over the last dimension of a contiguous float32 GPU tensor (fa_softmax_rows).

    `out` may be `x` itself (in place) or a separate tensor of the same shape.
    """
    if x.dtype != torch.float32 or not x.is_cuda or not x.is_contiguous() or x.dim() < 1:
        raise ValueError("softmax_rows needs a contiguous float32 GPU tensor")
    y = torch.empty_like(x) if out is None else out
    if y.shape != x.shape or y.dtype != x.dtype or not y.is_contiguous() or y.device != x.device:
        raise ValueError("out must be a contiguous float32 tensor shaped like x on the same GPU")
    cols = int(x.shape[-1])
    rows = int(x.numel() // cols) if cols else 0
    _check(load().fa_softmax_rows(_ptr(x), _ptr(y), rows, cols, _stream(x)))
    return y


class _AttentionFn(torch.autograd.Function):
    @staticmethod
    def forward(ctx, q, k, v, causal, block_mask, scale):
        o, lse = forward(q, k, v, causal=causal, block_mask=block_mask, scale=scale)
        ctx.save_for_backward(q, k, v, o, lse)
        ctx.args = (causal, block_mask, scale)
        return o

    @staticmethod
    def backward(ctx, do):
        q, k, v, o, lse = ctx.saved_tensors
        causal, block_mask, scale = ctx.args
        dq, dk, dv = backward(q, k, v, o, lse, do.contiguous(), causal=causal,
                              block_mask=block_mask, scale=scale)
        return dq, dk, dv, None, None, None


def attention(q, k, v, *, causal: bool = False, block_mask=None, scale: float | None = None):
    """Differentiable O = softmax(scale Q K^T, masked) V through the HIP kernels."""
    return _AttentionFn.apply(q, k, v, causal, block_mask, scale)
