"""Exact, IO-aware attention for AMD Instinct MI355X (gfx950).

O = softmax(scale Q K^T [causal and/or 128x128 block mask]) V and its
gradients, computed by hand-written HIP kernels (libfa.so, C ABI in
include/fa.h) that never write the N x N score or probability matrices to
device memory. This package is the thin Python binding:

    from exact_io_aware_61_amd import forward, backward, attention
    o, lse = forward(q, k, v, causal=True)
    dq, dk, dv = backward(q, k, v, o, lse, do, causal=True)
    o = attention(q, k, v, causal=True)      # torch.autograd-aware
    y = softmax_rows(x)                      # row softmax, online normalizer
    o, lse = decode(q_new, k_cache, v_cache, causal=True)   # newest queries vs a KV cache

Build the library first: python -m exact_io_aware_61_amd.build
"""
from ._binding import (EXPORTS, FA_MASK_BLOCK, FA_MASK_CAUSAL, LIB_PATH, MASK_BLOCK_SIZE, FaError,
                       attention, backward, bwd_dkdv, bwd_dq, bwd_preprocess, decode,
                       forward_kv_outer,
                       bwd_workspace_size, default_scale, forward, load, softmax_rows, strerror,
                       workspace)

__all__ = ["EXPORTS", "FA_MASK_BLOCK", "FA_MASK_CAUSAL", "LIB_PATH", "MASK_BLOCK_SIZE", "FaError",
           "attention", "backward", "bwd_dkdv", "bwd_dq", "bwd_preprocess", "decode",
           "forward_kv_outer",
           "bwd_workspace_size", "default_scale", "forward", "load", "softmax_rows", "strerror",
           "workspace"]
