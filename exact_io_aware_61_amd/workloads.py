"""Seeded synthetic inputs for exact attention: the five workloads and their generators.

This module draws random numbers and nothing else: it holds none of the
attention arithmetic. Both the HIP path and the CPU oracle receive the arrays
it returns, so the two never disagree about their inputs.

Workloads (shapes follow the tiled-attention description: Q, K, V are N x d per
(batch, head); the block mask works at 128 x 128 granularity, as block-sparse
attention on page 1, "Block-Sparse FlashAttention", keeps or drops whole blocks):

  tiny      B=1 H=2  N=256   d=64  dense
  dense2k   B=8 H=16 N=2048  d=64  dense
  causal8k  B=2 H=16 N=8192  d=128 causal (query i sees keys j <= i)
  causal32k B=1 H=8  N=32768 d=128 causal
  sparse16k B=4 H=16 N=16384 d=64  128x128 block mask, off-diagonal blocks kept
                                   with probability 0.25, diagonal always kept

Recipe: one numpy PCG64 generator per workload, seeded 1000 + index (index 1..5
in the order above); Q, K, V, dO are drawn in that order as float32 N(0, 1)
of shape [B, H, N, d] and rounded to bfloat16 (round-to-nearest-even, torch's
conversion). scale = float32(1/sqrt(d)). The block mask uses its own generator
seeded 1000 + index + 1: uniform [0, 1) draws < p over an [N/128, N/128] grid,
then the diagonal set to 1; one mask shared by every (batch, head).
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np
import torch

BLOCK = 128  # block-mask granularity (rows and columns)


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    index: int          # 1-based position in the workload list; seeds derive from it
    B: int
    H: int
    N: int
    d: int
    causal: bool = False
    block_keep: float | None = None   # None = no block mask

    @property
    def seed(self) -> int:
        return 1000 + self.index

    @property
    def scale(self) -> float:
        """float32(1/sqrt(d)), returned as the Python float of that float32."""
        return float(np.float32(1.0 / math.sqrt(self.d)))


WORKLOADS = {
    "tiny": Workload("tiny", 1, 1, 2, 256, 64),
    "dense2k": Workload("dense2k", 2, 8, 16, 2048, 64),
    "causal8k": Workload("causal8k", 3, 2, 16, 8192, 128, causal=True),
    "causal32k": Workload("causal32k", 4, 1, 8, 32768, 128, causal=True),
    "sparse16k": Workload("sparse16k", 5, 4, 16, 16384, 64, block_keep=0.25),
}


def bf16_normal(rng: np.random.Generator, shape) -> torch.Tensor:
    """float32 N(0,1) draws rounded to bfloat16 (RNE); returned as a CPU bf16 tensor."""
    x = rng.standard_normal(size=shape, dtype=np.float32)
    return torch.from_numpy(x).to(torch.bfloat16)


def make_qkv(B: int, H: int, N: int, d: int, seed: int, with_do: bool = True):
    """Q, K, V (and dO) as CPU bf16 tensors [B, H, N, d], drawn in that order."""
    rng = np.random.default_rng(seed)
    shape = (B, H, N, d)
    q = bf16_normal(rng, shape)
    k = bf16_normal(rng, shape)
    v = bf16_normal(rng, shape)
    do = bf16_normal(rng, shape) if with_do else None
    return q, k, v, do


def make_rising_scores(B: int, H: int, N: int, d: int, seed: int, *, q_lead: float = 16.0,
                       k_ramp: float = 8.0, rising: float = 0.75, late_outliers: int = 0):
    """Q, K, V, dO whose scores grow (or shrink) steadily along each query row.

    The draws of make_qkv(B, H, N, d, seed), then head-dim component 0 replaced:
    every query row gets +q_lead (probability `rising`, from its own generator,
    seed + 7) or -q_lead there, and key j gets a ramp from -k_ramp to +k_ramp
    over j = 0 .. N-1. The score of a +q_lead row then grows by about
    2 * q_lead * k_ramp (times the softmax scale) from the first key to the
    last, so the running row maximum of a tiled sweep keeps moving long after
    the first tile; -q_lead rows peak at the first keys instead. With
    late_outliers = n, the last n keys get component 0 equal to 3 * k_ramp: a
    jump of the row maximum at the very end. All values are rounded to bf16
    like every other input.
    """
    q, k, v, do = make_qkv(B, H, N, d, seed)
    rng = np.random.default_rng(seed + 7)
    sign = np.where(rng.random((B, H, N)) < rising, 1.0, -1.0).astype(np.float32)
    qn = q.float().numpy()
    kn = k.float().numpy()
    qn[..., 0] = q_lead * sign
    kn[..., 0] = np.linspace(-k_ramp, k_ramp, N, dtype=np.float32)[None, None, :]
    if late_outliers:
        kn[..., N - late_outliers:, 0] = 3.0 * k_ramp
    return (torch.from_numpy(qn).to(torch.bfloat16), torch.from_numpy(kn).to(torch.bfloat16),
            v, do)


def variant(w: Workload, block_keep: float | None = None, causal: bool | None = None) -> Workload:
    """The workload with another block-mask keep probability and/or the causal mask added.

    Same shapes and seeds, so Q, K, V, dO are the same draws; the block mask is
    drawn from the workload's mask generator with the new probability. The name
    records the change, e.g. "sparse16k:keep=0.05+causal".
    """
    keep = w.block_keep if block_keep is None else float(block_keep)
    cz = w.causal if causal is None else bool(causal)
    tag = w.name
    if keep != w.block_keep:
        tag += f":keep={keep:g}"
    if cz != w.causal:
        tag += "+causal" if cz else "-causal"
    return dataclasses.replace(w, name=tag, block_keep=keep, causal=cz)


def make_block_mask(N: int, keep: float, seed: int, block: int = BLOCK) -> np.ndarray:
    """uint8 [nb, nb] with nb = ceil(N/block): 1 = keep. Bernoulli(keep) off the diagonal,
    diagonal kept."""
    nb = -(-N // block)
    rng = np.random.default_rng(seed)
    m = (rng.random((nb, nb)) < keep).astype(np.uint8)
    np.fill_diagonal(m, 1)
    return m


def make_inputs(w: Workload, with_do: bool = True):
    """(q, k, v, do, block_mask-or-None) for a workload, all on the CPU."""
    q, k, v, do = make_qkv(w.B, w.H, w.N, w.d, w.seed, with_do)
    mask = None
    if w.block_keep is not None:
        mask = make_block_mask(w.N, w.block_keep, w.seed + 1)
    return q, k, v, do, mask


def kept_fraction(N: int, causal: bool, block_mask: np.ndarray | None, block: int = BLOCK) -> float:
    """Fraction rho of (query, key) pairs that are attended (counting, no attention math).

    Used for the algorithmic FLOP count 4*B*H*N^2*d*rho.
    """
    if block_mask is None:
        return (N + 1) / (2 * N) if causal else 1.0
    if N % block:
        raise ValueError("kept_fraction counts whole mask blocks: N must be a multiple of block")
    nb = N // block
    if not causal:
        return float(block_mask.astype(np.int64).sum()) / (nb * nb)
    # causal AND block: kept off-diagonal blocks below the diagonal are full,
    # diagonal blocks are lower triangles of block*(block+1)/2 pairs
    m = block_mask.astype(np.int64)
    below = np.tril(m, -1).sum() * block * block
    diag = np.trace(m) * block * (block + 1) // 2
    return float(below + diag) / (N * N)
