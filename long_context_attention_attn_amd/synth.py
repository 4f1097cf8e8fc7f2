"""Seeded synthetic inputs shaped like the lightning-attention layers of MiniMax-Text-01.

This module only draws random numbers and builds shapes; it holds none of the attention
arithmetic.  It is the one piece of code that both the GPU library's tests/benchmark and the
CPU oracle's callers use, so that both sides see bit-identical inputs.

Recipes (the pages give none; these are the stated workloads of this library):

* q, k, v ~ N(0, 1) / sqrt(D), drawn in fp32 in the order q, k, v, then cast with
  ``Tensor.to(dtype)`` (round to nearest even for bf16).
* decay: ``lambda_h = lo * (hi / lo) ** (h / (H - 1))`` -- geometric from ``lo`` to ``hi``
  over the heads (``lo`` for H = 1).
* varlen lengths: ``numpy.random.default_rng(seed).integers(lo, hi + 1, n)``.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import List, Optional

import numpy as np
import torch


def decay_geometric(H: int, lo: float, hi: float) -> torch.Tensor:
    """fp32 [H] decays geometric from lo (head 0) to hi (head H-1)."""
    if H == 1:
        vals = [lo]
    else:
        vals = [lo * (hi / lo) ** (h / (H - 1)) for h in range(H)]
    return torch.tensor(vals, dtype=torch.float32)


def varlen_lengths(n: int, lo: int, hi: int, seed: int) -> List[int]:
    """n sequence lengths uniform in [lo, hi] (inclusive)."""
    return [int(x) for x in np.random.default_rng(seed).integers(lo, hi + 1, n)]


def cu_from_lengths(lengths) -> torch.Tensor:
    """int32 [S+1] prefix offsets of packed sequences."""
    cu = [0]
    for n in lengths:
        cu.append(cu[-1] + int(n))
    return torch.tensor(cu, dtype=torch.int32)


def qkv(T: int, H: int, D: int, dtype: torch.dtype, seed: int, device="cpu",
        chunk_tokens: int = 1 << 16):
    """q, k, v each [T, H, D] ~ N(0,1)/sqrt(D) in ``dtype``.

    Drawn with a ``torch.Generator`` on ``device`` seeded with ``seed``; large tensors are drawn
    in fp32 chunks of ``chunk_tokens`` tokens (q entirely first, then k, then v), so the values
    depend only on (T, H, D, seed, device, chunk_tokens)."""
    dev = torch.device(device)
    g = torch.Generator(device=dev)
    g.manual_seed(seed)
    scale = 1.0 / math.sqrt(D)
    outs = []
    for _ in range(3):
        t = torch.empty((T, H, D), dtype=dtype, device=dev)
        for c0 in range(0, T, chunk_tokens):
            c1 = min(T, c0 + chunk_tokens)
            x = torch.randn((c1 - c0, H, D), generator=g, dtype=torch.float32, device=dev)
            t[c0:c1] = (x * scale).to(dtype)
        outs.append(t)
    return tuple(outs)


def ones(T: int, H: int, D: int, dtype: torch.dtype, device="cpu"):
    """q = k = v = 1 (the ones-vector case)."""
    t = torch.ones((T, H, D), dtype=dtype, device=device)
    return t, t.clone(), t.clone()


@dataclass
class Workload:
    """A named synthetic workload."""

    name: str
    H: int
    D: int
    dtype: torch.dtype
    decay_lo: float
    decay_hi: float
    lengths: List[int] = field(default_factory=list)
    seed: int = 0
    note: str = ""

    @property
    def T(self) -> int:
        return int(sum(self.lengths))

    @property
    def S(self) -> int:
        return len(self.lengths)

    def decay(self) -> torch.Tensor:
        return decay_geometric(self.H, self.decay_lo, self.decay_hi)

    def cu_seqlens(self) -> Optional[torch.Tensor]:
        return cu_from_lengths(self.lengths)

    def inputs(self, device="cpu"):
        return qkv(self.T, self.H, self.D, self.dtype, self.seed, device=device)


def workloads():
    """The five stated workloads (sizes of the lightning layers of MiniMax-Text-01)."""
    return {
        # Tiny causal linear attention without decay, fp32, one head.
        "tiny_fp32": Workload("tiny_fp32", H=1, D=64, dtype=torch.float32, decay_lo=1.0,
                              decay_hi=1.0, lengths=[256], seed=0,
                              note="1 x 256 tokens, 1 head, D=64, fp32, lambda=1"),
        # Lightning prefill, 8 heads x 8192 tokens.
        "prefill_8k": Workload("prefill_8k", H=8, D=128, dtype=torch.bfloat16, decay_lo=0.9,
                               decay_hi=0.999, lengths=[8192], seed=0,
                               note="1 x 8192 tokens, 8 heads, D=128, bf16"),
        # One MiniMax-like layer: 64 heads x 65,536 tokens.
        "prefill_64k": Workload("prefill_64k", H=64, D=128, dtype=torch.bfloat16, decay_lo=0.9,
                                decay_hi=0.9999, lengths=[65536], seed=0,
                                note="1 x 65536 tokens, 64 heads, D=128, bf16"),
        # Packed varlen prefill: 16 sequences of 1024..32768 tokens.
        "varlen_16": Workload("varlen_16", H=64, D=128, dtype=torch.bfloat16, decay_lo=0.9,
                              decay_hi=0.9999, lengths=varlen_lengths(16, 1024, 32768, 0),
                              seed=0, note="16 packed sequences, 64 heads, D=128, bf16"),
        # Long context: one 1,048,576-token sequence.
        "prefill_1m": Workload("prefill_1m", H=64, D=128, dtype=torch.bfloat16, decay_lo=0.9,
                               decay_hi=0.9999, lengths=[1 << 20], seed=0,
                               note="1 x 1048576 tokens, 64 heads, D=128, bf16"),
    }


def decode_batch(Bt: int, H: int, D: int, dtype: torch.dtype, seed: int, device="cpu"):
    """One decode token per sequence: q, k, v [Bt, H, D] (same recipe as ``qkv``)."""
    return qkv(Bt, H, D, dtype, seed, device=device)


def random_state(Bt: int, H: int, D: int, seed: int, device="cpu", scale: float = 1.0):
    """fp32 [Bt, H, D, D] state ~ N(0, scale^2) (a stand-in for a prefilled state)."""
    g = torch.Generator(device=torch.device(device))
    g.manual_seed(seed)
    return torch.randn((Bt, H, D, D), generator=g, dtype=torch.float32,
                       device=torch.device(device)) * scale
