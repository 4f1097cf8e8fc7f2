"""Serving helpers: multi-level padding buckets and graph-captured prefill.

The inference framework the pages describe pads batches to a few size levels so that few
distinct shapes have to be prepared, and keeps padding small by making the levels finer where
sizes are small ("MiniMax-01 technical report digest", futurefh.com, section 3: multi-level
padding; separate prefill and decode).  The prefill kernels here take packed ragged batches
(cu_seqlens) directly, so padding is never needed for correctness; it is needed to replay one
captured HIP graph for many batches, since a graph fixes every launch's grid and pointers.

A padded batch keeps the real sequences first, then one filler sequence that holds the padding
tokens, then empty sequences up to the padded sequence count.  Sequences are independent, so
the filler never changes a real output and empty sequences cost one short workgroup each.
"""
from __future__ import annotations

import bisect
from typing import List, Optional, Sequence, Tuple

import torch

from . import prefill


def multilevel(limit: int, first_step: int = 64, steps_per_level: int = 8) -> List[int]:
    """Padding levels up to (at least) ``limit``: multiples of ``first_step`` up to
    X0 = first_step * steps_per_level, then ``steps_per_level`` evenly spaced levels in every
    octave (X, 2X], X = X0, 2 X0, ...  A size n is then padded by less than
    max(first_step, n / steps_per_level)."""
    if limit < 1 or first_step < 1 or steps_per_level < 1:
        raise ValueError("limit, first_step and steps_per_level must be >= 1")
    levels = [first_step * i for i in range(1, steps_per_level + 1)]
    X = first_step * steps_per_level
    while levels[-1] < limit:
        step = X // steps_per_level
        levels += [X + step * i for i in range(1, steps_per_level + 1)]
        X *= 2
    return levels


def pad_to_level(n: int, levels: Sequence[int]) -> int:
    """Smallest level >= n (levels sorted ascending)."""
    i = bisect.bisect_left(levels, n)
    if i == len(levels):
        raise ValueError("size %d exceeds the largest level %d" % (n, levels[-1]))
    return levels[i]


def padded_batch(lengths: Sequence[int], token_levels: Sequence[int],
                 seq_levels: Sequence[int]) -> Tuple[int, int, List[int]]:
    """(T_pad, S_pad, cu_seqlens) for a batch of sequence lengths: T_pad and S_pad are levels,
    the real sequences come first, then a filler sequence of T_pad - T tokens (if any), then
    empty sequences.  S_pad counts real + filler + empty sequences."""
    if any(n < 0 for n in lengths):
        raise ValueError("negative sequence length")
    T = int(sum(lengths))
    T_pad = pad_to_level(max(T, 1), token_levels)
    S_real = len(lengths) + (1 if T_pad > T else 0)
    S_pad = pad_to_level(max(S_real, 1), seq_levels)
    cu = [0]
    for n in lengths:
        cu.append(cu[-1] + int(n))
    while len(cu) < S_pad + 1:
        cu.append(T_pad)
    return T_pad, S_pad, cu


class GraphedPrefill:
    """The prefill for one padded shape (T_pad tokens, S_pad sequences, H heads, head dim D),
    captured once in a HIP graph and replayed for any batch that fits.

    Inputs are copied into the graph's static buffers; outputs are views of its static output
    buffers, valid until the next call.  Not thread-safe; one stream."""

    def __init__(self, T_pad: int, S_pad: int, H: int, D: int, dtype=torch.bfloat16,
                 device="cuda", with_initial_state: bool = False, split=None,
                 static_scratch: bool = False):
        self.T_pad, self.S_pad, self.H, self.D = T_pad, S_pad, H, D
        dev = torch.device(device)
        self.q = torch.zeros((T_pad, H, D), dtype=dtype, device=dev)
        self.k = torch.zeros_like(self.q)
        self.v = torch.zeros_like(self.q)
        self.out = torch.empty_like(self.q)
        self.decay = torch.zeros((H,), dtype=torch.float32, device=dev)
        self.cu = torch.zeros((S_pad + 1,), dtype=torch.int32, device=dev)
        self.init = (torch.zeros((S_pad, H, D, D), dtype=torch.float32, device=dev)
                     if with_initial_state else None)
        self.final_state = torch.empty((S_pad, H, D, D), dtype=torch.float32, device=dev)
        self._split = split
        # with a split: keep the segment states in the library's static scratch, so the captured
        # launches allocate nothing (no workspace from the graph's memory pool); replays of
        # graphs that share one device's scratch must not overlap in time
        self._static = static_scratch
        self.cu[:] = torch.tensor([0] + [T_pad] * S_pad, dtype=torch.int32)
        # warm up (library load, device check) outside the capture
        s = torch.cuda.Stream(device=dev)
        s.wait_stream(torch.cuda.current_stream(dev))
        with torch.cuda.stream(s):
            self._launch()
        torch.cuda.current_stream(dev).wait_stream(s)
        torch.cuda.synchronize(dev)
        self.graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(self.graph):
            self._launch()

    def _launch(self):
        prefill(self.q, self.k, self.v, self.decay, self.cu, initial_state=self.init,
                out=self.out, final_state=self.final_state, split=self._split,
                static_scratch=self._static)

    def __call__(self, q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, decay: torch.Tensor,
                 lengths: Sequence[int], initial_state: Optional[torch.Tensor] = None):
        """Prefill of the packed batch q, k, v [T, H, D] with sequence lengths ``lengths``
        (sum = T); returns (out [T, H, D], final_state [len(lengths), H, D, D]) as views."""
        T = int(sum(lengths))
        if q.shape != (T, self.H, self.D):
            raise ValueError("q must be [sum(lengths), H, D]")
        S = len(lengths)
        need_filler = T < self.T_pad
        if T > self.T_pad or S + (1 if need_filler else 0) > self.S_pad:
            raise ValueError("batch (T=%d, S=%d) exceeds the captured shape (%d, %d)"
                             % (T, S, self.T_pad, self.S_pad))
        cu = [0]
        for n in lengths:
            cu.append(cu[-1] + int(n))
        cu += [self.T_pad] * (self.S_pad + 1 - len(cu))
        self.q[:T].copy_(q)
        self.k[:T].copy_(k)
        self.v[:T].copy_(v)
        self.decay.copy_(decay)
        self.cu.copy_(torch.tensor(cu, dtype=torch.int32), non_blocking=False)
        if self.init is not None:
            if initial_state is None:
                self.init.zero_()
            else:
                self.init[:S].copy_(initial_state)
        elif initial_state is not None:
            raise ValueError("this graph was captured without an initial state")
        self.graph.replay()
        return self.out[:T], self.final_state[:S]

