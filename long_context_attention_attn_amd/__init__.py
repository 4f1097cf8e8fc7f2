"""MI355X (gfx950) lightning-attention forward: prefill and decode.

Thin Python binding over the C ABI of ``liblightning_attn.so`` (declared in
``include/lightning_attn.h``).  This module only marshals arguments: it checks tensor
devices/dtypes/shapes, allocates outputs with torch (device memory), passes raw pointers and
the current HIP stream, and turns status codes into exceptions.  Every step of the
computation runs in the library's HIP kernels; there is no other implementation behind these
functions, and they raise if the compiled library is missing.

Lightning attention ("MiniMax-01 technical report digest", futurefh.com, section 1): causal
linear attention computed block-wise with an intra-block left product and an inter-block
right product over a running state; with a constant per-head decay lambda_h,
    o_t = sum_{s<=t} lambda^(t-s) (q_t . k_s) v_s  (+ lambda^(t+1) q_t S0 with an initial state)
Decode updates the fixed-size state once per token: S' = lambda S + k^T v, o = q S'.
"""
from __future__ import annotations

from typing import Optional, Tuple, Union

import torch

from . import _lib

__all__ = ["prefill", "backward", "lightning_attention", "decode_step", "decode_tokens",
           "LightningAttnError", "library_path"]

LightningAttnError = _lib.LightningAttnError
library_path = _lib.library_path

_DTYPES = {torch.float32: _lib.LA_F32, torch.bfloat16: _lib.LA_BF16}


def _check_act(name, x, dtype, device):
    if not isinstance(x, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor" % name)
    if x.device != device:
        raise ValueError("%s is on %s, expected %s" % (name, x.device, device))
    if x.dtype != dtype:
        raise ValueError("%s has dtype %s, expected %s" % (name, x.dtype, dtype))
    if not x.is_contiguous():
        raise ValueError("%s must be contiguous" % name)


def _stream_ptr(device) -> int:
    return int(torch.cuda.current_stream(device).cuda_stream)


def prefill(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, decay: torch.Tensor,
            cu_seqlens: Optional[torch.Tensor] = None, *,
            initial_state: Optional[torch.Tensor] = None,
            out: Optional[torch.Tensor] = None,
            final_state: Optional[torch.Tensor] = None,
            return_final_state: bool = True,
            split: Union[None, str, int] = None,
            static_scratch: bool = False,
            block_size: int = 0) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """Lightning-attention prefill over packed sequences.

    q, k, v: [T, H, D] bf16 or fp32 (same dtype), contiguous, on a gfx950 device.
    decay: [H] fp32 on the same device.  cu_seqlens: [S+1] int32 on the device, or None for
    one sequence.  initial_state: optional [S, H, D, D] fp32.  Returns (out [T, H, D],
    final_state [S, H, D, D] fp32 or None).  Runs asynchronously on the current stream.

    split: None = one scan per (sequence, head); an int n >= 1 = the sequence-split prefill
    with segments of n 64-token blocks (a workspace is allocated with torch); "auto" = the
    sequence split with the segment length the library suggests for this device, or the plain
    scan when it suggests none.  All give the same result up to rounding order.
    block_size: 0 = the library's default, or 64 / 128 tokens per block (128: bf16 only; the
    sequence split ignores it and picks the block size by segment length).  Every block size
    gives the same result up to rounding.
    static_scratch: with a sequence split, keep its segment states in the library's static
    device scratch (la_prefill_split_static) instead of a torch-allocated workspace, so the
    library call allocates nothing; sizes with la_prefill_split_workspace_size <= 32 MiB
    always fit (larger ones fit if one state per segment does).  Calls
    that overlap in time on one device share that scratch and must be ordered on one stream.
    """
    device = q.device
    if q.dim() != 3:
        raise ValueError("q must be [T, H, D]")
    T, H, D = q.shape
    dtype = q.dtype
    if dtype not in _DTYPES:
        raise ValueError("unsupported dtype %s" % dtype)
    for name, x in (("k", k), ("v", v)):
        _check_act(name, x, dtype, device)
        if x.shape != q.shape:
            raise ValueError("%s has shape %s, expected %s" % (name, tuple(x.shape), tuple(q.shape)))
    _check_act("q", q, dtype, device)
    _check_act("decay", decay, torch.float32, device)
    if decay.shape != (H,):
        raise ValueError("decay must be [H]")
    if cu_seqlens is not None:
        _check_act("cu_seqlens", cu_seqlens, torch.int32, device)
        if cu_seqlens.dim() != 1 or cu_seqlens.numel() < 2:
            raise ValueError("cu_seqlens must be [S+1] with S >= 1")
        S = cu_seqlens.numel() - 1
    else:
        S = 1
    if initial_state is not None:
        _check_act("initial_state", initial_state, torch.float32, device)
        if initial_state.shape != (S, H, D, D):
            raise ValueError("initial_state must be [S, H, D, D]")
    if out is None:
        out = torch.empty_like(q)
    else:
        _check_act("out", out, dtype, device)
        if out.shape != q.shape:
            raise ValueError("out must be [T, H, D]")
    if final_state is None and return_final_state:
        final_state = torch.empty((S, H, D, D), dtype=torch.float32, device=device)
    elif final_state is not None:
        _check_act("final_state", final_state, torch.float32, device)
        if final_state.shape != (S, H, D, D):
            raise ValueError("final_state must be [S, H, D, D]")
    seg_blocks = _seg_blocks(split, T, S, H, D, dtype)
    ptrs = (q.data_ptr(), k.data_ptr(), v.data_ptr(), decay.data_ptr(),
            0 if cu_seqlens is None else cu_seqlens.data_ptr(),
            0 if initial_state is None else initial_state.data_ptr(),
            out.data_ptr(), 0 if final_state is None else final_state.data_ptr())
    if seg_blocks > 0 and static_scratch:
        _lib.prefill_split_static(*ptrs, T, S, H, D, _DTYPES[dtype], seg_blocks,
                                  _stream_ptr(device))
    elif seg_blocks > 0:
        nbytes = _lib.prefill_split_workspace_size(T, S, H, D, seg_blocks)
        ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=device)
        # ws is allocated on the current stream, so torch's caching allocator reuses its memory
        # only for work queued after these kernels on that stream
        _lib.prefill_split(*ptrs, T, S, H, D, _DTYPES[dtype], seg_blocks, ws.data_ptr(), nbytes,
                           _stream_ptr(device))
    else:
        _lib.prefill_with_block_size(*ptrs, T, S, H, D, _DTYPES[dtype], block_size,
                                     _stream_ptr(device))
    return out, final_state


def _seg_blocks(split, T, S, H, D, dtype) -> int:
    """Segment length (in 64-token blocks) for ``split``; 0 = no sequence split."""
    if split == "auto":
        return _lib.prefill_split_blocks(T, S, H, D, _DTYPES[dtype])
    if split is None:
        return 0
    if isinstance(split, bool) or not isinstance(split, int) or split < 1:
        raise ValueError("split must be None, 'auto' or an int >= 1")
    return split


def backward(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, decay: torch.Tensor,
             d_out: torch.Tensor, cu_seqlens: Optional[torch.Tensor] = None, *,
             initial_state: Optional[torch.Tensor] = None,
             d_final_state: Optional[torch.Tensor] = None,
             want_d_initial_state: bool = True, split: Union[None, str, int] = None):
    """Gradients of the prefill: (dq, dk, dv [T, H, D], d_initial_state [S, H, D, D] or None).

    q, k, v, decay, cu_seqlens, initial_state: the prefill's inputs; d_out [T, H, D] (same dtype
    as q) is dL/dout, d_final_state [S, H, D, D] fp32 (or None = 0) is dL/dfinal_state.
    split: as for prefill (the sequence-split form of the three gradient scans)."""
    device = q.device
    if q.dim() != 3:
        raise ValueError("q must be [T, H, D]")
    T, H, D = q.shape
    dtype = q.dtype
    if dtype not in _DTYPES:
        raise ValueError("unsupported dtype %s" % dtype)
    for name, x in (("q", q), ("k", k), ("v", v), ("d_out", d_out)):
        _check_act(name, x, dtype, device)
        if x.shape != q.shape:
            raise ValueError("%s must be [T, H, D]" % name)
    _check_act("decay", decay, torch.float32, device)
    if decay.shape != (H,):
        raise ValueError("decay must be [H]")
    if cu_seqlens is not None:
        _check_act("cu_seqlens", cu_seqlens, torch.int32, device)
        if cu_seqlens.dim() != 1 or cu_seqlens.numel() < 2:
            raise ValueError("cu_seqlens must be [S+1] with S >= 1")
        S = cu_seqlens.numel() - 1
    else:
        S = 1
    for name, x in (("initial_state", initial_state), ("d_final_state", d_final_state)):
        if x is not None:
            _check_act(name, x, torch.float32, device)
            if x.shape != (S, H, D, D):
                raise ValueError("%s must be [S, H, D, D]" % name)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(q), torch.empty_like(q)
    d_init = (torch.empty((S, H, D, D), dtype=torch.float32, device=device)
              if want_d_initial_state else None)
    ptrs = (q.data_ptr(), k.data_ptr(), v.data_ptr(), decay.data_ptr(),
            0 if cu_seqlens is None else cu_seqlens.data_ptr(),
            0 if initial_state is None else initial_state.data_ptr(), d_out.data_ptr(),
            0 if d_final_state is None else d_final_state.data_ptr(), dq.data_ptr(),
            dk.data_ptr(), dv.data_ptr(), 0 if d_init is None else d_init.data_ptr())
    seg_blocks = _seg_blocks(split, T, S, H, D, dtype)
    if seg_blocks > 0:
        nbytes = _lib.prefill_split_workspace_size(T, S, H, D, seg_blocks)
        ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=device)
        _lib.backward_split(*ptrs, T, S, H, D, _DTYPES[dtype], seg_blocks, ws.data_ptr(), nbytes,
                            _stream_ptr(device))
    else:
        _lib.backward(*ptrs, T, S, H, D, _DTYPES[dtype], _stream_ptr(device))
    return dq, dk, dv, d_init


class _LightningAttention(torch.autograd.Function):
    """prefill as a differentiable op (gradients for q, k, v and the initial state)."""

    @staticmethod
    def forward(ctx, q, k, v, decay, cu_seqlens, initial_state, split):
        out, fs = prefill(q, k, v, decay, cu_seqlens, initial_state=initial_state, split=split)
        ctx.save_for_backward(q, k, v, decay, cu_seqlens, initial_state)
        ctx.split = split
        return out, fs

    @staticmethod
    def backward(ctx, d_out, d_fs):
        q, k, v, decay, cu_seqlens, initial_state = ctx.saved_tensors
        dq, dk, dv, d_init = backward(
            q, k, v, decay, d_out.contiguous(), cu_seqlens, initial_state=initial_state,
            d_final_state=None if d_fs is None else d_fs.contiguous(),
            want_d_initial_state=initial_state is not None and ctx.needs_input_grad[5],
            split=ctx.split)
        return dq, dk, dv, None, None, d_init, None


def lightning_attention(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, decay: torch.Tensor,
                        cu_seqlens: Optional[torch.Tensor] = None,
                        initial_state: Optional[torch.Tensor] = None,
                        split: Union[None, str, int] = None):
    """Differentiable prefill: (out, final_state); backward runs the library's gradient
    scans (sequence-split too when ``split`` is given).  decay and cu_seqlens get no
    gradient."""
    return _LightningAttention.apply(q, k, v, decay, cu_seqlens, initial_state, split)


def decode_step(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, decay: torch.Tensor,
                state: torch.Tensor, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """One recurrent decode step; ``state`` [Bt, H, D, D] fp32 is updated in place.

    q, k, v: [Bt, H, D] bf16 or fp32; decay [H] fp32.  Returns out [Bt, H, D]."""
    device = q.device
    if q.dim() != 3:
        raise ValueError("q must be [Bt, H, D]")
    Bt, H, D = q.shape
    dtype = q.dtype
    if dtype not in _DTYPES:
        raise ValueError("unsupported dtype %s" % dtype)
    for name, x in (("q", q), ("k", k), ("v", v)):
        _check_act(name, x, dtype, device)
        if x.shape != q.shape:
            raise ValueError("%s must be [Bt, H, D]" % name)
    _check_act("decay", decay, torch.float32, device)
    if decay.shape != (H,):
        raise ValueError("decay must be [H]")
    _check_act("state", state, torch.float32, device)
    if state.shape != (Bt, H, D, D):
        raise ValueError("state must be [Bt, H, D, D]")
    if out is None:
        out = torch.empty_like(q)
    else:
        _check_act("out", out, dtype, device)
        if out.shape != q.shape:
            raise ValueError("out must be [Bt, H, D]")
    _lib.decode_step(q.data_ptr(), k.data_ptr(), v.data_ptr(), decay.data_ptr(), state.data_ptr(),
                     out.data_ptr(), Bt, H, D, _DTYPES[dtype], _stream_ptr(device))
    return out


def decode_tokens(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, decay: torch.Tensor,
                  state: torch.Tensor, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """m decode steps per sequence in one pass; ``state`` [Bt, H, D, D] fp32 is updated in place.

    q, k, v: [Bt, m, H, D] bf16 or fp32 (token i of sequence b at [b, i]); decay [H] fp32.
    Returns out [Bt, m, H, D]."""
    device = q.device
    if q.dim() != 4:
        raise ValueError("q must be [Bt, m, H, D]")
    Bt, m, H, D = q.shape
    dtype = q.dtype
    if dtype not in _DTYPES:
        raise ValueError("unsupported dtype %s" % dtype)
    for name, x in (("q", q), ("k", k), ("v", v)):
        _check_act(name, x, dtype, device)
        if x.shape != q.shape:
            raise ValueError("%s must be [Bt, m, H, D]" % name)
    _check_act("decay", decay, torch.float32, device)
    if decay.shape != (H,):
        raise ValueError("decay must be [H]")
    _check_act("state", state, torch.float32, device)
    if state.shape != (Bt, H, D, D):
        raise ValueError("state must be [Bt, H, D, D]")
    if out is None:
        out = torch.empty_like(q)
    else:
        _check_act("out", out, dtype, device)
        if out.shape != q.shape:
            raise ValueError("out must be [Bt, m, H, D]")
    _lib.decode_tokens(q.data_ptr(), k.data_ptr(), v.data_ptr(), decay.data_ptr(),
                       state.data_ptr(), out.data_ptr(), Bt, m, H, D, _DTYPES[dtype],
                       _stream_ptr(device))
    return out
