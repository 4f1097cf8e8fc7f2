"""ctypes loader for liblightning_attn.so (the C ABI of include/lightning_attn.h).

The library is built in-tree by ``python -m long_context_attention_attn_amd.build`` (or the
repository's ``__graft_entry__.build()``).  torch is imported first so that the library binds
to the HIP runtime torch already loaded (one runtime per process, shared streams).  A missing
library is an error: there is no fallback implementation.
"""
from __future__ import annotations

import ctypes
import os
import threading

import torch  # noqa: F401  (must be loaded before the HIP library; see module docstring)

_HERE = os.path.dirname(os.path.abspath(__file__))
_PATH = os.path.join(_HERE, "liblightning_attn.so")

LA_OK, LA_ERR_INVALID_ARG, LA_ERR_UNSUPPORTED, LA_ERR_HIP = 0, 1, 2, 3
LA_F32, LA_BF16 = 0, 1
ABI_VERSION = 2  # LA_ABI_VERSION of include/lightning_attn.h

# Every symbol declared in include/lightning_attn.h.
EXPORTS = ("la_abi_version", "la_prefill", "la_prefill_ex", "la_prefill_with_block_size",
           "la_prefill_split",
           "la_prefill_split_static",
           "la_prefill_split_workspace_size", "la_prefill_split_blocks",
           "la_prefill_split_blocks_for", "la_backward",
           "la_backward_split",
           "la_decode_step", "la_decode_tokens",
           "la_status_str", "la_last_error")

_lock = threading.Lock()
_lib = None


class LightningAttnError(RuntimeError):
    """A non-OK status from the C ABI."""

    def __init__(self, status: int, detail: str):
        self.status = status
        super().__init__("%s: %s" % (_status_name(status), detail))


def library_path() -> str:
    return _PATH


def _status_name(s: int) -> str:
    return {0: "LA_OK", 1: "LA_ERR_INVALID_ARG", 2: "LA_ERR_UNSUPPORTED", 3: "LA_ERR_HIP"}.get(
        s, "LA_ERR_UNKNOWN(%d)" % s)


def load():
    """Load (once) and return the ctypes handle; raises if the library was not built."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(_PATH):
            raise RuntimeError(
                "liblightning_attn.so is not built (expected at %s); run "
                "`python -m long_context_attention_attn_amd.build`" % _PATH)
        lib = ctypes.CDLL(_PATH)
        vp, i32, i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
        lib.la_abi_version.argtypes = []
        lib.la_abi_version.restype = i32
        if lib.la_abi_version() != ABI_VERSION:
            raise RuntimeError(
                "liblightning_attn.so at %s has ABI version %d, expected %d; rebuild it with "
                "`python -m long_context_attention_attn_amd.build`"
                % (_PATH, lib.la_abi_version(), ABI_VERSION))
        lib.la_prefill.argtypes = [vp, vp, vp, vp, vp, vp, vp, i64, i32, i32, i32, ctypes.c_int, vp]
        lib.la_prefill.restype = ctypes.c_int
        lib.la_prefill_ex.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, i64, i32, i32, i32,
                                      ctypes.c_int, vp]
        lib.la_prefill_ex.restype = ctypes.c_int
        lib.la_prefill_with_block_size.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, i64, i32, i32,
                                                   i32, ctypes.c_int, i32, vp]
        lib.la_prefill_with_block_size.restype = ctypes.c_int
        lib.la_prefill_split.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, i64, i32, i32, i32,
                                         ctypes.c_int, i32, vp, ctypes.c_size_t, vp]
        lib.la_prefill_split.restype = ctypes.c_int
        lib.la_prefill_split_static.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, i64, i32, i32, i32,
                                                ctypes.c_int, i32, vp]
        lib.la_prefill_split_static.restype = ctypes.c_int
        lib.la_prefill_split_workspace_size.argtypes = [i64, i32, i32, i32, i32]
        lib.la_prefill_split_workspace_size.restype = ctypes.c_size_t
        lib.la_prefill_split_blocks.argtypes = [i64, i32, i32, i32, ctypes.c_int]
        lib.la_prefill_split_blocks.restype = i32
        lib.la_prefill_split_blocks_for.argtypes = [i64, i32, i32, i32, ctypes.c_int, i32]
        lib.la_prefill_split_blocks_for.restype = i32
        lib.la_backward.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, i64, i32,
                                    i32, i32, ctypes.c_int, vp]
        lib.la_backward.restype = ctypes.c_int
        lib.la_backward_split.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, i64,
                                          i32, i32, i32, ctypes.c_int, i32, vp, ctypes.c_size_t,
                                          vp]
        lib.la_backward_split.restype = ctypes.c_int
        lib.la_decode_step.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, i32, ctypes.c_int, vp]
        lib.la_decode_step.restype = ctypes.c_int
        lib.la_decode_tokens.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, ctypes.c_int,
                                         vp]
        lib.la_decode_tokens.restype = ctypes.c_int
        lib.la_status_str.argtypes = [ctypes.c_int]
        lib.la_status_str.restype = ctypes.c_char_p
        lib.la_last_error.argtypes = []
        lib.la_last_error.restype = ctypes.c_char_p
        _lib = lib
        return lib


def _raise(rc: int):
    if rc != LA_OK:
        detail = load().la_last_error().decode(errors="replace")
        raise LightningAttnError(rc, detail)


def _p(x: int):
    return ctypes.c_void_p(x) if x else None


def prefill(q, k, v, decay, cu_seqlens, out, final_state, T, S, H, D, dtype, stream):
    _raise(load().la_prefill(_p(q), _p(k), _p(v), _p(decay), _p(cu_seqlens), _p(out),
                             _p(final_state), T, S, H, D, dtype, _p(stream)))


def prefill_ex(q, k, v, decay, cu_seqlens, initial_state, out, final_state, T, S, H, D, dtype,
               stream):
    _raise(load().la_prefill_ex(_p(q), _p(k), _p(v), _p(decay), _p(cu_seqlens), _p(initial_state),
                                _p(out), _p(final_state), T, S, H, D, dtype, _p(stream)))


def prefill_with_block_size(q, k, v, decay, cu_seqlens, initial_state, out, final_state, T, S,
                            H, D, dtype, block_size, stream):
    _raise(load().la_prefill_with_block_size(_p(q), _p(k), _p(v), _p(decay), _p(cu_seqlens),
                                             _p(initial_state), _p(out), _p(final_state), T, S,
                                             H, D, dtype, block_size, _p(stream)))


def prefill_split(q, k, v, decay, cu_seqlens, initial_state, out, final_state, T, S, H, D, dtype,
                  seg_blocks, workspace, workspace_bytes, stream):
    _raise(load().la_prefill_split(_p(q), _p(k), _p(v), _p(decay), _p(cu_seqlens),
                                   _p(initial_state), _p(out), _p(final_state), T, S, H, D, dtype,
                                   seg_blocks, _p(workspace), workspace_bytes, _p(stream)))


def prefill_split_static(q, k, v, decay, cu_seqlens, initial_state, out, final_state, T, S, H, D,
                         dtype, seg_blocks, stream):
    _raise(load().la_prefill_split_static(_p(q), _p(k), _p(v), _p(decay), _p(cu_seqlens),
                                          _p(initial_state), _p(out), _p(final_state), T, S, H,
                                          D, dtype, seg_blocks, _p(stream)))


# LA_SPLIT_STATIC_SCRATCH_BYTES of include/lightning_attn.h (the static scratch of
# la_prefill_split_static, per device)
SPLIT_STATIC_SCRATCH_BYTES = 32 << 20


def prefill_split_workspace_size(T, S, H, D, seg_blocks) -> int:
    return int(load().la_prefill_split_workspace_size(T, S, H, D, seg_blocks))


def prefill_split_blocks(T, S, H, D, dtype) -> int:
    return int(load().la_prefill_split_blocks(T, S, H, D, dtype))


def prefill_split_blocks_for(T, S, H, D, dtype, compute_units) -> int:
    return int(load().la_prefill_split_blocks_for(T, S, H, D, dtype, compute_units))


def backward(q, k, v, decay, cu_seqlens, initial_state, d_out, d_final_state, dq, dk, dv,
             d_initial_state, T, S, H, D, dtype, stream):
    _raise(load().la_backward(_p(q), _p(k), _p(v), _p(decay), _p(cu_seqlens), _p(initial_state),
                              _p(d_out), _p(d_final_state), _p(dq), _p(dk), _p(dv),
                              _p(d_initial_state), T, S, H, D, dtype, _p(stream)))


def backward_split(q, k, v, decay, cu_seqlens, initial_state, d_out, d_final_state, dq, dk, dv,
                   d_initial_state, T, S, H, D, dtype, seg_blocks, workspace, workspace_bytes,
                   stream):
    _raise(load().la_backward_split(_p(q), _p(k), _p(v), _p(decay), _p(cu_seqlens),
                                    _p(initial_state), _p(d_out), _p(d_final_state), _p(dq),
                                    _p(dk), _p(dv), _p(d_initial_state), T, S, H, D, dtype,
                                    seg_blocks, _p(workspace), workspace_bytes, _p(stream)))


def decode_step(q, k, v, decay, state, out, Bt, H, D, dtype, stream):
    _raise(load().la_decode_step(_p(q), _p(k), _p(v), _p(decay), _p(state), _p(out), Bt, H, D,
                                 dtype, _p(stream)))


def decode_tokens(q, k, v, decay, state, out, Bt, m, H, D, dtype, stream):
    _raise(load().la_decode_tokens(_p(q), _p(k), _p(v), _p(decay), _p(state), _p(out), Bt, m, H,
                                   D, dtype, _p(stream)))


def raw_status(fn: str, *args) -> int:
    """Call an entry point with raw arguments and return its status (for ABI tests)."""
    return int(getattr(load(), fn)(*args))
