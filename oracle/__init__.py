"""fp64 CPU oracle for decayed causal linear attention ("lightning attention").

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the benchmark's
CPU-baseline leg may import this package; the product path (the HIP library and its binding)
never does, and the two share no code.  The arithmetic lives in plain C (``la_oracle.c``,
double precision, plain loops); this module only builds it with gcc, loads it with ctypes and
marshals numpy arrays.

Functions (all inputs are converted to contiguous float64; layouts [T, H, D] and
[S, H, D, D]; ``cu_seqlens`` int32 [S+1] or None for one sequence):

* ``quadratic``       -- O1, the quadratic masked form over every row (the authority).
* ``quadratic_rows``  -- O1 on selected global token rows.
* ``recurrent``       -- O2, the state recurrence S_t = lambda S_{t-1} + k_t^T v_t, o_t = q_t S_t.
* ``final_state``     -- O3, closed form sum_s lambda^(n-1-s) k_s^T v_s (+ lambda^n S0).
* ``decode_step``     -- O4, one recurrent step for a batch of states.
* ``unmasked_left`` / ``unmasked_right`` -- O5, (Q K^T) V and Q (K^T V) for one head.
* ``backward``        -- O6, gradients dq, dk, dv, dS0 of the prefill, term by term from the
  derivative of the definition (quadratic in n).
* ``backward_recurrent`` -- O7, the same gradients through a forward and a reverse state scan.

The definitions follow the pages' statement of causal linear attention and its association
orders (MiniMax-01 technical-report digest on futurefh.com, section 1; nabfollower blog,
section "The Core Tech: Lightning Attention") and of the fixed-state scan (nabfollower blog,
analogy section), with the constant per-head decay lambda^(t-s) as the reading adopted where
the pages are silent.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "la_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liblaoracle.so")
_lock = threading.Lock()

_DP = ctypes.POINTER(ctypes.c_double)
_IP = ctypes.POINTER(ctypes.c_int32)
_LP = ctypes.POINTER(ctypes.c_int64)


def build(force: bool = True, src: str = _SRC, out: str = _LIB_PATH) -> str:
    """Compile la_oracle.c into a shared library with gcc (OpenMP, -O2, no fast-math)."""
    if not force and os.path.exists(out):
        return out
    tmp = out + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-Wall", "-Wextra",
           "-o", tmp, src]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


def _bind(lib):
    i32, i64 = ctypes.c_int32, ctypes.c_int64
    lib.lao_quadratic.argtypes = [_DP, _DP, _DP, _DP, _IP, i32, i64, i32, i32, _DP, _DP]
    lib.lao_quadratic_rows.argtypes = [_DP, _DP, _DP, _DP, _IP, i32, i64, i32, i32, _DP,
                                       _LP, i64, _DP]
    lib.lao_recurrent.argtypes = [_DP, _DP, _DP, _DP, _IP, i32, i64, i32, i32, _DP, _DP, _DP]
    lib.lao_final_state.argtypes = [_DP, _DP, _DP, _IP, i32, i64, i32, i32, _DP, _DP]
    lib.lao_decode_step.argtypes = [_DP, _DP, _DP, _DP, i32, i32, i32, _DP, _DP]
    lib.lao_unmasked_left.argtypes = [_DP, _DP, _DP, i64, i32, _DP]
    lib.lao_unmasked_right.argtypes = [_DP, _DP, _DP, i64, i32, _DP]
    for name in ("lao_backward", "lao_backward_recurrent"):
        getattr(lib, name).argtypes = [_DP, _DP, _DP, _DP, _IP, i32, i64, i32, i32, _DP, _DP, _DP,
                                       _DP, _DP, _DP, _DP]
    lib.lao_num_threads.argtypes = []
    lib.lao_set_num_threads.argtypes = [ctypes.c_int]
    lib.lao_set_num_threads.restype = None
    for name in ("lao_quadratic", "lao_quadratic_rows", "lao_recurrent", "lao_final_state",
                 "lao_decode_step", "lao_unmasked_left", "lao_unmasked_right",
                 "lao_backward", "lao_backward_recurrent", "lao_num_threads"):
        getattr(lib, name).restype = ctypes.c_int
    return lib


def _f64(x):
    if x is None:
        return None
    if hasattr(x, "detach"):  # torch tensor -> numpy (exact upcast from bf16/fp32)
        import torch  # local: only reached with torch inputs

        x = x.detach().to("cpu").to(torch.float64).numpy()
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _i32(x):
    if x is None:
        return None
    if hasattr(x, "detach"):
        x = x.detach().to("cpu").numpy()
    return np.ascontiguousarray(np.asarray(x, dtype=np.int32))


def _ptr(a, typ=_DP):
    return None if a is None else a.ctypes.data_as(typ)


def _shape(x, cu):
    T, H, D = x.shape
    S = 1 if cu is None else len(cu) - 1
    return S, T, H, D


def _check(rc, what):
    if rc != 0:
        raise ValueError("oracle %s rejected its arguments" % what)


class Oracle:
    """The oracle's functions bound to one compiled copy of la_oracle.c."""

    def __init__(self, lib_path: str):
        self.path = lib_path
        self.lib = _bind(ctypes.CDLL(lib_path))

    def quadratic(self, q, k, v, decay, cu_seqlens=None, init_state=None):
        """O1: o_t = sum_{s<=t} lambda^(t-s)(q_t.k_s) v_s [+ lambda^(t+1) q_t S0] -> [T,H,D]."""
        q, k, v, decay, init_state = map(_f64, (q, k, v, decay, init_state))
        cu = _i32(cu_seqlens)
        S, T, H, D = _shape(q, cu)
        out = np.zeros((T, H, D), np.float64)
        rc = self.lib.lao_quadratic(_ptr(q), _ptr(k), _ptr(v), _ptr(decay), _ptr(cu, _IP), S, T,
                                    H, D, _ptr(init_state), _ptr(out))
        _check(rc, "quadratic")
        return out

    def quadratic_rows(self, q, k, v, decay, rows, cu_seqlens=None, init_state=None):
        """O1 on the global token rows ``rows`` -> [len(rows), H, D]."""
        q, k, v, decay, init_state = map(_f64, (q, k, v, decay, init_state))
        cu = _i32(cu_seqlens)
        rows = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
        S, T, H, D = _shape(q, cu)
        out = np.zeros((len(rows), H, D), np.float64)
        rc = self.lib.lao_quadratic_rows(_ptr(q), _ptr(k), _ptr(v), _ptr(decay), _ptr(cu, _IP),
                                         S, T, H, D, _ptr(init_state), _ptr(rows, _LP),
                                         len(rows), _ptr(out))
        _check(rc, "quadratic_rows")
        return out

    def recurrent(self, q, k, v, decay, cu_seqlens=None, init_state=None, want_out=True,
                  want_state=True):
        """O2 -> (out [T,H,D] or None, final_state [S,H,D,D] or None)."""
        q, k, v, decay, init_state = map(_f64, (q, k, v, decay, init_state))
        cu = _i32(cu_seqlens)
        S, T, H, D = _shape(k, cu)
        out = np.zeros((T, H, D), np.float64) if want_out else None
        st = np.zeros((S, H, D, D), np.float64) if want_state else None
        rc = self.lib.lao_recurrent(_ptr(q) if want_out else None, _ptr(k), _ptr(v), _ptr(decay),
                                    _ptr(cu, _IP), S, T, H, D, _ptr(init_state), _ptr(out),
                                    _ptr(st))
        _check(rc, "recurrent")
        return out, st

    def final_state(self, k, v, decay, cu_seqlens=None, init_state=None):
        """O3: closed-form final state per (sequence, head) -> [S,H,D,D]."""
        k, v, decay, init_state = map(_f64, (k, v, decay, init_state))
        cu = _i32(cu_seqlens)
        S, T, H, D = _shape(k, cu)
        st = np.zeros((S, H, D, D), np.float64)
        rc = self.lib.lao_final_state(_ptr(k), _ptr(v), _ptr(decay), _ptr(cu, _IP), S, T, H, D,
                                      _ptr(init_state), _ptr(st))
        _check(rc, "final_state")
        return st

    def decode_step(self, q, k, v, decay, state):
        """O4 -> (out [Bt,H,D], new_state [Bt,H,D,D]); the input state is not modified."""
        q, k, v, decay = map(_f64, (q, k, v, decay))
        st = _f64(state).copy()
        Bt, H, D = q.shape
        out = np.zeros((Bt, H, D), np.float64)
        rc = self.lib.lao_decode_step(_ptr(q), _ptr(k), _ptr(v), _ptr(decay), Bt, H, D,
                                      _ptr(st), _ptr(out))
        _check(rc, "decode_step")
        return out, st

    def unmasked_left(self, q, k, v):
        """O5 left association (Q K^T) V for one head; q, k, v are [n, D]."""
        q, k, v = map(_f64, (q, k, v))
        n, D = q.shape
        out = np.zeros((n, D), np.float64)
        _check(self.lib.lao_unmasked_left(_ptr(q), _ptr(k), _ptr(v), n, D, _ptr(out)),
               "unmasked_left")
        return out

    def unmasked_right(self, q, k, v):
        """O5 right association Q (K^T V) for one head; q, k, v are [n, D]."""
        q, k, v = map(_f64, (q, k, v))
        n, D = q.shape
        out = np.zeros((n, D), np.float64)
        _check(self.lib.lao_unmasked_right(_ptr(q), _ptr(k), _ptr(v), n, D, _ptr(out)),
               "unmasked_right")
        return out

    def _bwd(self, fn, q, k, v, decay, d_out, cu_seqlens, init_state, d_final, want_d_init):
        q, k, v, decay, d_out, init_state, d_final = map(
            _f64, (q, k, v, decay, d_out, init_state, d_final))
        cu = _i32(cu_seqlens)
        S, T, H, D = _shape(q, cu)
        dq, dk, dv = (np.zeros((T, H, D), np.float64) for _ in range(3))
        di = np.zeros((S, H, D, D), np.float64) if want_d_init else None
        rc = getattr(self.lib, fn)(_ptr(q), _ptr(k), _ptr(v), _ptr(decay), _ptr(cu, _IP), S, T,
                                   H, D, _ptr(init_state), _ptr(d_out), _ptr(d_final), _ptr(dq),
                                   _ptr(dk), _ptr(dv), _ptr(di))
        _check(rc, fn)
        return dq, dk, dv, di

    def backward(self, q, k, v, decay, d_out, cu_seqlens=None, init_state=None, d_final=None,
                 want_d_init=True):
        """O6 -> (dq, dk, dv [T,H,D], d_init [S,H,D,D] or None) for upstream gradients d_out
        [T,H,D] and d_final [S,H,D,D] (None = 0)."""
        return self._bwd("lao_backward", q, k, v, decay, d_out, cu_seqlens, init_state, d_final,
                         want_d_init)

    def backward_recurrent(self, q, k, v, decay, d_out, cu_seqlens=None, init_state=None,
                           d_final=None, want_d_init=True):
        """O7: the gradients of ``backward`` through a forward and a reverse state scan."""
        return self._bwd("lao_backward_recurrent", q, k, v, decay, d_out, cu_seqlens, init_state,
                         d_final, want_d_init)

    def num_threads(self) -> int:
        """OpenMP threads the oracle's parallel loops use."""
        return int(self.lib.lao_num_threads())

    def set_num_threads(self, n: int) -> None:
        """Threads for the oracle's later parallel loops."""
        self.lib.lao_set_num_threads(int(n))


_default = None


def default() -> Oracle:
    """The oracle built from la_oracle.c in this directory (built on first use if missing)."""
    global _default
    with _lock:
        if _default is None:
            if not os.path.exists(_LIB_PATH):
                build(force=True)
            _default = Oracle(_LIB_PATH)
        return _default


def quadratic(*a, **kw):
    return default().quadratic(*a, **kw)


def quadratic_rows(*a, **kw):
    return default().quadratic_rows(*a, **kw)


def recurrent(*a, **kw):
    return default().recurrent(*a, **kw)


def final_state(*a, **kw):
    return default().final_state(*a, **kw)


def decode_step(*a, **kw):
    return default().decode_step(*a, **kw)


def unmasked_left(*a, **kw):
    return default().unmasked_left(*a, **kw)


def unmasked_right(*a, **kw):
    return default().unmasked_right(*a, **kw)


def backward(*a, **kw):
    return default().backward(*a, **kw)


def backward_recurrent(*a, **kw):
    return default().backward_recurrent(*a, **kw)


def num_threads() -> int:
    return default().num_threads()
