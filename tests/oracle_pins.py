"""Pins that tie the fp64 oracle to facts other than its own formula.

Each ``pin_*`` function takes an ``oracle.Oracle`` and raises AssertionError when the oracle
disagrees with a closed form, a hand-worked example, a textbook routine, an invariant or a
second, different algorithm.  They are run against the real oracle (test_oracle_pins.py) and
against copies of the oracle with planted mistakes (test_oracle_mutants.py), which must each
fail at least one pin.

The facts pinned: the definition of causal linear attention with a constant per-head decay
(o_t = sum_{s<=t} lambda^(t-s) (q_t . k_s) v_s), the associativity (QK^T)V = Q(K^T V) that
linear attention rests on (nabfollower blog, "The Core Tech: Lightning Attention"), and the
fixed-state scan view S_t = lambda S_{t-1} + k_t^T v_t, o_t = q_t S_t (same blog, analogy
section); the block split into an intra-block left product and an inter-block right product
(futurefh.com technical-report digest, section 1) is pinned by ``block_form`` below.
"""
from __future__ import annotations

import numpy as np

TOL = 1e-12


def rel_err(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    nb = np.linalg.norm(b)
    if nb == 0.0:
        return float(np.linalg.norm(a - b))
    return float(np.linalg.norm(a - b) / nb)


def close(a, b, tol=TOL, what=""):
    e = rel_err(a, b)
    assert e <= tol, "%s: relative error %.3e > %.1e" % (what, e, tol)


def rnd(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


# --------------------------------------------------------------------------------------------
# Test-only block form of the method (numpy, fp64).  Written from the block equations the
# GPU kernels use, not from the oracle: for block i of length b with rows j = 0..b-1,
#   O_i  = ((Q_i K_i^T) * M) V_i + diag(lambda^(j+1)) Q_i KV_{i-1},  M[j, j'] = lambda^(j-j') [j' <= j]
#   KV_i = lambda^b KV_{i-1} + K_i^T diag(lambda^(b-1-j)) V_i,      KV_{-1} = S0 (or 0).
# --------------------------------------------------------------------------------------------
def block_form(q, k, v, lam, B, S0=None):
    n, D = q.shape
    KV = np.zeros((D, D)) if S0 is None else np.array(S0, np.float64)
    out = np.zeros((n, D))
    for i0 in range(0, n, B):
        b = min(B, n - i0)
        Qi, Ki, Vi = q[i0:i0 + b], k[i0:i0 + b], v[i0:i0 + b]
        j = np.arange(b)
        diff = j[:, None] - j[None, :]
        M = np.where(diff >= 0, np.power(lam, np.maximum(diff, 0).astype(np.float64)), 0.0)
        intra = ((Qi @ Ki.T) * M) @ Vi
        inter = np.power(lam, (j + 1).astype(np.float64))[:, None] * (Qi @ KV)
        out[i0:i0 + b] = intra + inter
        KV = lam ** b * KV + Ki.T @ (np.power(lam, (b - 1 - j).astype(np.float64))[:, None] * Vi)
    return out, KV


# --------------------------------------------------------------------------------------------
# Pins
# --------------------------------------------------------------------------------------------
def pin_worked_example(o):
    """Hand-worked example: n=3, D=2, lambda=1/2, small integers (exact in binary).

    q = [[1,0],[0,1],[1,1]], k = [[1,0],[1,1],[0,1]], v = [[1,2],[3,0],[0,1]].
      o_0 = (q0.k0) v0                                   = 1*(1,2)               = (1, 2)
      o_1 = (q1.k1) v1 + 1/2 (q1.k0) v0                  = (3,0) + 0             = (3, 0)
      o_2 = (q2.k2) v2 + 1/2 (q2.k1) v1 + 1/4 (q2.k0) v0 = (0,1)+(3,0)+(1/4,1/2) = (13/4, 3/2)
      state = k2^T v2 + 1/2 k1^T v1 + 1/4 k0^T v0
            = [[0,0],[0,1]] + [[3/2,0],[3/2,0]] + [[1/4,1/2],[0,0]] = [[7/4,1/2],[3/2,1]]
    """
    q = np.array([[1, 0], [0, 1], [1, 1]], np.float64)[:, None, :]
    k = np.array([[1, 0], [1, 1], [0, 1]], np.float64)[:, None, :]
    v = np.array([[1, 2], [3, 0], [0, 1]], np.float64)[:, None, :]
    lam = np.array([0.5])
    want_o = np.array([[1, 2], [3, 0], [3.25, 1.5]])[:, None, :]
    want_s = np.array([[1.75, 0.5], [1.5, 1.0]])[None, None]
    assert np.array_equal(o.quadratic(q, k, v, lam), want_o), "quadratic worked example"
    ro, rs = o.recurrent(q, k, v, lam)
    assert np.array_equal(ro, want_o), "recurrent worked example (out)"
    assert np.array_equal(rs, want_s), "recurrent worked example (state)"
    assert np.array_equal(o.final_state(k, v, lam), want_s), "final_state worked example"
    assert np.array_equal(o.quadratic_rows(q, k, v, lam, [2, 0]), want_o[[2, 0]]), "rows example"


def pin_decode_worked_example(o):
    """Hand-worked decode step: lambda=1/2, S=[[1,2],[3,4]], k=(1,0), v=(0,2), q=(1,1).
      S' = S/2 + k^T v = [[1/2,1],[3/2,2]] + [[0,2],[0,0]] = [[1/2,3],[3/2,2]]
      o  = q S'        = (1/2 + 3/2, 3 + 2)              = (2, 5)
    """
    S = np.array([[1, 2], [3, 4]], np.float64)[None, None]
    q = np.array([[[1, 1]]], np.float64)
    k = np.array([[[1, 0]]], np.float64)
    v = np.array([[[0, 2]]], np.float64)
    out, S1 = o.decode_step(q, k, v, np.array([0.5]), S)
    assert np.array_equal(out, np.array([[[2.0, 5.0]]])), "decode worked example (out)"
    assert np.array_equal(S1, np.array([[[[0.5, 3], [1.5, 2]]]])), "decode worked example (state)"


def pin_unmasked_worked_example(o):
    """(QK^T)V = Q(K^T V) on a 2x2 hand example: Q=[[1,2],[0,1]], K=[[1,0],[1,1]], V=[[2,0],[1,3]].
      QK^T = [[1,3],[0,1]];  (QK^T)V = [[5,9],[1,3]]
      K^T V = [[3,3],[1,3]];  Q(K^T V) = [[5,9],[1,3]]
    """
    q = np.array([[1, 2], [0, 1]], np.float64)
    k = np.array([[1, 0], [1, 1]], np.float64)
    v = np.array([[2, 0], [1, 3]], np.float64)
    want = np.array([[5, 9], [1, 3]], np.float64)
    assert np.array_equal(o.unmasked_left(q, k, v), want), "unmasked left worked example"
    assert np.array_equal(o.unmasked_right(q, k, v), want), "unmasked right worked example"


def pin_ones_closed_form(o):
    """q = k = v = 1: o_t = D (1 - lambda^(t+1)) / (1 - lambda) (D (t+1) at lambda = 1),
    state = (1 - lambda^n) / (1 - lambda) (n at lambda = 1) in every entry."""
    n, D = 37, 8
    lams = np.array([0.0, 0.5, 0.9, 1.0])
    H = len(lams)
    one = np.ones((n, H, D))
    t = np.arange(n, dtype=np.float64)
    want = np.zeros((n, H, D))
    want_s = np.zeros((1, H, D, D))
    for h, lam in enumerate(lams):
        if lam == 1.0:
            want[:, h, :] = (D * (t + 1))[:, None]
            want_s[0, h] = n
        else:
            want[:, h, :] = (D * (1 - lam ** (t + 1)) / (1 - lam))[:, None]
            want_s[0, h] = (1 - lam ** n) / (1 - lam)
    close(o.quadratic(one, one, one, lams), want, 1e-13, "ones quadratic")
    ro, rs = o.recurrent(one, one, one, lams)
    close(ro, want, 1e-13, "ones recurrent")
    close(rs, want_s, 1e-13, "ones recurrent state")
    close(o.final_state(one, one, lams), want_s, 1e-13, "ones final_state")


def pin_lambda_one_is_cumsum(o):
    """lambda = 1 (no decay): o_t = q_t (sum_{s<=t} k_s^T v_s), with the prefix sum taken by
    numpy.cumsum."""
    n, H, D = 50, 2, 6
    q, k, v = rnd((n, H, D), 1), rnd((n, H, D), 2), rnd((n, H, D), 3)
    lams = np.ones(H)
    outer = np.einsum("tha,thb->thab", k, v)
    pref = np.cumsum(outer, axis=0)
    want = np.einsum("tha,thab->thb", q, pref)
    close(o.quadratic(q, k, v, lams), want, TOL, "lambda=1 quadratic")
    ro, rs = o.recurrent(q, k, v, lams)
    close(ro, want, TOL, "lambda=1 recurrent")
    close(rs[0], pref[-1], TOL, "lambda=1 state")
    close(o.final_state(k, v, lams)[0], pref[-1], TOL, "lambda=1 final_state")


def pin_lambda_zero_is_diagonal(o):
    """lambda = 0: only s = t survives (0^0 = 1): o_t = (q_t . k_t) v_t, state = k_{n-1}^T v_{n-1}."""
    n, H, D = 20, 3, 5
    q, k, v = rnd((n, H, D), 4), rnd((n, H, D), 5), rnd((n, H, D), 6)
    lams = np.zeros(H)
    want = np.einsum("thd,thd->th", q, k)[:, :, None] * v
    want_s = np.einsum("ha,hb->hab", k[-1], v[-1])[None]
    close(o.quadratic(q, k, v, lams), want, TOL, "lambda=0 quadratic")
    ro, rs = o.recurrent(q, k, v, lams)
    close(ro, want, TOL, "lambda=0 recurrent")
    close(rs, want_s, TOL, "lambda=0 state")
    close(o.final_state(k, v, lams), want_s, TOL, "lambda=0 final_state")


def pin_impulse_response(o):
    """One key/value pair at s0 with k = e_a, v = e_b: o_t = lambda^(t-s0) q_t[a] e_b for
    t >= s0 and 0 before; state[a][b] = lambda^(n-1-s0), all other entries 0.  Fixes the
    direction and offset of the exponent and which index belongs to k and which to v."""
    n, D, s0, a, b = 12, 4, 3, 1, 2
    lam = 0.75
    q = rnd((n, 1, D), 7)
    k = np.zeros((n, 1, D))
    v = np.zeros((n, 1, D))
    k[s0, 0, a] = 1.0
    v[s0, 0, b] = 1.0
    want = np.zeros((n, 1, D))
    for t in range(s0, n):
        want[t, 0, b] = lam ** (t - s0) * q[t, 0, a]
    want_s = np.zeros((1, 1, D, D))
    want_s[0, 0, a, b] = lam ** (n - 1 - s0)
    lams = np.array([lam])
    close(o.quadratic(q, k, v, lams), want, TOL, "impulse quadratic")
    ro, rs = o.recurrent(q, k, v, lams)
    close(ro, want, TOL, "impulse recurrent")
    close(rs, want_s, TOL, "impulse state")
    close(o.final_state(k, v, lams), want_s, TOL, "impulse final_state")


def pin_unmasked_associativity(o):
    """(Q K^T) V = Q (K^T V), and both equal numpy's matmul of the same association."""
    n, D = 40, 7
    q, k, v = rnd((n, D), 8), rnd((n, D), 9), rnd((n, D), 10)
    left = o.unmasked_left(q, k, v)
    right = o.unmasked_right(q, k, v)
    close(left, right, TOL, "associativity")
    close(left, (q @ k.T) @ v, TOL, "left vs numpy")
    close(right, q @ (k.T @ v), TOL, "right vs numpy")


def pin_quadratic_equals_recurrent(o):
    """The quadratic form and the state recurrence are different algorithms for one result."""
    lengths = [1, 17, 64, 65, 0, 30]
    T, H, D = sum(lengths), 3, 8
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    q, k, v = rnd((T, H, D), 11), rnd((T, H, D), 12), rnd((T, H, D), 13)
    lams = np.array([0.3, 0.9, 0.999])
    a = o.quadratic(q, k, v, lams, cu)
    b, st = o.recurrent(q, k, v, lams, cu)
    close(a, b, TOL, "quadratic vs recurrent")
    close(o.final_state(k, v, lams, cu), st, TOL, "final_state vs recurrent")
    rows = [0, 1, 17, 18, 81, 82, 146, T - 1]
    close(o.quadratic_rows(q, k, v, lams, rows, cu), a[rows], TOL, "rows vs full")


def pin_varlen_is_concatenation(o):
    """Packing sequences does not change any result; an empty sequence has a zero state."""
    lengths = [5, 0, 9, 1]
    T, H, D = sum(lengths), 2, 4
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    q, k, v = rnd((T, H, D), 14), rnd((T, H, D), 15), rnd((T, H, D), 16)
    lams = np.array([0.6, 0.95])
    packed = o.quadratic(q, k, v, lams, cu)
    _, st = o.recurrent(q, k, v, lams, cu)
    for s, n in enumerate(lengths):
        sl = slice(cu[s], cu[s + 1])
        if n == 0:
            assert np.all(st[s] == 0.0), "empty sequence state"
            continue
        close(packed[sl], o.quadratic(q[sl], k[sl], v[sl], lams), TOL, "varlen out")
        close(st[s], o.final_state(k[sl], v[sl], lams)[0], TOL, "varlen state")


def pin_causality(o):
    """Changing later tokens (even to NaN/inf) leaves earlier outputs bit-identical."""
    n, H, D, t0 = 30, 2, 4, 17
    q, k, v = rnd((n, H, D), 17), rnd((n, H, D), 18), rnd((n, H, D), 19)
    lams = np.array([0.8, 1.0])
    base = o.quadratic(q, k, v, lams)
    k2, v2 = k.copy(), v.copy()
    k2[t0:] = np.nan
    v2[t0:] = np.inf
    pert = o.quadratic(q, k2, v2, lams)
    assert np.array_equal(base[:t0], pert[:t0]), "future leaked into the past (quadratic)"
    r1, _ = o.recurrent(q, k2, v2, lams)
    assert np.array_equal(o.recurrent(q, k, v, lams)[0][:t0], r1[:t0]), "future leaked (recurrent)"


def pin_linearity_in_v(o):
    """o is linear in v: o(a v1 + b v2) = a o(v1) + b o(v2)."""
    n, H, D = 25, 2, 5
    q, k = rnd((n, H, D), 20), rnd((n, H, D), 21)
    v1, v2 = rnd((n, H, D), 22), rnd((n, H, D), 23)
    lams = np.array([0.7, 0.97])
    lhs = o.quadratic(q, k, 2.0 * v1 - 3.0 * v2, lams)
    rhs = 2.0 * o.quadratic(q, k, v1, lams) - 3.0 * o.quadratic(q, k, v2, lams)
    close(lhs, rhs, TOL, "linearity")


def pin_initial_state_is_chunking(o):
    """Prefill of [0, m) gives a state S; prefill of [m, n) from S equals rows m.. of the whole
    prefill, and its final state equals the whole sequence's."""
    n, m, H, D = 41, 16, 2, 6
    q, k, v = rnd((n, H, D), 24), rnd((n, H, D), 25), rnd((n, H, D), 26)
    lams = np.array([0.85, 0.99])
    whole = o.quadratic(q, k, v, lams)
    _, S_whole = o.recurrent(q, k, v, lams)
    S_m = o.final_state(k[:m], v[:m], lams)
    tail_q = o.quadratic(q[m:], k[m:], v[m:], lams, init_state=S_m)
    tail_r, S_tail = o.recurrent(q[m:], k[m:], v[m:], lams, init_state=S_m)
    close(tail_q, whole[m:], TOL, "chunked quadratic")
    close(tail_r, whole[m:], TOL, "chunked recurrent")
    close(S_tail, S_whole, TOL, "chunked state")
    close(o.final_state(k[m:], v[m:], lams, init_state=S_m), S_whole, TOL, "chunked final_state")
    rows = [m, m + 1, n - 1]
    close(o.quadratic_rows(q[m:], k[m:], v[m:], lams, [r - m for r in rows], init_state=S_m),
          whole[rows], TOL, "chunked rows")


def pin_decode_extends_prefill(o):
    """Prefill of n tokens then one decode step on token n equals prefill of n+1 tokens."""
    n, H, D = 23, 3, 5
    q, k, v = rnd((n + 1, H, D), 27), rnd((n + 1, H, D), 28), rnd((n + 1, H, D), 29)
    lams = np.array([0.5, 0.9, 1.0])
    _, S_n = o.recurrent(q[:n], k[:n], v[:n], lams)
    out, S1 = o.decode_step(q[n:], k[n:], v[n:], lams, S_n)
    full = o.quadratic(q, k, v, lams)
    close(out[0], full[n], TOL, "decode out")
    close(S1, o.final_state(k, v, lams), TOL, "decode state")


def pin_block_form(o):
    """The intra/inter block split equals the definition for any block size, including a
    ragged last block; with an initial state as well."""
    n, D = 70, 6
    q, k, v = rnd((n, 1, D), 30), rnd((n, 1, D), 31), rnd((n, 1, D), 32)
    S0 = rnd((1, 1, D, D), 33)
    for lam in (0.0, 0.6, 0.99, 1.0):
        want = o.quadratic(q, k, v, np.array([lam]), init_state=S0)[:, 0]
        want_s = o.final_state(k, v, np.array([lam]), init_state=S0)[0, 0]
        for B in (1, 3, 16, 64, n):
            got, KV = block_form(q[:, 0], k[:, 0], v[:, 0], lam, B, S0[0, 0])
            close(got, want, TOL, "block form out lam=%g B=%d" % (lam, B))
            close(KV, want_s, TOL, "block form state lam=%g B=%d" % (lam, B))


# --------------------------------------------------------------------------------------------
# Backward pins.  The gradients are those of L = <do, o> + <dSn, final_state>; L is linear in
# each of q, k, v and S0 separately, so a central difference of the (already pinned) forward
# oracle is exact up to rounding, for any step.
# --------------------------------------------------------------------------------------------
def _loss(o, q, k, v, lams, cu, S0, do, dSn):
    return float(np.sum(do * o.quadratic(q, k, v, lams, cu, init_state=S0)) +
                 np.sum(dSn * o.final_state(k, v, lams, cu, init_state=S0)))


def _bwd_case(seed):
    """Packed lengths 3, 0, 4 (an empty sequence), H=3 heads with lambda 0, 0.6, 1, D=3."""
    lengths = [3, 0, 4]
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    T, H, D, S = int(cu[-1]), 3, 3, len(lengths)
    lams = np.array([0.0, 0.6, 1.0])
    q, k, v, do = (rnd((T, H, D), seed + i) for i in range(4))
    S0, dSn = rnd((S, H, D, D), seed + 4), rnd((S, H, D, D), seed + 5)
    return q, k, v, lams, cu, S0, do, dSn


def pin_backward_finite_difference(o):
    """Every entry of dq, dk, dv, dS0 (both O6 and O7) equals the central difference of the
    forward oracle's loss."""
    q, k, v, lams, cu, S0, do, dSn = _bwd_case(40)
    args = dict(q=q, k=k, v=v, S0=S0)
    eps = 0.25
    num = {}
    for name, x in args.items():
        g = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            a = {n: (y.copy() if n == name else y) for n, y in args.items()}
            a[name][idx] += eps
            lp = _loss(o, a["q"], a["k"], a["v"], lams, cu, a["S0"], do, dSn)
            a[name][idx] -= 2 * eps
            lm = _loss(o, a["q"], a["k"], a["v"], lams, cu, a["S0"], do, dSn)
            g[idx] = (lp - lm) / (2 * eps)
        num[name] = g
    for fn in (o.backward, o.backward_recurrent):
        dq, dk, dv, dS0 = fn(q, k, v, lams, do, cu, init_state=S0, d_final=dSn)
        close(dq, num["q"], 1e-12, "%s dq vs finite difference" % fn.__name__)
        close(dk, num["k"], 1e-12, "%s dk vs finite difference" % fn.__name__)
        close(dv, num["v"], 1e-12, "%s dv vs finite difference" % fn.__name__)
        close(dS0, num["S0"], 1e-12, "%s dS0 vs finite difference" % fn.__name__)


def pin_backward_autograd(o):
    """torch autograd (fp64, CPU) through the explicit mask-matrix form
    o = ((Q K^T) * Dm) V + diag(lambda^(t+1)) Q S0, final = K^T diag(lambda^(n-1-s)) V + lambda^n S0."""
    import torch

    n, D = 20, 5
    lams = [0.0, 0.5, 0.95, 1.0]
    H = len(lams)
    q, k, v, do = (rnd((n, H, D), 50 + i) for i in range(4))
    S0, dSn = rnd((1, H, D, D), 54), rnd((1, H, D, D), 55)
    want = [np.zeros((n, H, D)) for _ in range(3)] + [np.zeros((1, H, D, D))]
    t = torch.arange(n, dtype=torch.float64)
    for h, lam in enumerate(lams):
        Q, K, V, S = (torch.tensor(x[:, h] if x.ndim == 3 else x[0, h], requires_grad=True)
                      for x in (q, k, v, S0))
        diff = t[:, None] - t[None, :]
        Dm = torch.where(diff >= 0, torch.tensor(lam, dtype=torch.float64) ** diff.clamp(min=0),
                         torch.zeros((), dtype=torch.float64))
        out = ((Q @ K.T) * Dm) @ V + (lam ** (t + 1))[:, None] * (Q @ S)
        fin = K.T @ ((lam ** (n - 1 - t))[:, None] * V) + lam ** n * S
        L = (out * torch.tensor(do[:, h])).sum() + (fin * torch.tensor(dSn[0, h])).sum()
        gq, gk, gv, gs = torch.autograd.grad(L, (Q, K, V, S))
        want[0][:, h], want[1][:, h], want[2][:, h], want[3][0, h] = (
            gq.numpy(), gk.numpy(), gv.numpy(), gs.numpy())
    for fn in (o.backward, o.backward_recurrent):
        got = fn(q, k, v, np.array(lams), do, init_state=S0, d_final=dSn)
        for name, g, w in zip(("dq", "dk", "dv", "dS0"), got, want):
            close(g, w, 1e-12, "%s %s vs autograd" % (fn.__name__, name))


def pin_backward_lambda_zero(o):
    """lambda = 0: o_t = (q_t . k_t) v_t and final = k_{n-1}^T v_{n-1}, so dq_t = (do_t . v_t) k_t,
    dk_t = (do_t . v_t) q_t (+ dSn v_t at the last token), dv_t = (q_t . k_t) do_t (+ dSn^T k_t
    at the last token), dS0 = 0 (n >= 1)."""
    n, D = 6, 4
    q, k, v, do = (rnd((n, 1, D), 60 + i) for i in range(4))
    dSn = rnd((1, 1, D, D), 64)
    S0 = rnd((1, 1, D, D), 65)
    c = np.sum(do * v, axis=2, keepdims=True)
    qk = np.sum(q * k, axis=2, keepdims=True)
    wq, wk, wv = c * k, c * q, qk * do
    wk[-1, 0] += dSn[0, 0] @ v[-1, 0]
    wv[-1, 0] += dSn[0, 0].T @ k[-1, 0]
    for fn in (o.backward, o.backward_recurrent):
        dq, dk, dv, dS0 = fn(q, k, v, np.array([0.0]), do, init_state=S0, d_final=dSn)
        close(dq, wq, 1e-14, "lambda=0 dq")
        close(dk, wk, 1e-14, "lambda=0 dk")
        close(dv, wv, 1e-14, "lambda=0 dv")
        assert np.all(dS0 == 0.0), "lambda=0 dS0"


def pin_backward_ones_closed_form(o):
    """q = k = v = do = 1, no initial or final-state terms: dq_t = D (1 - lambda^(t+1)) / (1 - lambda),
    dk_s = dv_s = D (1 - lambda^(n-s)) / (1 - lambda) (D (t+1), D (n-s) at lambda = 1), and
    dS0 = sum_t lambda^(t+1) = lambda (1 - lambda^n) / (1 - lambda) (n at lambda = 1)."""
    n, D = 29, 4
    lams = np.array([0.0, 0.5, 0.9, 1.0])
    H = len(lams)
    one = np.ones((n, H, D))
    t = np.arange(n, dtype=np.float64)
    wq, wkv = np.zeros((n, H, D)), np.zeros((n, H, D))
    wS = np.zeros((1, H, D, D))
    for h, lam in enumerate(lams):
        if lam == 1.0:
            wq[:, h], wkv[:, h], wS[0, h] = (D * (t + 1))[:, None], (D * (n - t))[:, None], n
        else:
            wq[:, h] = (D * (1 - lam ** (t + 1)) / (1 - lam))[:, None]
            wkv[:, h] = (D * (1 - lam ** (n - t)) / (1 - lam))[:, None]
            wS[0, h] = lam * (1 - lam ** n) / (1 - lam)
    for fn in (o.backward, o.backward_recurrent):
        dq, dk, dv, dS0 = fn(one, one, one, lams, one)
        close(dq, wq, 1e-13, "ones dq")
        close(dk, wkv, 1e-13, "ones dk")
        close(dv, wkv, 1e-13, "ones dv")
        close(dS0, wS, 1e-13, "ones dS0")


def pin_backward_homogeneity(o):
    """o is linear in q, so <q, dq> = <do, o>; every term of L that holds k also holds v, so
    <k, dk> = <v, dv>; L is affine in S0, so <S0, dS0> = L(S0) - L(0)."""
    q, k, v, lams, cu, S0, do, dSn = _bwd_case(70)
    dq, dk, dv, dS0 = o.backward(q, k, v, lams, do, cu, init_state=S0, d_final=dSn)
    out = o.quadratic(q, k, v, lams, cu, init_state=S0)
    close(np.sum(q * dq), np.sum(do * out), 1e-12, "<q,dq> = <do,o>")
    close(np.sum(k * dk), np.sum(v * dv), 1e-12, "<k,dk> = <v,dv>")
    l1 = _loss(o, q, k, v, lams, cu, S0, do, dSn)
    l0 = _loss(o, q, k, v, lams, cu, np.zeros_like(S0), do, dSn)
    close(np.sum(S0 * dS0), l1 - l0, 1e-12, "<S0,dS0> = L(S0) - L(0)")


def pin_backward_varlen_is_concatenation(o):
    """Packed gradients equal per-sequence gradients; an empty sequence gives dS0 = dSn."""
    q, k, v, lams, cu, S0, do, dSn = _bwd_case(80)
    for fn in (o.backward, o.backward_recurrent):
        dq, dk, dv, dS0 = fn(q, k, v, lams, do, cu, init_state=S0, d_final=dSn)
        for s in range(len(cu) - 1):
            a, b = int(cu[s]), int(cu[s + 1])
            if a == b:
                close(dS0[s], dSn[s], 0.0, "empty sequence dS0")
                continue
            g = fn(q[a:b], k[a:b], v[a:b], lams, do[a:b], init_state=S0[s:s + 1],
                   d_final=dSn[s:s + 1])
            for name, x, y in zip(("dq", "dk", "dv"), (dq, dk, dv), g):
                close(x[a:b], y, 1e-14, "varlen %s seq %d" % (name, s))
            close(dS0[s], g[3][0], 1e-14, "varlen dS0 seq %d" % s)


ALL_PINS = [
    pin_worked_example,
    pin_decode_worked_example,
    pin_unmasked_worked_example,
    pin_ones_closed_form,
    pin_lambda_one_is_cumsum,
    pin_lambda_zero_is_diagonal,
    pin_impulse_response,
    pin_unmasked_associativity,
    pin_quadratic_equals_recurrent,
    pin_varlen_is_concatenation,
    pin_causality,
    pin_linearity_in_v,
    pin_initial_state_is_chunking,
    pin_decode_extends_prefill,
    pin_block_form,
    pin_backward_finite_difference,
    pin_backward_autograd,
    pin_backward_lambda_zero,
    pin_backward_ones_closed_form,
    pin_backward_homogeneity,
    pin_backward_varlen_is_concatenation,
]
