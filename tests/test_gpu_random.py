"""Randomized GPU parity sweep (seeded, reproducible): random packed batches through the
prefill (plain or sequence-split), the backward (plain or split) and a decode step from the
prefilled states, each against the fp64 oracle (O1 quadratic form, O3 final states, O6
gradients, O4 decode).

Each case draws 1-5 sequences of 0-700 tokens (some empty), 1-5 heads (head counts that are not
multiples of 8 exercise the workgroup-mapping tail), d in {64, 128}, bf16 or fp32 storage,
lambda per head in [0.5, 1] with exact 0 and 1 mixed in, an initial state and a final-state
gradient or not, and a segment length of 1-3 blocks or no split.  Cases 48-63 draw 1-4
sequences of 0-3,000 tokens with segments of 5, 9 or 16 blocks (or no split), so that the
segment-state kernel's waves get several 32-token chunks, partial ones first.  Tolerances as
everywhere: relative L2 per (sequence, head) slice <= 2e-2 (bf16) / 1e-4 (fp32)."""
import numpy as np
import pytest
import torch

import long_context_attention_attn_amd as la
import oracle
from gpu_util import BF16_TOL, F32_TOL, banner, dev, slice_errors, state_errors, to_np
from long_context_attention_attn_amd import synth

pytestmark = pytest.mark.gpu

CASES = 64
LONG_FROM = 48  # cases from here on use long sequences and long segments
TOL = {torch.bfloat16: BF16_TOL, torch.float32: F32_TOL}


def _config(i):
    rng = np.random.default_rng(1000 + i)
    long = i >= LONG_FROM
    S = int(rng.integers(1, 5 if long else 6))
    lengths = [int(x) for x in rng.integers(0, 3001 if long else 701, S)]
    if rng.random() < 0.3:
        lengths[int(rng.integers(0, S))] = 0
    H = int(rng.integers(1, 6))
    D = int(rng.choice([64, 128]))
    dtype = torch.bfloat16 if rng.random() < 0.6 else torch.float32
    lam = rng.uniform(0.5, 1.0, H)
    if rng.random() < 0.4:
        lam[int(rng.integers(0, H))] = 0.0
    if rng.random() < 0.4:
        lam[int(rng.integers(0, H))] = 1.0
    if long:
        split = [None, 5, 9, 16][int(rng.integers(0, 4))]
    else:
        split = int(rng.integers(1, 4)) if rng.random() < 0.5 else None
    return dict(lengths=lengths, H=H, D=D, dtype=dtype, lam=lam, init=bool(rng.random() < 0.5),
                dfs=bool(rng.random() < 0.5), split=split)


def _worst(got, ref, cu):
    return float(slice_errors(to_np(got), ref, cu).max()) if int(cu[-1]) > 0 else 0.0


@pytest.mark.parametrize("i", range(CASES))
def test_random_case(i):
    cfg = _config(i)
    lengths, H, D, dtype = cfg["lengths"], cfg["H"], cfg["D"], cfg["dtype"]
    banner("random case %d: lengths=%s H=%d D=%d %s lam=%s init=%s dfs=%s split=%s"
           % (i, lengths, H, D, dtype, np.round(cfg["lam"], 3).tolist(), cfg["init"], cfg["dfs"],
              cfg["split"]))
    d = dev()
    tol = TOL[dtype]
    S = len(lengths)
    cu = synth.cu_from_lengths(lengths)
    T = int(cu[-1])
    q, k, v = synth.qkv(T, H, D, dtype, seed=2000 + i)
    do, _, _ = synth.qkv(T, H, D, dtype, seed=3000 + i)
    decay = torch.tensor(cfg["lam"], dtype=torch.float32)
    init = synth.random_state(S, H, D, seed=4000 + i, scale=0.1) if cfg["init"] else None
    dfs = synth.random_state(S, H, D, seed=5000 + i, scale=0.1) if cfg["dfs"] else None
    gi = lambda x: None if x is None else x.to(d)

    # prefill
    out, fs = la.prefill(q.to(d), k.to(d), v.to(d), decay.to(d), cu.to(d),
                         initial_state=gi(init), split=cfg["split"])
    torch.cuda.synchronize()
    ref = oracle.quadratic(q, k, v, decay, cu, init_state=init)
    ref_s = oracle.final_state(k, v, decay, cu, init_state=init)
    e_out = _worst(out, ref, cu)
    e_st = float(state_errors(to_np(fs), ref_s).max())

    # backward
    dq, dk, dv, di = la.backward(q.to(d), k.to(d), v.to(d), decay.to(d), do.to(d), cu.to(d),
                                 initial_state=gi(init), d_final_state=gi(dfs),
                                 split=cfg["split"])
    torch.cuda.synchronize()
    rg = oracle.backward(q, k, v, decay, do, cu, init_state=init, d_final=dfs)
    e_bwd = max(_worst(g, r, cu) for g, r in zip((dq, dk, dv), rg[:3]))
    e_di = float(state_errors(to_np(di), rg[3]).max())

    # one decode step from the prefilled states (the oracle steps the GPU's states)
    qd, kd, vd = synth.decode_batch(S, H, D, dtype, seed=6000 + i)
    st = fs.clone()
    od = la.decode_step(qd.to(d), kd.to(d), vd.to(d), decay.to(d), st)
    torch.cuda.synchronize()
    ref_od, ref_st = oracle.decode_step(qd, kd, vd, decay, fs.cpu())
    e_dec = float(max(np.linalg.norm(to_np(od)[b] - ref_od[b]) /
                      max(np.linalg.norm(ref_od[b]), 1e-30) for b in range(S)))
    e_dst = float(state_errors(to_np(st), ref_st).max())

    print("case %d: out %.2e state %.2e bwd %.2e dS0 %.2e decode %.2e dstate %.2e"
          % (i, e_out, e_st, e_bwd, e_di, e_dec, e_dst), flush=True)
    assert e_out <= tol and e_st <= tol, "prefill"
    assert e_bwd <= tol and e_di <= tol, "backward"
    assert e_dec <= tol and e_dst <= F32_TOL, "decode"
