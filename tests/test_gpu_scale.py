"""GPU parity at the full workload sizes, in the launch configuration the benchmark times:

* 64 heads x 65,536 tokens (one MiniMax-like layer): every output and state of all heads
  against the oracle's recurrent form, plus block-edge rows and 32 random rows of every head
  (256 random rows of heads {0, 21, 42, 63}) against the quadratic (definition) form;
* 16 packed sequences of 1,024..32,768 tokens x 64 heads: every output and state of every
  (sequence, head) pair against the recurrent form;
* 1,048,576 tokens x 64 heads (int64 indexing: T*H*D > 2^31): heads {0, 21, 42, 63} against
  the recurrent form;
* one decode step for 256 sequences x 64 heads of fp32 128x128 states: every pair;
* the sequence-split backward of 65,536 tokens x 8 heads (all heads) against the oracle's
  two-scan gradient form (the 64-head backward is in test_gpu_backward.py);
* the fp32-storage path at length: 2 packed sequences of 40,003 and 25,590 tokens x 8 heads
  with initial states (prefill, plain and split), and the backward of 16,411 tokens x 4 heads
  (plain and split), at the fp32 tolerance;
* a split prefill of 1,200,000 tokens x 8 heads with 1,048,576-token segments (past the
  offset range of the token-parallel segment states: the state-only scan runs instead).
"""
import numpy as np
import pytest
import torch

import long_context_attention_attn_amd as la
import oracle
from gpu_util import BF16_TOL, F32_TOL, banner, dev, rel, slice_errors, state_errors, to_np
from long_context_attention_attn_amd import synth

pytestmark = pytest.mark.gpu

SAMPLED_HEADS = [0, 21, 42, 63]


def _heads(x, heads):
    return x[:, heads, :].contiguous().cpu()


def test_prefill_64k_all_heads():
    wl = synth.workloads()["prefill_64k"]
    banner("prefill_64k T=65536 H=64 D=128 bf16 (GPU inputs)")
    q, k, v = wl.inputs(device="cuda")
    decay = wl.decay()
    out, fs = la.prefill(q, k, v, decay.to(dev()))
    torch.cuda.synchronize()
    worst, worst_s = 0.0, 0.0
    for h0 in range(0, wl.H, 16):
        hs = list(range(h0, h0 + 16))
        qh, kh, vh = _heads(q, hs), _heads(k, hs), _heads(v, hs)
        ref, ref_s = oracle.recurrent(qh, kh, vh, decay[hs])
        e = slice_errors(to_np(_heads(out, hs)), ref, [0, wl.T])
        es = state_errors(to_np(fs[:, hs]), ref_s)
        worst, worst_s = max(worst, e.max()), max(worst_s, es.max())
        print("heads %d..%d: out %.2e state %.2e" % (h0, h0 + 15, e.max(), es.max()), flush=True)
    # Sampled rows against the quadratic (definition) form: block edges and 32 random rows on
    # every head, 256 random rows on heads spanning the decay range.
    rng = np.random.default_rng(0)
    edges = [0, 1, 63, 64, 65, 127, 128, 129, 4095, 4096, 4097, wl.T - 65, wl.T - 64, wl.T - 2,
             wl.T - 1]
    qc, kc, vc = q.cpu(), k.cpu(), v.cpu()
    for hs, n_rand in ((list(range(wl.H)), 32), (SAMPLED_HEADS, 256)):
        rows = sorted(set(edges + [int(x) for x in rng.integers(0, wl.T, n_rand)]))
        refr = oracle.quadratic_rows(qc[:, hs].contiguous(), kc[:, hs].contiguous(),
                                     vc[:, hs].contiguous(), decay[hs], rows)
        got = to_np(out[rows][:, hs])
        for i, h in enumerate(hs):
            assert rel(got[:, i], refr[:, i]) <= BF16_TOL, "row sample head %d" % h
        print("%d rows x %d heads against the quadratic form: ok" % (len(rows), len(hs)),
              flush=True)
    print("prefill_64k: worst out %.2e worst state %.2e" % (worst, worst_s))
    assert worst <= BF16_TOL and worst_s <= BF16_TOL


def test_varlen_16_all_heads():
    wl = synth.workloads()["varlen_16"]
    banner("varlen_16 T=%d S=16 H=64 D=128 bf16 (GPU inputs)" % wl.T)
    q, k, v = wl.inputs(device="cuda")
    decay = wl.decay()
    cu = wl.cu_seqlens()
    out, fs = la.prefill(q, k, v, decay.to(dev()), cu.to(dev()))
    torch.cuda.synchronize()
    worst, worst_s = 0.0, 0.0
    for h0 in range(0, wl.H, 16):
        hs = list(range(h0, h0 + 16))
        ref, ref_s = oracle.recurrent(_heads(q, hs), _heads(k, hs), _heads(v, hs), decay[hs], cu)
        e = slice_errors(to_np(_heads(out, hs)), ref, cu)
        es = state_errors(to_np(fs[:, hs]), ref_s)
        worst, worst_s = max(worst, e.max()), max(worst_s, es.max())
        print("heads %d..%d: out %.2e state %.2e" % (h0, h0 + 15, e.max(), es.max()), flush=True)
    print("varlen_16: worst out %.2e worst state %.2e" % (worst, worst_s))
    assert worst <= BF16_TOL and worst_s <= BF16_TOL


def test_prefill_1m_sampled_heads():
    wl = synth.workloads()["prefill_1m"]
    banner("prefill_1m T=1048576 H=64 D=128 bf16 (GPU inputs)")
    q, k, v = wl.inputs(device="cuda")
    decay = wl.decay()
    out, fs = la.prefill(q, k, v, decay.to(dev()))
    torch.cuda.synchronize()
    hs = SAMPLED_HEADS
    qh, kh, vh, oh = _heads(q, hs), _heads(k, hs), _heads(v, hs), _heads(out, hs)
    del q, k, v, out
    ref, ref_s = oracle.recurrent(qh, kh, vh, decay[hs])
    e = slice_errors(to_np(oh), ref, [0, wl.T])
    es = state_errors(to_np(fs[:, hs]), ref_s)
    print("prefill_1m: out", np.array2string(e[0], formatter={"float_kind": lambda x: "%.2e" % x}), "state",
          np.array2string(es[0], formatter={"float_kind": lambda x: "%.2e" % x}))
    assert e.max() <= BF16_TOL and es.max() <= BF16_TOL


def test_decode_256x64():
    banner("decode Bt=256 H=64 D=128 bf16, fp32 states")
    Bt, H, D = 256, 64, 128
    q, k, v = synth.decode_batch(Bt, H, D, torch.bfloat16, seed=2)
    decay = synth.decay_geometric(H, 0.9, 0.9999)
    st0 = synth.random_state(Bt, H, D, seed=1, scale=0.1)
    st = st0.to(dev())
    out = la.decode_step(q.to(dev()), k.to(dev()), v.to(dev()), decay.to(dev()), st)
    torch.cuda.synchronize()
    ref_o, ref_s = oracle.decode_step(q, k, v, decay, st0)
    got = to_np(out)
    e = max(rel(got[b, h], ref_o[b, h]) for b in range(Bt) for h in range(H))
    es = float(np.abs(to_np(st) - ref_s).max() / np.abs(ref_s).max())
    print("decode_256x64: out %.2e state(max-abs rel) %.2e" % (e, es))
    assert e <= BF16_TOL and es <= 1e-6


def test_prefill_64k_d64_all_heads():
    """65,536 tokens x 16 heads x d64 (bf16, GPU inputs): every head against the recurrent form,
    plus sampled rows against the quadratic form."""
    banner("prefill T=65536 H=16 D=64 bf16 (GPU inputs)")
    T, H, D = 65536, 16, 64
    q, k, v = synth.qkv(T, H, D, torch.bfloat16, seed=7, device="cuda")
    decay = synth.decay_geometric(H, 0.9, 0.9999)
    out, fs = la.prefill(q, k, v, decay.to(dev()))
    torch.cuda.synchronize()
    qc, kc, vc = q.cpu(), k.cpu(), v.cpu()
    ref, ref_s = oracle.recurrent(qc, kc, vc, decay)
    e = slice_errors(to_np(out), ref, [0, T])
    es = state_errors(to_np(fs), ref_s)
    rows = [0, 63, 64, 4097, T - 1]
    er = max(rel(to_np(out[rows])[:, h], oracle.quadratic_rows(qc, kc, vc, decay, rows)[:, h])
             for h in range(H))
    print("prefill d64: out %.2e state %.2e rows %.2e" % (e.max(), es.max(), er))
    assert e.max() <= BF16_TOL and es.max() <= BF16_TOL and er <= BF16_TOL


def _check_grads(got, want, T, what):
    worst = 0.0
    for name, g, w in zip(("dq", "dk", "dv"), got, want):
        e = slice_errors(to_np(g), w, [0, T])
        print("%s %s: max rel-L2 %.2e" % (what, name, e.max()), flush=True)
        worst = max(worst, float(e.max()))
    assert worst <= BF16_TOL, "%s: %.3e" % (what, worst)


def test_backward_split_64k_8_heads():
    """The benchmark's few-chain backward: 65,536 tokens x 8 heads, split as the library
    suggests for this device; all heads against O7."""
    T, H, D = 65536, 8, 128
    banner("backward split T=65536 H=8 D=128 bf16 (auto segments)")
    q, k, v = synth.qkv(T, H, D, torch.bfloat16, seed=0, device="cuda")
    do, _, _ = synth.qkv(T, H, D, torch.bfloat16, seed=50, device="cuda")
    decay = synth.decay_geometric(H, 0.9, 0.9999)
    dq, dk, dv, _ = la.backward(q, k, v, decay.to(dev()), do, want_d_initial_state=False,
                                split="auto")
    torch.cuda.synchronize()
    want = oracle.backward_recurrent(q.cpu(), k.cpu(), v.cpu(), decay, do.cpu(),
                                     want_d_init=False)
    _check_grads([x.cpu() for x in (dq, dk, dv)], want[:3], T, "backward split 64k x 8")


def test_prefill_f32_long_ragged_init():
    """fp32 storage, 2 packed sequences with ragged tails (40,003 and 25,590 tokens) x 8 heads,
    initial states ~ N(0, 0.1^2): every head of both sequences, outputs and final states, against
    the recurrent form; the sequence-split prefill the same way."""
    cu = torch.tensor([0, 40003, 65593], dtype=torch.int32)
    T, H, D, S = 65593, 8, 128, 2
    banner("prefill fp32 T=%d (2 sequences) H=%d D=%d with initial states" % (T, H, D))
    q, k, v = synth.qkv(T, H, D, torch.float32, seed=11)
    decay = synth.decay_geometric(H, 0.9, 0.9999)
    s0 = synth.random_state(S, H, D, seed=12, scale=0.1)
    ref, ref_s = oracle.recurrent(q, k, v, decay, cu, s0)
    args = [x.to(dev()) for x in (q, k, v, decay)]
    for split in (None, "auto"):
        out, fs = la.prefill(*args, cu.to(dev()), initial_state=s0.to(dev()), split=split)
        torch.cuda.synchronize()
        e = slice_errors(to_np(out), ref, cu.tolist())
        es = state_errors(to_np(fs), ref_s)
        print("fp32 prefill split=%s: out %.2e state %.2e" % (split, e.max(), es.max()),
              flush=True)
        assert e.max() <= F32_TOL and es.max() <= F32_TOL, split


def test_backward_f32_16k():
    """fp32 storage backward, 16,411 tokens x 4 heads (a ragged tail; the fp32 kernel in its
    reversed, state-only and inclusive-initial-state modes), plain and split, against O7."""
    T, H, D = 16411, 4, 128
    banner("backward fp32 T=%d H=%d D=%d" % (T, H, D))
    q, k, v = synth.qkv(T, H, D, torch.float32, seed=13)
    do, _, _ = synth.qkv(T, H, D, torch.float32, seed=14)
    decay = synth.decay_geometric(H, 0.9, 0.9999)
    want = oracle.backward_recurrent(q, k, v, decay, do, want_d_init=False)
    args = [x.to(dev()) for x in (q, k, v, decay, do)]
    for split in (None, 4):
        dq, dk, dv, _ = la.backward(*args, want_d_initial_state=False, split=split)
        torch.cuda.synchronize()
        worst = 0.0
        for name, g, w in zip(("dq", "dk", "dv"), (dq, dk, dv), want[:3]):
            e = slice_errors(to_np(g), w, [0, T])
            worst = max(worst, float(e.max()))
        print("fp32 backward split=%s: worst rel-L2 %.2e" % (split, worst), flush=True)
        assert worst <= F32_TOL, split


def test_split_segments_past_offset_range():
    """Split prefill whose longest segment (1,048,576 tokens x 8 heads x d128 bf16) is past the
    32-bit offset range of the token-parallel segment states, so step 2 runs the block scan's
    state-only form instead: heads {0, 7} against the recurrent form, outputs and final states."""
    T, H, D, seg_blocks = 1_200_000, 8, 128, 16384
    banner("split prefill T=%d H=%d D=%d bf16 seg_blocks=%d (segment-state fallback)"
           % (T, H, D, seg_blocks))
    q, k, v = synth.qkv(T, H, D, torch.bfloat16, seed=21, device="cuda")
    decay = synth.decay_geometric(H, 0.9, 0.9999)
    out, fs = la.prefill(q, k, v, decay.to(dev()), split=seg_blocks)
    torch.cuda.synchronize()
    heads = [0, H - 1]
    ref, ref_s = oracle.recurrent(_heads(q, heads), _heads(k, heads), _heads(v, heads),
                                  decay[heads])
    e = slice_errors(to_np(_heads(out, heads)), ref, [0, T])
    es = state_errors(to_np(fs[:, heads]), ref_s)
    print("split fallback: out %.2e state %.2e" % (e.max(), es.max()))
    assert e.max() <= BF16_TOL and es.max() <= BF16_TOL
