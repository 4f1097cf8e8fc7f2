"""GPU parity of the sequence-split prefill (segments scanned in parallel, then combined) against
the fp64 oracle, and against the plain prefill.

Segment lengths of 1 and 2 blocks put segment boundaries inside every sequence of the ragged
batch, next to empty sequences and partial last blocks; segments of 9 and 16 blocks give every
wave of the bf16 segment-state kernel several 32-token chunks (an odd and an even number, and a
partial last chunk) at both head sizes, forward and reversed; the 8k x 8 and 64k x 8 cases are
the few-chain shapes the split exists for.
"""
import numpy as np
import pytest
import torch

import long_context_attention_attn_amd as la
import oracle
from gpu_util import BF16_TOL, F32_TOL, banner, dev, slice_errors, state_errors, to_np
from long_context_attention_attn_amd import synth

pytestmark = pytest.mark.gpu

TOL = {torch.bfloat16: BF16_TOL, torch.float32: F32_TOL}
RAGGED = [1, 63, 64, 65, 0, 130, 200, 7]


def _split_prefill(q, k, v, decay, cu=None, init=None, split=None):
    d = dev()
    out, fs = la.prefill(q.to(d), k.to(d), v.to(d), decay.to(d), None if cu is None else cu.to(d),
                         initial_state=None if init is None else init.to(d), split=split)
    torch.cuda.synchronize()
    return out, fs


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "f32"])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("with_init", [False, True], ids=["zero_state", "init_state"])
@pytest.mark.parametrize("seg_blocks", [1, 2])
def test_split_ragged_varlen(dtype, D, with_init, seg_blocks):
    banner("split ragged dtype=%s D=%d init=%s seg_blocks=%d" % (dtype, D, with_init, seg_blocks))
    H = 3
    cu = synth.cu_from_lengths(RAGGED)
    q, k, v = synth.qkv(int(cu[-1]), H, D, dtype, seed=3)
    decay = torch.tensor([0.0, 0.95, 1.0], dtype=torch.float32)
    init = synth.random_state(len(RAGGED), H, D, seed=4, scale=0.1) if with_init else None
    out, fs = _split_prefill(q, k, v, decay, cu, init, split=seg_blocks)
    ref = oracle.quadratic(q, k, v, decay, cu, init_state=init)
    ref_s = oracle.final_state(k, v, decay, cu, init_state=init)
    e = slice_errors(to_np(out), ref, cu)
    es = state_errors(to_np(fs), ref_s)
    print("split ragged: max out %.2e max state %.2e" % (e.max(), es.max()))
    assert e.max() <= TOL[dtype] and es.max() <= TOL[dtype]
    if not with_init:
        assert torch.count_nonzero(fs[4]).item() == 0
    else:
        assert torch.equal(fs[4].cpu(), init[4])


def test_split_8k_full_quadratic():
    """8 heads x 8,192 tokens (32 workgroups unsplit): split into 16-block segments and 'auto',
    every row against the quadratic oracle."""
    wl = synth.workloads()["prefill_8k"]
    banner("split prefill_8k T=8192 H=8 D=128 bf16")
    q, k, v = wl.inputs()
    decay = wl.decay()
    ref = oracle.quadratic(q, k, v, decay)
    ref_s = oracle.final_state(k, v, decay)
    for split in (16, "auto"):
        out, fs = _split_prefill(q, k, v, decay, split=split)
        e = slice_errors(to_np(out), ref, [0, wl.T])
        es = state_errors(to_np(fs), ref_s)
        print("split=%s: out %.2e state %.2e" % (split, e.max(), es.max()))
        assert e.max() <= BF16_TOL and es.max() <= BF16_TOL


def test_split_matches_plain_and_is_deterministic():
    banner("split vs plain T=5000 H=4 D=128 bf16")
    q, k, v = synth.qkv(5000, 4, 128, torch.bfloat16, seed=21)
    decay = synth.decay_geometric(4, 0.9, 0.9999)
    o1, s1 = _split_prefill(q, k, v, decay, split=3)
    o2, s2 = _split_prefill(q, k, v, decay, split=3)
    assert torch.equal(o1, o2) and torch.equal(s1, s2)
    op, sp = _split_prefill(q, k, v, decay)
    assert slice_errors(to_np(o1), to_np(op), [0, 5000]).max() <= BF16_TOL
    assert state_errors(to_np(s1), to_np(sp)).max() <= BF16_TOL


def test_split_64k_8_heads_recurrent():
    """65,536 tokens x 8 heads (one device's share of the 64-head layer under 8-way head
    sharding): 'auto' split, all heads against the recurrent oracle."""
    banner("split T=65536 H=8 D=128 bf16 auto")
    T, H, D = 65536, 8, 128
    q, k, v = synth.qkv(T, H, D, torch.bfloat16, seed=0)
    decay = synth.decay_geometric(H, 0.9, 0.9999)
    out, fs = _split_prefill(q, k, v, decay, split="auto")
    ref, ref_s = oracle.recurrent(q, k, v, decay)
    e = slice_errors(to_np(out), ref, [0, T])
    es = state_errors(to_np(fs), ref_s)
    print("split 64k x 8: out", np.array2string(e[0], formatter={"float_kind": lambda x: "%.2e" % x}),
          "state max %.2e" % es.max())
    assert e.max() <= BF16_TOL and es.max() <= BF16_TOL


LONG = [3001, 1, 2500, 0, 700, 1153]


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("seg_blocks", [9, 16])
def test_split_long_segments(D, seg_blocks):
    """bf16, segments of 576 or 1,024 tokens over ragged sequences of 0..3,001 tokens (18 or 32
    chunks per full segment: 2-4 per wave, partial last chunks), lambda = 0, 0.9, 0.999, 1 and an
    initial state: the split prefill against O1 and O3, and the split backward (its reversed
    segment states) against O7."""
    banner("split long segments D=%d seg_blocks=%d" % (D, seg_blocks))
    H = 4
    cu = synth.cu_from_lengths(LONG)
    T = int(cu[-1])
    q, k, v = synth.qkv(T, H, D, torch.bfloat16, seed=60)
    do, _, _ = synth.qkv(T, H, D, torch.bfloat16, seed=61)
    decay = torch.tensor([0.0, 0.9, 0.999, 1.0], dtype=torch.float32)
    init = synth.random_state(len(LONG), H, D, seed=62, scale=0.1)
    dfs = synth.random_state(len(LONG), H, D, seed=63, scale=0.1)
    out, fs = _split_prefill(q, k, v, decay, cu, init, split=seg_blocks)
    ref = oracle.quadratic(q, k, v, decay, cu, init_state=init)
    ref_s = oracle.final_state(k, v, decay, cu, init_state=init)
    e = slice_errors(to_np(out), ref, cu)
    es = state_errors(to_np(fs), ref_s)
    d = dev()
    g = la.backward(q.to(d), k.to(d), v.to(d), decay.to(d), do.to(d), cu.to(d),
                    initial_state=init.to(d), d_final_state=dfs.to(d), split=seg_blocks)
    torch.cuda.synchronize()
    want = oracle.backward_recurrent(q, k, v, decay, do, cu, init_state=init, d_final=dfs)
    eg = [float(slice_errors(to_np(x), w, cu).max()) for x, w in zip(g[:3], want[:3])]
    eg.append(float(state_errors(to_np(g[3]), want[3]).max()))
    print("split long: out %.2e state %.2e dq %.2e dk %.2e dv %.2e d_init %.2e"
          % (e.max(), es.max(), *eg))
    assert e.max() <= BF16_TOL and es.max() <= BF16_TOL and max(eg) <= BF16_TOL


def test_split_suggestion_uses_the_device():
    """la_prefill_split_blocks on the device equals the pure rule at the device's CU count, and
    split="auto" runs the suggested segment length (same outputs as that explicit split)."""
    from long_context_attention_attn_amd import _lib

    cus = torch.cuda.get_device_properties(0).multi_processor_count
    for T, S, H, D, dt in ((65536, 1, 8, 128, 1), (4096, 1, 8, 128, 1), (1024, 1, 8, 128, 0),
                           (512, 1, 1, 64, 1), (65536, 1, 64, 128, 1), (200000, 4, 4, 64, 0)):
        assert (_lib.prefill_split_blocks(T, S, H, D, dt)
                == _lib.prefill_split_blocks_for(T, S, H, D, dt, cus)), (T, S, H, D, dt)
    T, H, D = 8192, 8, 128
    seg = _lib.prefill_split_blocks(T, 1, H, D, _lib.LA_BF16)
    assert seg > 0
    q, k, v = synth.qkv(T, H, D, torch.bfloat16, seed=70)
    decay = synth.decay_geometric(H, 0.9, 0.9999)
    oa, fa = _split_prefill(q, k, v, decay, split="auto")
    ob, fb = _split_prefill(q, k, v, decay, split=seg)
    assert torch.equal(oa, ob) and torch.equal(fa, fb)


@pytest.mark.parametrize("D", [64, 128])
def test_split_two_launch_path_packed(D):
    """The bf16 split in two launches (segments found on the device, incoming states formed in
    the segment prefill's prologue): packed sequences with empty ones, initial states, up to 16
    segments per sequence, against the oracle; bitwise deterministic."""
    lengths = [1000, 0, 1, 64, 2049, 0, 700]
    H = 3
    banner("split two-launch D=%d lengths=%s" % (D, lengths))
    d = dev()
    cu = synth.cu_from_lengths(lengths)
    T = int(cu[-1])
    q, k, v = synth.qkv(T, H, D, torch.bfloat16, seed=61)
    decay = torch.tensor([0.0, 0.93, 1.0], dtype=torch.float32)
    init = synth.random_state(len(lengths), H, D, seed=62, scale=0.1)
    seg = 4  # 256-token segments: ceil(T / 256) = 16, within the two-launch path's bound
    assert (T + 64 * seg - 1) // (64 * seg) <= 16
    outs = []
    for _ in range(2):
        out, fs = la.prefill(q.to(d), k.to(d), v.to(d), decay.to(d), cu.to(d),
                             initial_state=init.to(d), split=seg)
        torch.cuda.synchronize()
        outs.append((out.cpu(), fs.cpu()))
    assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1])
    ref = oracle.quadratic(q, k, v, decay, cu, init_state=init)
    ref_s = oracle.final_state(k, v, decay, cu, init_state=init)
    e = slice_errors(to_np(outs[0][0]), ref, cu).max()
    es = state_errors(to_np(outs[0][1]), ref_s).max()
    print("two-launch split D=%d: out %.2e state %.2e" % (D, e, es))
    assert e <= BF16_TOL and es <= BF16_TOL
    # empty sequences keep their initial state exactly
    for s in (1, 5):
        assert torch.equal(outs[0][1][s], init[s])


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("seg_blocks", [64, 66])
def test_split_long_segment_kernels(D, seg_blocks):
    """Segments of 4,096 tokens (whole 128-token blocks: the 128-token segment scans) and of
    4,224 tokens (the 64-token ones) over packed sequences with an empty one and a partial last
    block, from initial states: the split prefill against the recurrent form, the split
    backward against O7."""
    lengths = [9000, 0, 4096, 5000, 129]
    H = 2
    banner("split long segment kernels D=%d seg_blocks=%d" % (D, seg_blocks))
    d = dev()
    cu = synth.cu_from_lengths(lengths)
    q, k, v = synth.qkv(int(cu[-1]), H, D, torch.bfloat16, seed=63)
    decay = torch.tensor([0.95, 0.9999], dtype=torch.float32)
    init = synth.random_state(len(lengths), H, D, seed=64, scale=0.1)
    out, fs = la.prefill(q.to(d), k.to(d), v.to(d), decay.to(d), cu.to(d),
                         initial_state=init.to(d), split=seg_blocks)
    torch.cuda.synchronize()
    ref, ref_s = oracle.recurrent(q, k, v, decay, cu, init_state=init)
    e = slice_errors(to_np(out), ref, cu).max()
    es = state_errors(to_np(fs), ref_s).max()
    print("long segments D=%d seg=%d: out %.2e state %.2e" % (D, seg_blocks, e, es))
    assert e <= BF16_TOL and es <= BF16_TOL
    assert torch.equal(fs.cpu()[1], init[1])
    # the split backward over the same segments (its reversed segment scans with per-sequence
    # inclusive states) against O7
    do, _, _ = synth.qkv(int(cu[-1]), H, D, torch.bfloat16, seed=65)
    dfs = synth.random_state(len(lengths), H, D, seed=66, scale=0.1)
    g = la.backward(q.to(d), k.to(d), v.to(d), decay.to(d), do.to(d), cu.to(d),
                    initial_state=init.to(d), d_final_state=dfs.to(d), split=seg_blocks)
    torch.cuda.synchronize()
    want = oracle.backward_recurrent(q, k, v, decay, do, cu, init_state=init, d_final=dfs)
    eg = [float(slice_errors(to_np(x), w, cu).max()) for x, w in zip(g[:3], want[:3])]
    eg.append(float(state_errors(to_np(g[3]), want[3]).max()))
    print("  backward: dq %.2e dk %.2e dv %.2e d_init %.2e" % tuple(eg))
    assert max(eg) <= BF16_TOL


@pytest.mark.gpu
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("lengths,seg_blocks", [([16384], 128), ([12288, 0, 3000], 64)])
def test_split_sub_segment_states(D, lengths, seg_blocks):
    """Too few segments before each sequence's last to fill the device, so the two-launch state
    pass computes their states in sub-segments that the later segments' prologues add up: one
    sequence in two 8,192-token segments (four 2,048-token sub-segments), and a packed batch
    whose first sequence has three 4,096-token segments (two sub-segments each) beside an empty
    and a one-segment sequence.  From initial states, against the recurrent form, with the plain
    prefill beside it."""
    H = 2
    banner("split sub-segment states D=%d lengths=%s seg_blocks=%d" % (D, lengths, seg_blocks))
    d = dev()
    cu = synth.cu_from_lengths(lengths)
    T = int(cu[-1])
    q, k, v = synth.qkv(T, H, D, torch.bfloat16, seed=71)
    decay = torch.tensor([0.999, 0.99995], dtype=torch.float32)
    init = synth.random_state(len(lengths), H, D, seed=72, scale=0.1)
    out, fs = la.prefill(q.to(d), k.to(d), v.to(d), decay.to(d), cu.to(d),
                         initial_state=init.to(d), split=seg_blocks)
    po, pfs = la.prefill(q.to(d), k.to(d), v.to(d), decay.to(d), cu.to(d),
                         initial_state=init.to(d))
    torch.cuda.synchronize()
    ref, ref_s = oracle.recurrent(q, k, v, decay, cu, init_state=init)
    e = slice_errors(to_np(out), ref, cu).max()
    es = state_errors(to_np(fs), ref_s).max()
    ep = slice_errors(to_np(po), ref, cu).max()
    print("sub-segment states D=%d: out %.2e state %.2e (plain %.2e)" % (D, e, es, ep))
    assert e <= BF16_TOL and es <= BF16_TOL and ep <= BF16_TOL
