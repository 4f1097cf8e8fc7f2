"""GPU parity of the backward (dq, dk, dv, d_initial_state) against the fp64 oracle's gradients:
the term-by-term form (O6) on ragged varlen batches, the two-scan form (O7) at larger sizes.

Tolerances as for the prefill: relative L2 error per (sequence, head) slice <= 2e-2 for bf16
storage, <= 1e-4 for fp32 storage."""
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


def _gpu_backward(q, k, v, decay, do, cu=None, init=None, dfs=None):
    d = dev()
    g = la.backward(q.to(d), k.to(d), v.to(d), decay.to(d), do.to(d),
                    None if cu is None else cu.to(d),
                    initial_state=None if init is None else init.to(d),
                    d_final_state=None if dfs is None else dfs.to(d))
    torch.cuda.synchronize()
    return g


def _compare(got, want, cu, tol, what):
    names = ("dq", "dk", "dv")
    worst = {}
    for name, g, w in zip(names, got[:3], want[:3]):
        e = slice_errors(to_np(g), w, cu)
        worst[name] = float(e.max())
    worst["d_init"] = float(state_errors(to_np(got[3]), want[3]).max())
    print(what, " ".join("%s %.2e" % kv for kv in worst.items()), flush=True)
    for name, e in worst.items():
        assert e <= tol, "%s: %s error %.3e > %.1e" % (what, name, e, tol)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "f32"])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("with_states", [False, True], ids=["no_states", "states"])
def test_backward_ragged_varlen(dtype, D, with_states):
    """Lengths 1, 63, 64, 65, 0, 130, 200, 7; lambda = 0, 0.95, 1; with and without an initial
    state and a final-state gradient; every row against O6."""
    banner("backward ragged dtype=%s D=%d states=%s" % (dtype, D, with_states))
    H = 3
    cu = synth.cu_from_lengths(RAGGED)
    T = int(cu[-1])
    q, k, v = synth.qkv(T, H, D, dtype, seed=3)
    do, _, _ = synth.qkv(T, H, D, dtype, seed=30)
    decay = torch.tensor([0.0, 0.95, 1.0], dtype=torch.float32)
    init = synth.random_state(len(RAGGED), H, D, seed=4, scale=0.1) if with_states else None
    dfs = synth.random_state(len(RAGGED), H, D, seed=31, scale=0.1) if with_states else None
    got = _gpu_backward(q, k, v, decay, do, cu, init, dfs)
    want = oracle.backward(q, k, v, decay, do, cu, init_state=init, d_final=dfs)
    _compare(got, want, cu, TOL[dtype], "ragged")
    # empty sequence: no gradient flows through it except dS0 = dSn
    if with_states:
        assert torch.equal(got[3][4].cpu(), dfs[4])
    else:
        assert torch.count_nonzero(got[3][4]).item() == 0


def test_backward_8k_recurrent():
    """8 heads x 8,192 tokens, D=128, bf16, lambda 0.9 -> 0.999, with an initial state and a
    final-state gradient: all heads against O7."""
    wl = synth.workloads()["prefill_8k"]
    banner("backward prefill_8k T=8192 H=8 D=128 bf16")
    q, k, v = wl.inputs()
    do, _, _ = synth.qkv(wl.T, wl.H, wl.D, torch.bfloat16, seed=40)
    decay = wl.decay()
    init = synth.random_state(1, wl.H, wl.D, seed=41, scale=0.05)
    dfs = synth.random_state(1, wl.H, wl.D, seed=42, scale=0.05)
    got = _gpu_backward(q, k, v, decay, do, None, init, dfs)
    want = oracle.backward_recurrent(q, k, v, decay, do, init_state=init, d_final=dfs)
    _compare(got, want, [0, wl.T], BF16_TOL, "8k")


def test_backward_64k_sampled_heads():
    """The 65,536-token x 64-head layer (GPU inputs): heads {0, 21, 42, 63} against O7."""
    wl = synth.workloads()["prefill_64k"]
    banner("backward prefill_64k T=65536 H=64 D=128 bf16 (GPU inputs)")
    q, k, v = wl.inputs(device="cuda")
    do, _, _ = synth.qkv(wl.T, wl.H, wl.D, torch.bfloat16, seed=50, device="cuda")
    decay = wl.decay()
    dq, dk, dv, di = la.backward(q, k, v, decay.to(dev()), do)
    torch.cuda.synchronize()
    hs = [0, 21, 42, 63]
    pick = lambda x: x[:, hs, :].contiguous().cpu()
    want = oracle.backward_recurrent(pick(q), pick(k), pick(v), decay[hs], pick(do))
    got = (pick(dq), pick(dk), pick(dv), di[:, hs].cpu())
    _compare(got, want, [0, wl.T], BF16_TOL, "64k sampled heads")


def test_backward_deterministic():
    banner("backward determinism T=3000 H=4 D=128 bf16")
    q, k, v = synth.qkv(3000, 4, 128, torch.bfloat16, seed=60)
    do, _, _ = synth.qkv(3000, 4, 128, torch.bfloat16, seed=61)
    decay = synth.decay_geometric(4, 0.9, 0.999)
    a = _gpu_backward(q, k, v, decay, do)
    b = _gpu_backward(q, k, v, decay, do)
    for x, y in zip(a, b):
        assert torch.equal(x, y)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "f32"])
def test_autograd_function(dtype):
    """torch.autograd through lightning_attention (loss = <W, out> + <W2, final_state>) gives the
    oracle's gradients for q, k, v and the initial state."""
    banner("autograd dtype=%s" % dtype)
    lengths = [100, 0, 37]
    H, D = 2, 64
    cu = synth.cu_from_lengths(lengths)
    T = int(cu[-1])
    q, k, v = synth.qkv(T, H, D, dtype, seed=70)
    W, _, _ = synth.qkv(T, H, D, dtype, seed=71)
    W2 = synth.random_state(len(lengths), H, D, seed=72, scale=0.1)
    init = synth.random_state(len(lengths), H, D, seed=73, scale=0.1)
    decay = torch.tensor([0.9, 1.0])
    d = dev()
    qg, kg, vg, sg = (x.to(d).requires_grad_() for x in (q, k, v, init))
    out, fs = la.lightning_attention(qg, kg, vg, decay.to(d), cu.to(d), sg)
    loss = (out.float() * W.to(d).float()).sum() + (fs * W2.to(d)).sum()
    loss.backward()
    torch.cuda.synchronize()
    # the upstream gradient autograd hands the op is W in the output dtype
    want = oracle.backward(q, k, v, decay, W, cu, init_state=init, d_final=W2)
    got = (qg.grad, kg.grad, vg.grad, sg.grad)
    _compare(got, want, cu, TOL[dtype], "autograd")


def _gpu_backward_split(q, k, v, decay, do, cu, init, dfs, seg_blocks):
    d = dev()
    g = la.backward(q.to(d), k.to(d), v.to(d), decay.to(d), do.to(d),
                    None if cu is None else cu.to(d),
                    initial_state=None if init is None else init.to(d),
                    d_final_state=None if dfs is None else dfs.to(d), split=seg_blocks)
    torch.cuda.synchronize()
    return g


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "f32"])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("with_states", [False, True], ids=["no_states", "states"])
@pytest.mark.parametrize("seg_blocks", [1, 2])
def test_backward_split_ragged_varlen(dtype, D, with_states, seg_blocks):
    """The sequence-split backward on the ragged batch (segments of 64 or 128 tokens cut the
    65-, 130- and 200-token sequences; the last segment of the 65-token one has a single token,
    where the reversed scans' first segment decays dSn by lambda^0; lambda = 0, 0.95, 1): every
    row against O6, and dS0 of the empty sequence = dSn."""
    banner("backward split ragged dtype=%s D=%d states=%s seg_blocks=%d"
           % (dtype, D, with_states, seg_blocks))
    H = 3
    cu = synth.cu_from_lengths(RAGGED)
    T = int(cu[-1])
    q, k, v = synth.qkv(T, H, D, dtype, seed=3)
    do, _, _ = synth.qkv(T, H, D, dtype, seed=30)
    decay = torch.tensor([0.0, 0.95, 1.0], dtype=torch.float32)
    init = synth.random_state(len(RAGGED), H, D, seed=4, scale=0.1) if with_states else None
    dfs = synth.random_state(len(RAGGED), H, D, seed=31, scale=0.1) if with_states else None
    got = _gpu_backward_split(q, k, v, decay, do, cu, init, dfs, seg_blocks)
    want = oracle.backward(q, k, v, decay, do, cu, init_state=init, d_final=dfs)
    _compare(got, want, cu, TOL[dtype], "split ragged")
    if with_states:
        assert torch.equal(got[3][4].cpu(), dfs[4])
    else:
        assert torch.count_nonzero(got[3][4]).item() == 0


def test_backward_split_8k_recurrent():
    """8 heads x 8,192 tokens, D=128, bf16, 16-block segments (8 per sequence), with an initial
    state and a final-state gradient: all heads against O7, and against the unsplit backward.

    The two paths round different bf16 operands (the split's segment states weight each token by
    its power of lambda within the segment, the plain scan by its power within a 64-token block),
    so they agree to bf16 rounding, not bit for bit: the fp32 d_initial_state of each is checked
    against the oracle, and the split's error must stay within twice the plain one's."""
    wl = synth.workloads()["prefill_8k"]
    banner("backward split prefill_8k T=8192 H=8 D=128 bf16 seg_blocks=16")
    q, k, v = wl.inputs()
    do, _, _ = synth.qkv(wl.T, wl.H, wl.D, torch.bfloat16, seed=40)
    decay = wl.decay()
    init = synth.random_state(1, wl.H, wl.D, seed=41, scale=0.05)
    dfs = synth.random_state(1, wl.H, wl.D, seed=42, scale=0.05)
    got = _gpu_backward_split(q, k, v, decay, do, None, init, dfs, 16)
    want = oracle.backward_recurrent(q, k, v, decay, do, init_state=init, d_final=dfs)
    _compare(got, want, [0, wl.T], BF16_TOL, "split 8k")
    plain = _gpu_backward(q, k, v, decay, do, None, init, dfs)
    _compare(plain, want, [0, wl.T], BF16_TOL, "plain 8k")
    for name, a, b in zip(("dq", "dk", "dv"), got[:3], plain[:3]):
        e = slice_errors(to_np(a), to_np(b).astype(np.float64), [0, wl.T])
        assert float(e.max()) <= BF16_TOL, name
    e_split = state_errors(to_np(got[3]), want[3]).max()
    e_plain = state_errors(to_np(plain[3]), want[3]).max()
    print("d_init vs oracle: split %.2e plain %.2e" % (e_split, e_plain))
    assert e_split <= 2 * e_plain + 1e-5


def test_autograd_split_matches_plain():
    """lightning_attention(split=2) gives the same gradients as split=None (fp32, 2 heads,
    ragged lengths), within fp32 rounding."""
    banner("autograd split vs plain")
    d = dev()
    cu = synth.cu_from_lengths([300, 5, 129]).to(d)
    T = 434
    grads = []
    for split in (None, 2):
        q, k, v = (x.to(d).requires_grad_(True) for x in synth.qkv(T, 2, 64, torch.float32, seed=7))
        decay = torch.tensor([0.9, 0.99], device=d)
        init = synth.random_state(3, 2, 64, seed=8, scale=0.1).to(d).requires_grad_(True)
        out, fs = la.lightning_attention(q, k, v, decay, cu, initial_state=init, split=split)
        (out.square().sum() + fs.square().sum()).backward()
        grads.append([x.grad.detach().cpu().double() for x in (q, k, v, init)])
    for a, b in zip(*grads):
        assert float((a - b).norm() / b.norm()) <= 1e-4


def test_backward_split_empty_and_deterministic():
    """Split backward: a batch of empty sequences (no segments) leaves dS0 = dSn; two calls on
    the same inputs give bitwise-equal gradients."""
    banner("backward split empty batch and determinism")
    d = dev()
    H, D = 2, 128
    dfs = synth.random_state(2, H, D, seed=70, scale=0.1)
    z = torch.zeros((0, H, D), dtype=torch.bfloat16)
    cu = torch.tensor([0, 0, 0], dtype=torch.int32)
    decay = torch.tensor([0.9, 0.5], dtype=torch.float32)
    _, _, _, di = _gpu_backward_split(z, z, z, decay, z, cu, None, dfs, 4)
    assert torch.equal(di.cpu(), dfs)
    q, k, v = synth.qkv(3000, 4, 128, torch.bfloat16, seed=60)
    do, _, _ = synth.qkv(3000, 4, 128, torch.bfloat16, seed=61)
    dec = synth.decay_geometric(4, 0.9, 0.999)
    a = _gpu_backward_split(q, k, v, dec, do, None, None, None, 4)
    b = _gpu_backward_split(q, k, v, dec, do, None, None, None, 4)
    for x, y in zip(a, b):
        assert torch.equal(x, y)
