"""GPU checks of the finite-input contract of include/lightning_attn.h.

The definition masks future tokens by selection (o_t sums over s <= t only), so a non-finite
value can never reach an earlier output.  The kernels keep that exactly for q and k: future
scores are selected away in registers and the running state carries a token only forward.  For
v it holds across blocks but not inside one: the intra-block product multiplies the exactly-zero
masked weights by v on the matrix cores, and 0 * inf is NaN there.  So a non-finite v at local
token t of a block can reach earlier rows of the same operand group (32 tokens in bf16, the
16-token tile in fp32), never an earlier group, block or sequence.  Each case compares a run
with one poisoned token against a clean run bit for bit on the rows the contract keeps clean.
"""
import pytest
import torch

import long_context_attention_attn_amd as la
from gpu_util import banner, dev
from long_context_attention_attn_amd import synth

pytestmark = pytest.mark.gpu

T, H = 300, 4
DTYPES = [torch.bfloat16, torch.float32]


def _prefill(q, k, v, decay, cu=None):
    d = dev()
    out, fs = la.prefill(q.to(d), k.to(d), v.to(d), decay.to(d), None if cu is None else cu.to(d))
    torch.cuda.synchronize()
    return out.cpu(), fs.cpu()


def _inputs(dtype, D):
    q, k, v = synth.qkv(T, H, D, dtype, seed=21)
    return q, k, v, synth.decay_geometric(H, 0.9, 0.999)


@pytest.mark.parametrize("bad", [float("nan"), float("inf")], ids=["nan", "inf"])
@pytest.mark.parametrize("dtype", DTYPES, ids=["bf16", "f32"])
@pytest.mark.parametrize("D", [64, 128])
def test_nonfinite_q_reaches_only_its_row(dtype, D, bad):
    """A non-finite q at token 150 (inside block 2) changes only row 150's output."""
    banner("nonfinite q dtype=%s D=%d" % (dtype, D))
    q, k, v, decay = _inputs(dtype, D)
    o0, s0 = _prefill(q, k, v, decay)
    qb = q.clone()
    qb[150, :, 3] = bad
    o1, s1 = _prefill(qb, k, v, decay)
    assert torch.isfinite(o0).all()
    assert torch.equal(o1[:150], o0[:150]) and torch.equal(o1[151:], o0[151:])
    assert not torch.isfinite(o1[150]).all()
    assert torch.equal(s1, s0)  # q never enters the state


@pytest.mark.parametrize("dtype", DTYPES, ids=["bf16", "f32"])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("t", [150, 128, 191], ids=["mid", "first", "last"])
def test_nonfinite_k_never_reaches_earlier_rows(dtype, D, t):
    """A NaN k at token t leaves every row before t bit-identical (its future scores are
    selected away, not multiplied by zero), including the earlier rows of t's own block."""
    banner("nonfinite k dtype=%s D=%d t=%d" % (dtype, D, t))
    q, k, v, decay = _inputs(dtype, D)
    o0, _ = _prefill(q, k, v, decay)
    kb = k.clone()
    kb[t, :, 5] = float("nan")
    o1, s1 = _prefill(q, kb, v, decay)
    assert torch.equal(o1[:t], o0[:t])
    assert not torch.isfinite(o1[t:]).all()
    assert not torch.isfinite(s1).all()


# bf16: the intra product contracts 32 keys per matrix instruction; fp32: 16-key tiles.
GROUP = {torch.bfloat16: 32, torch.float32: 16}


@pytest.mark.parametrize("bad", [float("nan"), float("inf")], ids=["nan", "inf"])
@pytest.mark.parametrize("dtype", DTYPES, ids=["bf16", "f32"])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("t", [180, 129, 255], ids=["mid", "second", "last"])
def test_nonfinite_v_stays_in_its_operand_group(dtype, D, t, bad):
    """A non-finite v at token t never reaches a row before its operand group inside the block
    (so never an earlier block)."""
    banner("nonfinite v dtype=%s D=%d t=%d" % (dtype, D, t))
    q, k, v, decay = _inputs(dtype, D)
    o0, _ = _prefill(q, k, v, decay)
    vb = v.clone()
    vb[t, :, 7] = bad
    o1, _ = _prefill(q, k, vb, decay)
    g0 = t // GROUP[dtype] * GROUP[dtype]
    assert g0 // 64 == t // 64
    assert torch.equal(o1[:g0], o0[:g0])
    assert not torch.isfinite(o1[t:]).all()


@pytest.mark.parametrize("dtype", DTYPES, ids=["bf16", "f32"])
def test_nonfinite_token_stays_in_its_sequence(dtype):
    """Packed sequences [0, 100), [100, 230), [230, 300): NaN q, k and v at token 150 of the
    middle sequence leave the other sequences' outputs and final states bit-identical and the
    middle sequence's rows before its operand group too."""
    banner("nonfinite packed dtype=%s" % dtype)
    D = 128
    q, k, v, decay = _inputs(dtype, D)
    cu = synth.cu_from_lengths([100, 130, 70])
    o0, s0 = _prefill(q, k, v, decay, cu)
    qb, kb, vb = q.clone(), k.clone(), v.clone()
    qb[150], kb[150], vb[150] = float("nan"), float("nan"), float("nan")
    o1, s1 = _prefill(qb, kb, vb, decay, cu)
    assert torch.equal(o1[:100], o0[:100]) and torch.equal(o1[230:], o0[230:])
    assert torch.equal(s1[0], s0[0]) and torch.equal(s1[2], s0[2])
    # token 150 is local token 50 of the middle sequence: group start 32 (bf16) or 48 (fp32)
    g0 = 100 + 50 // GROUP[dtype] * GROUP[dtype]
    assert torch.equal(o1[100:g0], o0[100:g0])
    assert not torch.isfinite(s1[1]).all()
