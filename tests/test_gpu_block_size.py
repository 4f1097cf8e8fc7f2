"""Block-size invariance on the GPU: the split into blocks (intra-block left product, inter-block
right product through the running state) is exact algebra for any block size B, so the 64- and
128-token kernels must each match the oracle to the bf16 tolerance and agree with each other to
rounding.  Cases span ragged and empty sequences, partial last blocks on either side of 64 and
128, lambda = 0 and 1, an initial state, both head sizes, and a 65,536-token run against the
recurrent form."""
import numpy as np
import pytest
import torch

import long_context_attention_attn_amd as la
import oracle
from gpu_util import BF16_TOL, banner, dev, rel, slice_errors, state_errors, to_np
from long_context_attention_attn_amd import synth

pytestmark = pytest.mark.gpu

LENGTHS = [1, 127, 128, 129, 0, 300, 64, 200, 7, 256]


def _prefill(q, k, v, decay, cu=None, init=None, block_size=0):
    d = dev()
    out, fs = la.prefill(q.to(d), k.to(d), v.to(d), decay.to(d), None if cu is None else cu.to(d),
                         initial_state=None if init is None else init.to(d), block_size=block_size)
    torch.cuda.synchronize()
    return out.cpu(), fs.cpu()


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("with_init", [False, True], ids=["zero_state", "init_state"])
def test_block_sizes_match_oracle_and_each_other(D, with_init):
    banner("block size invariance D=%d init=%s" % (D, with_init))
    H = 4
    cu = synth.cu_from_lengths(LENGTHS)
    q, k, v = synth.qkv(int(cu[-1]), H, D, torch.bfloat16, seed=41)
    decay = torch.tensor([0.0, 0.9, 0.999, 1.0], dtype=torch.float32)
    init = synth.random_state(len(LENGTHS), H, D, seed=42, scale=0.1) if with_init else None
    ref = oracle.quadratic(q, k, v, decay, cu, init_state=init)
    ref_s = oracle.final_state(k, v, decay, cu, init_state=init)
    res = {}
    for B in (64, 128):
        out, fs = _prefill(q, k, v, decay, cu, init, block_size=B)
        e = slice_errors(to_np(out), ref, cu).max()
        es = state_errors(to_np(fs), ref_s).max()
        print("B=%d: out %.2e state %.2e" % (B, e, es))
        assert e <= BF16_TOL and es <= BF16_TOL
        res[B] = (to_np(out), to_np(fs))
    # the two block sizes round different intermediate products to bf16, nothing else
    assert slice_errors(res[128][0], res[64][0], cu).max() <= BF16_TOL
    assert state_errors(res[128][1], res[64][1]).max() <= BF16_TOL


def test_default_block_is_128_for_bf16_bitwise():
    banner("default block size")
    cu = synth.cu_from_lengths([300, 65])
    q, k, v = synth.qkv(365, 2, 128, torch.bfloat16, seed=43)
    decay = synth.decay_geometric(2, 0.9, 0.999)
    o0, s0 = _prefill(q, k, v, decay, cu)
    o1, s1 = _prefill(q, k, v, decay, cu, block_size=128)
    o2, _ = _prefill(q, k, v, decay, cu, block_size=64)
    assert torch.equal(o0, o1) and torch.equal(s0, s1)
    assert not torch.equal(o0, o2)  # the 64-token kernel rounds differently


def test_block128_deterministic_and_causal():
    """Bitwise run-to-run determinism, and tokens from t0 = 190 on (inside a 128-token block)
    replaced by other finite values leave every earlier output bit-identical."""
    banner("block 128 determinism and causality")
    T, H, D, t0 = 400, 4, 128, 190
    q, k, v = synth.qkv(T, H, D, torch.bfloat16, seed=44)
    q2, k2, v2 = synth.qkv(T, H, D, torch.bfloat16, seed=45)
    decay = synth.decay_geometric(H, 0.9, 0.999)
    o1, s1 = _prefill(q, k, v, decay, block_size=128)
    o2, s2 = _prefill(q, k, v, decay, block_size=128)
    assert torch.equal(o1, o2) and torch.equal(s1, s2)
    qa, ka, va = q.clone(), k.clone(), v.clone()
    qa[t0:], ka[t0:], va[t0:] = q2[t0:], k2[t0:], v2[t0:]
    o3, _ = _prefill(qa, ka, va, decay, block_size=128)
    assert torch.equal(o1[:t0], o3[:t0]) and not torch.equal(o1[t0:], o3[t0:])


@pytest.mark.parametrize("t", [180, 129, 255], ids=["mid", "second", "last"])
def test_block128_nonfinite_v_stays_in_its_operand_group(t):
    """The finite-input contract at B = 128: a NaN v reaches no row before its 32-token operand
    group; NaN q and k reach no earlier row at all."""
    banner("block 128 nonfinite t=%d" % t)
    T, H, D = 300, 4, 128
    q, k, v = synth.qkv(T, H, D, torch.bfloat16, seed=46)
    decay = synth.decay_geometric(H, 0.9, 0.999)
    o0, _ = _prefill(q, k, v, decay, block_size=128)
    g0 = t // 32 * 32
    vb = v.clone()
    vb[t, :, 7] = float("nan")
    o1, _ = _prefill(q, k, vb, decay, block_size=128)
    assert torch.equal(o1[:g0], o0[:g0]) and not torch.isfinite(o1[t:]).all()
    kb, qb = k.clone(), q.clone()
    kb[t, :, 3] = float("nan")
    qb[t, :, 3] = float("nan")
    o2, _ = _prefill(qb, kb, v, decay, block_size=128)
    assert torch.equal(o2[:t], o0[:t]) and not torch.isfinite(o2[t]).all()


def test_block128_65k_tokens_against_recurrent_form():
    """65,536 tokens x 8 heads (lambda geometric 0.9 -> 0.9999) at both block sizes against the
    oracle's recurrent form on every head."""
    banner("block 128 65536 x 8")
    T, H, D = 65536, 8, 128
    q, k, v = synth.qkv(T, H, D, torch.bfloat16, seed=0)
    decay = synth.decay_geometric(H, 0.9, 0.9999)
    ref, ref_s = oracle.recurrent(q, k, v, decay)
    outs = {}
    for B in (64, 128):
        out, fs = _prefill(q, k, v, decay, block_size=B)
        e = slice_errors(to_np(out), ref, [0, T]).max()
        es = state_errors(to_np(fs), ref_s).max()
        print("B=%d: out %.2e state %.2e" % (B, e, es))
        assert e <= BF16_TOL and es <= BF16_TOL
        outs[B] = to_np(out)
    assert max(rel(outs[128][:, h], outs[64][:, h]) for h in range(H)) <= BF16_TOL
