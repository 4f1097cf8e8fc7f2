"""GPU parity of the multi-token decode step (m tokens per sequence, state read once) against
the fp64 oracle's recurrent form over m-token sequences from the given states, and against m
single-token decode steps."""
import numpy as np
import pytest
import torch

import long_context_attention_attn_amd as la
import oracle
from gpu_util import BF16_TOL, F32_TOL, banner, dev, slice_errors, state_errors, to_np
from long_context_attention_attn_amd import synth

pytestmark = pytest.mark.gpu

TOL = {torch.bfloat16: BF16_TOL, torch.float32: F32_TOL}


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "f32"])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("m", [1, 3, 8, 11, 20])
def test_decode_tokens_vs_oracle(dtype, D, m):
    banner("decode_tokens dtype=%s D=%d m=%d" % (dtype, D, m))
    Bt, H = 5, 4
    q, k, v = synth.qkv(Bt * m, H, D, dtype, seed=80 + m)
    decay = torch.tensor([0.0, 0.5, 0.99, 1.0], dtype=torch.float32)
    st0 = synth.random_state(Bt, H, D, seed=81, scale=0.3)
    st = st0.to(dev())
    d = dev()
    out = la.decode_tokens(q.view(Bt, m, H, D).to(d), k.view(Bt, m, H, D).to(d),
                           v.view(Bt, m, H, D).to(d), decay.to(d), st)
    torch.cuda.synchronize()
    cu = torch.arange(0, Bt * m + 1, m, dtype=torch.int32)
    ref, ref_s = oracle.recurrent(q, k, v, decay, cu, init_state=st0)
    e = slice_errors(to_np(out.view(Bt * m, H, D)), ref, cu)
    es = state_errors(to_np(st), ref_s)
    print("decode_tokens: out %.2e state %.2e" % (e.max(), es.max()))
    assert e.max() <= TOL[dtype]
    assert es.max() <= 1e-6  # fp32 state: m fused multiply-adds per element


def test_decode_tokens_equals_single_steps():
    """One 6-token pass equals six decode_step calls (bf16, D=128), within rounding."""
    banner("decode_tokens vs 6 decode steps")
    Bt, m, H, D = 16, 6, 8, 128
    d = dev()
    q, k, v = synth.qkv(Bt * m, H, D, torch.bfloat16, seed=90, device=d)
    decay = synth.decay_geometric(H, 0.9, 0.9999).to(d)
    st0 = synth.random_state(Bt, H, D, seed=91, device=d, scale=0.1)
    sa, sb = st0.clone(), st0.clone()
    out = la.decode_tokens(q.view(Bt, m, H, D), k.view(Bt, m, H, D), v.view(Bt, m, H, D), decay,
                           sa)
    q4, k4, v4 = (x.view(Bt, m, H, D) for x in (q, k, v))
    outs = [la.decode_step(q4[:, i].contiguous(), k4[:, i].contiguous(), v4[:, i].contiguous(),
                           decay, sb) for i in range(m)]
    torch.cuda.synchronize()
    ref = torch.stack(outs, dim=1)
    e = slice_errors(to_np(out.view(Bt * m, H, D)), to_np(ref.view(Bt * m, H, D)),
                     list(range(0, Bt * m + 1, m)))
    assert e.max() <= BF16_TOL
    assert float((sa - sb).abs().max() / sb.abs().max()) <= 1e-6
