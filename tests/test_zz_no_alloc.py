"""The allocation-free split prefill (la_prefill_split_static, segment states in the library's
static device scratch) against la_prefill_split with a caller workspace: two calls in a row
through the C ABI, the second with a smaller input (the scratch keeps the first call's
contents), each bit-identical to the workspace form, which shares its kernels and arithmetic,
and within the bf16/fp32 tolerance of the oracle."""
import pytest
import torch

import long_context_attention_attn_amd as la
import oracle
from gpu_util import BF16_TOL, F32_TOL, banner, dev, slice_errors, state_errors, to_np
from long_context_attention_attn_amd import _lib, synth

pytestmark = pytest.mark.gpu

CASES = [
    # (lengths, H, D, dtype, seg_blocks): the second is smaller than the first in tokens,
    # heads, segments and workspace bytes
    ([1000, 1, 1999], 8, 128, torch.bfloat16, 4),
    ([300, 129], 3, 64, torch.float32, 2),
]


def _run(lengths, H, D, dtype, seg, static):
    d = dev()
    cu = synth.cu_from_lengths(lengths)
    T = int(cu[-1])
    q, k, v = synth.qkv(T, H, D, dtype, seed=31)
    decay = synth.decay_geometric(H, 0.9, 0.999)
    init = synth.random_state(len(lengths), H, D, seed=32, scale=0.1)
    out, fs = la.prefill(q.to(d), k.to(d), v.to(d), decay.to(d), cu.to(d),
                         initial_state=init.to(d), split=seg, static_scratch=static)
    torch.cuda.synchronize()
    return (q, k, v, decay, cu, init), out.cpu(), fs.cpu()


def test_static_scratch_matches_workspace_twice():
    sizes = [_lib.prefill_split_workspace_size(sum(l), len(l), H, D, seg)
             for l, H, D, _, seg in CASES]
    assert sizes[0] > sizes[1] and sizes[0] <= _lib.SPLIT_STATIC_SCRATCH_BYTES
    for lengths, H, D, dtype, seg in CASES:
        banner("static split lengths=%s H=%d D=%d %s seg=%d" % (lengths, H, D, dtype, seg))
        inputs, o_ref, s_ref = _run(lengths, H, D, dtype, seg, static=False)
        _, o, s = _run(lengths, H, D, dtype, seg, static=True)
        assert torch.equal(o, o_ref) and torch.equal(s, s_ref)
        q, k, v, decay, cu, init = inputs
        tol = BF16_TOL if dtype == torch.bfloat16 else F32_TOL
        ref = oracle.quadratic(q, k, v, decay, cu, init_state=init)
        ref_s = oracle.final_state(k, v, decay, cu, init_state=init)
        assert slice_errors(to_np(o), ref, cu).max() <= tol
        assert state_errors(to_np(s), ref_s).max() <= tol


def test_static_scratch_rejects_oversize():
    banner("static split oversize")
    d = dev()
    T, H, D = 64 * 70, 8, 128  # 1-block segments need 35 MiB of segment states
    q = torch.zeros((T, H, D), dtype=torch.bfloat16, device=d)
    decay = torch.full((H,), 0.9, device=d)
    with pytest.raises(_lib.LightningAttnError, match="static scratch"):
        la.prefill(q, q, q, decay, split=1, static_scratch=True)
