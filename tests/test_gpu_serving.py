"""GPU checks of the serving helpers: one captured HIP graph of a padded prefill shape replayed
for several different batches, each replay compared bit for bit with the eager prefill of the
unpadded batch (sequences are independent, so padding must not change any real output), with
eager work and synchronisation between the replays; one replay also against the oracle."""
import pytest
import torch

import long_context_attention_attn_amd as la
import oracle
from gpu_util import BF16_TOL, banner, dev, slice_errors, state_errors, to_np
from long_context_attention_attn_amd import serving, synth

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("with_init", [False, True], ids=["zero_state", "init_state"])
def test_graphed_prefill_replays(with_init):
    banner("graphed prefill replays init=%s" % with_init)
    H, D = 4, 128
    tl, sl = serving.multilevel(1 << 14), [1, 2, 4, 8, 16]
    T_pad, _, _ = serving.padded_batch([700, 200, 60], tl, sl)  # 960 tokens
    S_pad = serving.pad_to_level(6, sl)  # up to 7 real sequences and the filler
    gp = serving.GraphedPrefill(T_pad, S_pad, H, D, with_initial_state=with_init)
    d = dev()
    decay = synth.decay_geometric(H, 0.9, 0.999).to(d)
    batches = [[100, 0, 300], [1, 63, 64, 65, 500], [T_pad - 1], [100, 0, 300]]
    for it, lengths in enumerate(batches):
        T = sum(lengths)
        q, k, v = synth.qkv(T, H, D, torch.bfloat16, seed=100 + it, device=d)
        init = (synth.random_state(len(lengths), H, D, seed=200 + it, device=d, scale=0.1)
                if with_init else None)
        out_g, fs_g = gp(q, k, v, decay, lengths, initial_state=init)
        out_g, fs_g = out_g.clone(), fs_g.clone()
        cu = synth.cu_from_lengths(lengths).to(d)
        out_e, fs_e = la.prefill(q, k, v, decay, cu, initial_state=init)  # eager, in between
        torch.cuda.synchronize()
        assert torch.equal(out_g, out_e), "replay %d out" % it
        assert torch.equal(fs_g, fs_e), "replay %d final state" % it
        if it == 1:
            qc, kc, vc = q.cpu(), k.cpu(), v.cpu()
            ref = oracle.quadratic(qc, kc, vc, decay.cpu(), cu.cpu(),
                                   init_state=None if init is None else init.cpu())
            assert slice_errors(to_np(out_g), ref, cu.cpu()).max() <= BF16_TOL
            ref_s = oracle.final_state(kc, vc, decay.cpu(), cu.cpu(),
                                       init_state=None if init is None else init.cpu())
            assert state_errors(to_np(fs_g), ref_s).max() <= BF16_TOL
    with pytest.raises(ValueError):
        q, k, v = synth.qkv(T_pad + 1, H, D, torch.bfloat16, seed=1, device=d)
        gp(q, k, v, decay, [T_pad + 1])


def test_graphed_split_static_scratch_replays():
    """A few-chain split prefill (4 heads, 1,024-token segments) captured with its segment states
    in the library's static scratch, so the captured launches allocate nothing, replayed for four
    batches with eager work and synchronisation between the replays.  Every replay equals, bit
    for bit, the eager static-scratch split of the same padded batch run right after it, and
    matches the recurrent oracle."""
    banner("graphed split static scratch")
    H, D, seg = 4, 128, 16
    T_pad, S_pad = 8192, 4
    gp = serving.GraphedPrefill(T_pad, S_pad, H, D, with_initial_state=True, split=seg,
                                static_scratch=True)
    d = dev()
    decay = synth.decay_geometric(H, 0.9, 0.999).to(d)
    batches = [[8000], [3000, 0, 4100], [1, 1023, 1025], [8000]]
    for it, lengths in enumerate(batches):
        T = sum(lengths)
        q, k, v = synth.qkv(T, H, D, torch.bfloat16, seed=300 + it, device=d)
        init = synth.random_state(len(lengths), H, D, seed=400 + it, device=d, scale=0.1)
        out_g, fs_g = gp(q, k, v, decay, lengths, initial_state=init)
        out_g, fs_g = out_g.clone(), fs_g.clone()
        # the same padded batch, eager, through the same static scratch
        out_e, fs_e = la.prefill(gp.q, gp.k, gp.v, gp.decay, gp.cu, initial_state=gp.init,
                                 split=seg, static_scratch=True)
        torch.cuda.synchronize()
        assert torch.equal(out_g, out_e[:T]), "replay %d out" % it
        assert torch.equal(fs_g, fs_e[:len(lengths)]), "replay %d final state" % it
        cu = synth.cu_from_lengths(lengths)
        ref, ref_s = oracle.recurrent(q.cpu(), k.cpu(), v.cpu(), decay.cpu(), cu,
                                      init_state=init.cpu())
        assert slice_errors(to_np(out_g), ref, cu).max() <= BF16_TOL, "replay %d" % it
        assert state_errors(to_np(fs_g), ref_s).max() <= BF16_TOL, "replay %d state" % it
