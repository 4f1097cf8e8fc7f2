"""Host-side checks of the C ABI (no GPU needed, no kernel launched).

* the shared library loads and exports every function include/lightning_attn.h declares;
* argument validation returns the documented status codes before any HIP call;
* on a machine without a GPU, a well-formed call reports LA_ERR_HIP (no device).
"""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "lightning_attn.h")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(la_[a-z_0-9]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    from long_context_attention_attn_amd import _lib

    if not os.path.exists(_lib.library_path()):
        from long_context_attention_attn_amd import build

        build.build()
    return _lib.load()


def test_exports_every_declared_symbol(lib):
    from long_context_attention_attn_amd import _lib

    declared = _declared_functions()
    assert set(declared) == set(_lib.EXPORTS), declared
    for name in declared:
        assert hasattr(lib, name), "missing export %s" % name


def test_version_and_status_strings(lib):
    assert lib.la_abi_version() == 2
    assert lib.la_status_str(0) == b"LA_OK"
    assert lib.la_status_str(1) == b"LA_ERR_INVALID_ARG"
    assert lib.la_status_str(2) == b"LA_ERR_UNSUPPORTED"
    assert lib.la_status_str(3) == b"LA_ERR_HIP"
    assert lib.la_status_str(99) == b"LA_ERR_UNKNOWN"


# Fake, never-dereferenced 16-byte aligned "device" addresses for validation-only calls.
P = ctypes.c_void_p(0x100000)
P2 = ctypes.c_void_p(0x200000)
MISALIGNED = ctypes.c_void_p(0x100008)
OUT = ctypes.c_void_p(0x700000)


def _prefill(lib, q=P, k=P, v=P, decay=P, cu=None, out=P2, fs=None, T=64, S=1, H=2, D=128,
             dt=1, init=None):
    return lib.la_prefill_ex(q, k, v, decay, cu, init, out, fs, T, S, H, D, dt, None)


@pytest.mark.parametrize("kwargs,status", [
    (dict(D=96), 2), (dict(D=32), 2), (dict(dt=7), 2),
    (dict(H=0), 1), (dict(T=-1), 1), (dict(S=0), 1), (dict(S=2), 1),  # S=2 without cu_seqlens
    (dict(q=None), 1), (dict(out=None), 1), (dict(decay=None), 1),
    (dict(q=MISALIGNED), 1), (dict(init=P2, fs=P2), 1),
    # byte-range overlaps: q, k, v are 64 x 2 x 128 bf16 = 32 KiB, states 2 x 64 KiB
    (dict(out=ctypes.c_void_p(0x100000 + 0x7ff0)), 1), (dict(v=ctypes.c_void_p(0x200000 - 0x10)), 1),
    (dict(fs=ctypes.c_void_p(0x204000)), 1), (dict(init=ctypes.c_void_p(0x200010)), 1),
    (dict(init=ctypes.c_void_p(0x300000), fs=ctypes.c_void_p(0x310000)), 1),
    # decay ([H] fp32) or cu_seqlens ([S+1] int32) inside a written buffer
    (dict(decay=ctypes.c_void_p(0x200000 + 0x100)), 1),
    (dict(cu=ctypes.c_void_p(0x700000 + 0x40), fs=ctypes.c_void_p(0x700000)), 1),
    (dict(decay=ctypes.c_void_p(0x700000 + 0x8), fs=ctypes.c_void_p(0x700000)), 1),
])
def test_prefill_validation(lib, kwargs, status):
    assert _prefill(lib, **kwargs) == status
    assert lib.la_last_error() != b""


def test_read_only_buffers_may_share_memory(lib):
    import torch

    if torch.cuda.is_available():
        pytest.skip("a GPU is visible")
    # q, k, v, decay and the initial state all read: overlapping them is no hazard, so
    # validation passes and the device check (no GPU here) reports the HIP error.
    assert _prefill(lib, init=ctypes.c_void_p(0x100010), decay=ctypes.c_void_p(0x100020)) == 3


def test_prefill_empty_is_noop(lib):
    # T = 0 and no final state requested: nothing to do, no HIP call.
    assert _prefill(lib, q=None, k=None, v=None, out=None, T=0) == 0


@pytest.mark.parametrize("kwargs,status", [
    (dict(D=100), 2), (dict(H=0), 1), (dict(Bt=-3), 1), (dict(state=None), 1),
    (dict(state=MISALIGNED), 1), (dict(q=None), 1),
])
def test_decode_validation(lib, kwargs, status):
    a = dict(q=P, k=P, v=P, decay=P, state=P2, out=OUT, Bt=4, H=2, D=128, dt=1)
    a.update(kwargs)
    rc = lib.la_decode_step(a["q"], a["k"], a["v"], a["decay"], a["state"], a["out"], a["Bt"],
                            a["H"], a["D"], a["dt"], None)
    assert rc == status


def test_decode_zero_batch_is_noop(lib):
    assert lib.la_decode_step(None, None, None, P, None, None, 0, 2, 128, 1, None) == 0


def test_no_device_reports_hip_error(lib):
    import torch

    if torch.cuda.is_available():
        pytest.skip("a GPU is visible")
    # Well-formed arguments: validation passes, the device check fails.
    assert _prefill(lib) == 3
    assert b"hip" in lib.la_last_error().lower()


def test_binding_rejects_cpu_tensors():
    import torch

    import long_context_attention_attn_amd as la

    q = torch.zeros(8, 1, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        la.prefill(q, q, q.to(torch.float32), torch.ones(1))


def _split(lib, seg_blocks=4, ws=ctypes.c_void_p(0x300000), ws_bytes=1 << 30, T=1000, S=1, H=2,
           D=128, cu=None, init=None, fs=None, q=P):
    return lib.la_prefill_split(q, P, P, P, cu, init, P2, fs, T, S, H, D, 1, seg_blocks, ws,
                                ws_bytes, None)


@pytest.mark.parametrize("kwargs", [
    dict(seg_blocks=0), dict(seg_blocks=-2), dict(ws=None), dict(ws=ctypes.c_void_p(0x300010)),
    dict(ws_bytes=1000), dict(T=1 << 31), dict(S=0), dict(S=3), dict(init=P2, fs=P2),
    dict(q=None),
])
def test_split_validation(lib, kwargs):
    assert _split(lib, **kwargs) == 1
    assert lib.la_last_error() != b""


def test_split_workspace_size(lib):
    def expect(T, S, H, D, nb, sub=1):
        a = lambda x: (x + 255) // 256 * 256
        cap = -(-T // (64 * nb)) + S - 1 if T > 0 else 0
        return a(cap * sub * H * D * D * 4) + a((cap + 1) * 4) + a((S + 1) * 4) + a(cap * 4)

    for args in [(8192, 1, 8, 128, 16), (1000, 3, 2, 64, 1), (1, 1, 1, 128, 7), (0, 2, 4, 64, 2),
                 (272568, 16, 64, 128, 64), (65536, 1, 16, 128, 256)]:
        assert lib.la_prefill_split_workspace_size(*args) == expect(*args), args
    # sub-segment states of the bf16 two-launch form: one sequence in two segments, 64 heads x 2
    # slices at d = 64 (128 workgroups; 512 fit one round) -> 4 sub-segments of 8,192 tokens;
    # 32 heads x 4 slices at d = 128 (256 fit) -> 2; segments of 4,096 tokens over one head -> 2
    # (sub-segments keep 2,048 tokens); 16,384 tokens in 8,192-token segments -> 4; no more
    # segments than sequences (perhaps none cut) -> 1
    for args, sub in [((65536, 1, 64, 64, 512), 4), ((65536, 1, 32, 128, 512), 2),
                      ((8192, 1, 1, 128, 64), 2), ((16384, 1, 2, 64, 128), 4),
                      ((65536, 1, 32, 64, 256), 2), ((15288, 3, 2, 128, 64), 2),
                      ((18225, 5, 2, 128, 64), 1)]:
        assert lib.la_prefill_split_workspace_size(*args) == expect(*args, sub=sub), args
    assert lib.la_prefill_split_workspace_size(100, 1, 1, 96, 4) == 0
    assert lib.la_prefill_split_workspace_size(100, 1, 1, 128, 0) == 0


def test_split_without_device(lib):
    import torch

    if torch.cuda.is_available():
        pytest.skip("a GPU is visible")
    assert lib.la_prefill_split_blocks(8192, 1, 8, 128, 1) == 0
    assert _split(lib) == 3


G1, G2, G3 = ctypes.c_void_p(0x400000), ctypes.c_void_p(0x500000), ctypes.c_void_p(0x600000)


def _backward(lib, dq=G1, dk=G2, dv=G3, d_out=P2, dinit=None, init=None, dfs=None, T=64, S=1,
              D=128, q=P, decay=P):
    return lib.la_backward(q, P, P, decay, None, init, d_out, dfs, dq, dk, dv, dinit, T, S, 2, D,
                           1, None)


@pytest.mark.parametrize("kwargs,status", [
    (dict(dq=None), 1), (dict(dv=None), 1), (dict(d_out=None), 1),
    (dict(dk=ctypes.c_void_p(0x500004)), 1), (dict(dq=P), 1), (dict(dk=P2), 1),
    (dict(dv=G1), 1), (dict(dinit=P2, init=P2), 1), (dict(dinit=G1, dfs=G1), 1),
    (dict(S=0), 1), (dict(D=80), 2),
])
def test_backward_validation(lib, kwargs, status):
    assert _backward(lib, **kwargs) == status
    assert lib.la_last_error() != b""


def test_backward_empty_without_state_grad_is_noop(lib):
    assert _backward(lib, q=None, d_out=None, dq=None, dk=None, dv=None, T=0) == 0


def test_backward_without_device(lib):
    import torch

    if torch.cuda.is_available():
        pytest.skip("a GPU is visible")
    assert _backward(lib) == 3


@pytest.mark.parametrize("kwargs,status", [
    (dict(m=0), 1), (dict(m=-1), 1), (dict(Bt=-1), 1), (dict(state=None), 1),
    (dict(state=MISALIGNED), 1), (dict(D=100), 2), (dict(q=None), 1),
])
def test_decode_tokens_validation(lib, kwargs, status):
    a = dict(q=P, k=P, v=P, decay=P, state=P2, out=OUT, Bt=4, m=3, H=2, D=128, dt=1)
    a.update(kwargs)
    rc = lib.la_decode_tokens(a["q"], a["k"], a["v"], a["decay"], a["state"], a["out"], a["Bt"],
                              a["m"], a["H"], a["D"], a["dt"], None)
    assert rc == status


def test_adjacent_buffers_are_not_overlaps(lib):
    import torch

    if torch.cuda.is_available():
        pytest.skip("a GPU is visible")
    # out starts right after q ends; states back to back: validation passes, the device check
    # (no GPU here) reports the HIP error.
    end = 0x100000 + 64 * 2 * 128 * 2
    assert _prefill(lib, out=ctypes.c_void_p(end), init=ctypes.c_void_p(0x300000),
                    fs=ctypes.c_void_p(0x300000 + 2 * 128 * 128 * 4)) == 3
    rc = lib.la_decode_step(P, P, P, P, P2, ctypes.c_void_p(0x100000 + 4 * 2 * 128 * 2), 4, 2,
                            128, 1, None)
    assert rc == 3


@pytest.mark.parametrize("kwargs", [
    dict(out=ctypes.c_void_p(0x100100)), dict(state=ctypes.c_void_p(0x700000)),
    dict(state=ctypes.c_void_p(0x100000 - 0x10)),
    # decay inside the state (read while other workgroups update it) or inside out
    dict(decay=ctypes.c_void_p(0x200000 + 0x1000)), dict(decay=ctypes.c_void_p(0x700000 + 0x10)),
])
def test_decode_overlap_rejected(lib, kwargs):
    a = dict(q=P, k=P, v=P, decay=P, state=P2, out=OUT)
    a.update(kwargs)
    assert lib.la_decode_step(a["q"], a["k"], a["v"], a["decay"], a["state"], a["out"], 4, 2, 128,
                              1, None) == 1
    assert b"overlap" in lib.la_last_error()
    assert lib.la_decode_tokens(a["q"], a["k"], a["v"], a["decay"], a["state"], a["out"], 4, 3, 2,
                                128, 1, None) == 1


S1, S2 = ctypes.c_void_p(0x900000), ctypes.c_void_p(0xa00000)  # state-sized (2 x 64 KiB)


@pytest.mark.parametrize("kwargs", [
    dict(dq=ctypes.c_void_p(0x200000 + 0x4000)), dict(dv=ctypes.c_void_p(0x500000 + 0x7f00)),
    dict(dk=ctypes.c_void_p(0x100000 + 0x10)),
    # d_initial_state against every activation and gradient buffer
    dict(dinit=ctypes.c_void_p(0x400000 + 0x100)), dict(dinit=ctypes.c_void_p(0x500000)),
    dict(dinit=ctypes.c_void_p(0x600000 + 0x10)), dict(dinit=ctypes.c_void_p(0x100000)),
    dict(dinit=ctypes.c_void_p(0x200000 + 0x40)),
    # the state inputs inside a gradient buffer
    dict(init=ctypes.c_void_p(0x400000), dinit=S1), dict(dfs=ctypes.c_void_p(0x600000), dinit=S1),
    dict(init=ctypes.c_void_p(0x500000 + 0x100)), dict(dfs=ctypes.c_void_p(0x400000 + 0x7000)),
    # decay inside a written buffer
    dict(decay=ctypes.c_void_p(0x400000 + 0x20)), dict(decay=ctypes.c_void_p(0x900000 + 0x20),
                                                       dinit=S1),
])
def test_backward_overlap_rejected(lib, kwargs):
    assert _backward(lib, **kwargs) == 1
    assert b"overlap" in lib.la_last_error()


@pytest.mark.parametrize("ws", [0x100000, 0x200000 - 0x100, 0x700000])
def test_split_workspace_overlap_rejected(lib, ws):
    # a workspace that overlaps q (at P), out (at P2) or the final states (at 0x700000)
    assert _split(lib, ws=ctypes.c_void_p(ws), fs=ctypes.c_void_p(0x700000)) == 1
    assert b"overlap" in lib.la_last_error()


def _backward_split(lib, seg_blocks=4, ws=ctypes.c_void_p(0x800000), ws_bytes=1 << 30, T=1000,
                    dq=G1, q=P, D=128):
    return lib.la_backward_split(q, P, P, P, None, None, P2, None, dq, G2, G3, None, T, 1, 2, D,
                                 1, seg_blocks, ws, ws_bytes, None)


@pytest.mark.parametrize("kwargs,status", [
    (dict(seg_blocks=0), 1), (dict(ws=None), 1), (dict(ws=ctypes.c_void_p(0x800010)), 1),
    (dict(ws_bytes=4096), 1), (dict(T=1 << 31), 1), (dict(dq=None), 1), (dict(D=80), 2),
    # workspace over dq (at 0x400000) or over q (at 0x100000)
    (dict(ws=ctypes.c_void_p(0x400000)), 1), (dict(ws=ctypes.c_void_p(0x100000)), 1),
])
def test_backward_split_validation(lib, kwargs, status):
    assert _backward_split(lib, **kwargs) == status
    assert lib.la_last_error() != b""


def test_backward_split_without_device(lib):
    import torch

    if torch.cuda.is_available():
        pytest.skip("a GPU is visible")
    assert _backward_split(lib) == 3


# Plain-vs-split choices timed on one MI355X (256 CUs), 20 calls of each path after warm-up,
# one sequence, the suggested segment length: (dtype, D, H, T, split wins).  Only cases where one
# path beat the other by 10% or more are pins; closer ones may go either way.  Examples, plain
# against split in us: bf16 D = 128 H = 1: T = 1024 17.8 / 23.7, T = 2048 29.4 / 25.5; H = 32
# T = 65536 945 / 857.  bf16 D = 64: H = 64 T = 65536 931 / 788; H = 32 T = 2048 22.4 / 27.8.
# fp32 D = 128: H = 1 T = 1024 73.8 / 47.2; H = 32 T = 16384 1128 / 967.  fp32 D = 64: H = 64
# T = 1024 48.8 / 56.4.
SPLIT_MEASURED = [
    (1, 128, 1, 512, False), (1, 128, 1, 1024, False), (1, 128, 1, 2048, True),
    (1, 128, 1, 4096, True), (1, 128, 1, 16384, True), (1, 128, 1, 65536, True),
    (1, 128, 8, 512, False), (1, 128, 8, 1024, False), (1, 128, 8, 4096, True),
    (1, 128, 8, 16384, True), (1, 128, 8, 65536, True), (1, 128, 32, 512, False),
    (1, 128, 32, 1024, False), (1, 128, 32, 2048, False), (1, 128, 32, 65536, True),
    (0, 128, 1, 512, False), (0, 128, 1, 1024, True), (0, 128, 1, 2048, True),
    (0, 128, 1, 4096, True), (0, 128, 1, 16384, True), (0, 128, 1, 65536, True),
    (0, 128, 8, 512, False), (0, 128, 8, 1024, True), (0, 128, 8, 2048, True),
    (0, 128, 8, 4096, True), (0, 128, 8, 16384, True), (0, 128, 8, 65536, True),
    (0, 128, 32, 512, False), (0, 128, 32, 16384, True), (0, 64, 1, 512, False),
    (0, 64, 1, 1024, True), (0, 64, 1, 2048, True), (0, 64, 1, 4096, True),
    (0, 64, 1, 16384, True), (0, 64, 1, 65536, True), (0, 64, 8, 512, False),
    (0, 64, 8, 1024, True), (0, 64, 8, 2048, True), (0, 64, 8, 4096, True),
    (0, 64, 8, 16384, True), (0, 64, 8, 65536, True), (0, 64, 32, 512, False),
    (0, 64, 32, 1024, True), (0, 64, 32, 2048, True), (0, 64, 32, 4096, True),
    (0, 64, 32, 16384, True), (0, 64, 64, 512, False), (0, 64, 64, 1024, False),
    (1, 64, 1, 512, False), (1, 64, 1, 1024, False), (1, 64, 1, 4096, True),
    (1, 64, 1, 16384, True), (1, 64, 1, 65536, True), (1, 64, 8, 512, False),
    (1, 64, 8, 1024, False), (1, 64, 8, 4096, True), (1, 64, 8, 16384, True),
    (1, 64, 8, 65536, True), (1, 64, 32, 512, False), (1, 64, 32, 1024, False),
    (1, 64, 32, 2048, False), (1, 64, 32, 4096, True), (1, 64, 32, 16384, True),
    (1, 64, 32, 65536, True), (1, 64, 64, 512, False), (1, 64, 64, 1024, False),
    (1, 64, 64, 2048, False), (1, 64, 64, 4096, False), (1, 64, 64, 16384, True),
    (1, 64, 64, 65536, True),
]


# Several sequences (S equal lengths of T / S tokens), timed the same way: (dtype, D, H, S, T,
# split wins).  fp32 D = 64 one head, 8 x 1,024 tokens: plain 47.0 us / split 35.5; fp32
# D = 128 74.3 / 48.7; bf16 D = 128 17.9 / 25.1; bf16 D = 64 13.8 / 22.4; bf16 D = 64
# H = 4, 4 x 8,192: 76.6 / 41.1; fp32 D = 128 H = 8, 2 x 32,768: 2234 / 971; bf16 D = 128
# H = 16, 2 x 8,192 (two segments per sequence, the last one's state not computed): 103.3 / 91.4.
SPLIT_MEASURED_BATCHED = [
    (0, 64, 1, 8, 8192, True), (0, 128, 1, 8, 8192, True), (1, 128, 1, 8, 8192, False),
    (1, 64, 1, 8, 8192, False), (1, 64, 4, 4, 32768, True), (0, 128, 8, 2, 65536, True),
    (1, 128, 16, 2, 16384, True),
]


@pytest.mark.parametrize("dtype,D,H,T,split", SPLIT_MEASURED)
def test_split_suggestion_matches_measured_choice(lib, dtype, D, H, T, split):
    seg = lib.la_prefill_split_blocks_for(T, 1, H, D, dtype, 256)
    assert (seg > 0) == split, (dtype, D, H, T, seg)


@pytest.mark.parametrize("dtype,D,H,S,T,split", SPLIT_MEASURED_BATCHED)
def test_split_suggestion_matches_measured_choice_batched(lib, dtype, D, H, S, T, split):
    seg = lib.la_prefill_split_blocks_for(T, S, H, D, dtype, 256)
    assert (seg > 0) == split, (dtype, D, H, S, T, seg)


def test_split_suggestion_rules(lib):
    f = lib.la_prefill_split_blocks_for
    # the plain launch already fills 256 CUs: 64 heads x 4 slices, or 2 x 32 heads
    assert f(65536, 1, 64, 128, 1, 256) == 0
    assert f(65536, 2, 32, 128, 1, 256) == 0
    # few chains over a long sequence: about one segment workgroup per CU
    assert f(65536, 1, 8, 128, 1, 256) == 128
    assert f(65536, 1, 8, 64, 1, 256) == 64
    # at least 4 blocks per segment, never a segment covering the whole sequence
    assert f(16384, 1, 1, 128, 1, 256) == 4
    assert f(256, 1, 1, 128, 1, 256) == 0
    # invalid sizes, dtype or device size
    for args in ((0, 1, 8, 128, 1, 256), (4096, 0, 8, 128, 1, 256), (4096, 1, 0, 128, 1, 256),
                 (4096, 1, 8, 96, 1, 256), (4096, 1, 8, 128, 7, 256), (4096, 1, 8, 128, 1, 0)):
        assert f(*args) == 0, args


FAR_IN, FAR_OUT = ctypes.c_void_p(0x10000000), ctypes.c_void_p(0x40000000)  # 768 MiB apart


def _split_static(lib, T=1000, seg_blocks=4, H=2, D=128, S=1, cu=None, q=FAR_IN, dt=1):
    return lib.la_prefill_split_static(q, FAR_IN, FAR_IN, P, cu, None, FAR_OUT, None, T, S, H, D,
                                       dt, seg_blocks, None)


@pytest.mark.parametrize("kwargs,status", [
    (dict(seg_blocks=0), 1), (dict(T=1 << 31), 1), (dict(q=None), 1), (dict(D=80), 2),
    (dict(dt=9), 2), (dict(S=2), 1),
    # 65,536 tokens x 8 heads in 1-block segments: 1,024 x 8 x 64 KiB of segment states, far
    # beyond the 32 MiB static scratch
    (dict(T=65536, H=8, seg_blocks=1), 1),
])
def test_split_static_validation(lib, kwargs, status):
    assert _split_static(lib, **kwargs) == status
    assert lib.la_last_error() != b""
    if kwargs.get("T") == 65536:
        assert b"static scratch" in lib.la_last_error()


def test_split_static_limit(lib):
    from long_context_attention_attn_amd import _lib

    # the largest single-sequence 8-head D=128 split that fits: its workspace is at most the
    # scratch; one more segment does not fit and is rejected before any HIP call
    cap = _lib.SPLIT_STATIC_SCRATCH_BYTES
    assert cap == 32 << 20
    fits = lib.la_prefill_split_workspace_size(64 * 60, 1, 8, 128, 1)
    over = lib.la_prefill_split_workspace_size(64 * 70, 1, 8, 128, 1)
    assert fits <= cap < over
    assert _split_static(lib, T=64 * 70, H=8, seg_blocks=1) == 1
    assert b"static scratch" in lib.la_last_error()


def test_split_static_falls_back_to_one_state_per_segment(lib):
    """8 sequences of ~36,864 tokens x 16 heads in 32,768-token segments (two per sequence):
    the bf16 two-launch form would keep 2 sub-segment states per segment (32 MiB of states, past
    the scratch); the static call keeps one per segment (16 MiB) instead, so without a device it
    gets past the size check and fails only at the device check."""
    import torch

    if torch.cuda.is_available():
        pytest.skip("a GPU is visible")
    from long_context_attention_attn_amd import _lib

    T, S, H, D, nb = 294912, 8, 16, 128, 512
    assert lib.la_prefill_split_workspace_size(T, S, H, D, nb) > _lib.SPLIT_STATIC_SCRATCH_BYTES
    GiB = 1 << 30
    q, k, v = (ctypes.c_void_p(x * GiB) for x in (16, 20, 24))  # 2.4 GB each at fp32
    out, cu = ctypes.c_void_p(28 * GiB), ctypes.c_void_p(32 * GiB)
    st = lib.la_prefill_split_static(q, k, v, P, cu, None, out, None, T, S, H, D, 1, nb, None)
    assert st == 3, lib.la_last_error()
    # fp32 storage has no sub-segment states: the same sizes fit as they are
    assert lib.la_prefill_split_static(q, k, v, P, cu, None, out, None, T, S, H, D, 0, nb,
                                       None) == 3


def test_split_static_without_device(lib):
    import torch

    if torch.cuda.is_available():
        pytest.skip("a GPU is visible")
    assert _split_static(lib) == 3


def _prefill_bs(lib, block_size, dt=1):
    return lib.la_prefill_with_block_size(P, P, P, P, None, None, P2, None, 64, 1, 2, 128, dt,
                                          block_size, None)


@pytest.mark.parametrize("block_size,dt,status", [
    (32, 1, 1), (256, 1, 1), (-1, 1, 1), (96, 1, 1),  # only 0, 64 and 128
    (128, 0, 2),                                        # 128-token blocks: bf16 only
])
def test_block_size_validation(lib, block_size, dt, status):
    assert _prefill_bs(lib, block_size, dt) == status
    assert lib.la_last_error() != b""


def test_block_size_without_device(lib):
    import torch

    if torch.cuda.is_available():
        pytest.skip("a GPU is visible")
    for bs, dt in ((0, 1), (64, 1), (128, 1), (0, 0), (64, 0)):
        assert _prefill_bs(lib, bs, dt) == 3, (bs, dt)


@pytest.mark.parametrize("env,dt,status", [
    ("96", 1, 1), ("abc", 1, 1),  # an invalid LA_BLOCK fails bf16 calls that use the default
    ("96", 0, 3),                 # fp32 has one block size and ignores LA_BLOCK
    ("128", 1, 3), ("64", 1, 3), ("", 1, 3),
])
def test_la_block_environment(env, dt, status):
    """LA_BLOCK sets the default block size of bf16 prefills (read once per process, so each
    case runs in a child process; no GPU here, so valid calls end at the device check)."""
    import subprocess
    import sys

    import torch

    if torch.cuda.is_available():
        pytest.skip("a GPU is visible")
    script = ("import sys, ctypes; sys.path.insert(0, %r)\n"
              "from long_context_attention_attn_amd import _lib\n"
              "lib = _lib.load(); P = ctypes.c_void_p(0x100000); O = ctypes.c_void_p(0x200000)\n"
              "print(lib.la_prefill(P, P, P, P, None, O, None, 64, 1, 2, 128, %d, None))\n"
              % (ROOT, dt))
    r = subprocess.run([sys.executable, "-c", script], capture_output=True, text=True,
                       env=dict(os.environ, LA_BLOCK=env), timeout=120)
    assert r.returncode == 0, r.stderr
    assert int(r.stdout.strip().splitlines()[-1]) == status
