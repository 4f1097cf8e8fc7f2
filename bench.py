#!/usr/bin/env python3
"""Benchmark of the lightning-attention hot path on one MI355X.

One step = the whole hot path on one batch of synthetic input:
  * prefill of one MiniMax-like layer: 64 heads x 65,536 tokens, head dim 128, bf16 storage,
    lambda_h geometric 0.9 -> 0.9999 (outputs + final fp32 states), then
  * one decode step for 256 sequences x 64 heads with fp32 128x128 states.
Inputs are resident in HBM before the timed region.  The timed region holds exactly K steps
bracketed by device synchronisation; per-kernel durations come from HIP events recorded on
the stream the kernels run on.

`value` is prefill tokens/s (65,536 tokens over the prefill's own time from HIP events); the
whole step's rate is step_tokens_per_s.  Prints ONE JSON line with the roofline of the dominant
kernel (prefill: achieved from this run's HIP events, and the committed rocprofv3 trace's
figure beside it) and the fp64 CPU oracle timed on a bounded sample of the same workload
(--no-cpu-baseline skips it).  Extra legs, timed after the K steps (--no-extras skips them):
the packed 16-sequence and the 1,048,576-token prefills at 64 heads; few-chain prefill and
backward, plain and sequence-split; the 64-head backward; multi-token decode; the fp32-storage
prefill; and ceilings re-measured on the device (copy bandwidth, library GEMM rates).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "prefill tokens/s + TFLOP/s (% bf16 MFMA peak) H=64 d=128; decode GB/s"
HBM_PEAK_GBPS = 8000.0         # MI355X HBM3E, published
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA, published

T_PREFILL, H, D = 65536, 64, 128
BT_DECODE = 256
BLOCK_FLOP_B = 64              # FLOP accounting at block size 64, whatever the kernel's B
KERNEL_BLOCK = 128             # the bf16 prefill's block size (the library default)
PREFILL_KERNEL = "prefill_bf16_b128_kernel<128, false, false>"
# sources the committed profiles of that kernel were taken with
PREFILL_SOURCES = ("long_context_attention_attn_amd/csrc/prefill_bf16_b128.hip",
                   "long_context_attention_attn_amd/csrc/bf16_tiles.h")


EXTRA_LEGS = ("varlen_prefill", "long_prefill", "few_chain_prefill", "backward",
              "few_chain_backward", "decode_tokens", "fp32_prefill", "measured_peaks")


def prefill_flop(T, H, D, B=BLOCK_FLOP_B):
    # per token-head: intra 4*B*D (QK^T and PV over full BxB tiles) + inter 2*D^2 + state 2*D^2
    return T * H * (4 * B * D + 4 * D * D)


def prefill_bytes(T, H, D, S=1):
    # read q, k, v and write out (bf16) + write the fp32 final state
    return T * H * D * 2 * 4 + S * H * D * D * 4 + H * 4


def decode_bytes(Bt, H, D):
    # state read + write (fp32), q, k, v read and out write (bf16), decay
    return 2 * Bt * H * D * D * 4 + 4 * Bt * H * D * 2 + H * 4


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the extra legs timed after the K steps")
    ap.add_argument("--extras", default=",".join(EXTRA_LEGS),
                    help="comma-separated extra legs to run (default: all of %s)"
                         % ", ".join(EXTRA_LEGS))
    ap.add_argument("--cpu-sample-tokens", type=int, default=65536)
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="instead of the benchmark, time a plain device-to-device copy of this "
                         "many MiB (K times); used to calibrate HBM byte counters")
    args = ap.parse_args()
    chosen = [x for x in args.extras.split(",") if x]
    for name in chosen:
        if name not in EXTRA_LEGS:
            print("unknown extra leg %r (known: %s)" % (name, ", ".join(EXTRA_LEGS)),
                  file=sys.stderr)
            sys.exit(2)
    if args.gpus != 1:
        print("bench.py measures one GPU only: the hot path runs on a single MI355X and there "
              "is no multi-GPU path (heads and sequences would shard with no communication).  "
              "Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch

    import long_context_attention_attn_amd as la
    from long_context_attention_attn_amd import synth

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.copy_probe_mib:
        copy_probe(args.copy_probe_mib, args.steps, args.warmup)
        return
    wl = synth.workloads()["prefill_64k"]
    assert (wl.T, wl.H, wl.D) == (T_PREFILL, H, D)
    q, k, v = wl.inputs(device=dev)
    decay = wl.decay().to(dev)
    out = torch.empty_like(q)
    fs = torch.empty((1, H, D, D), dtype=torch.float32, device=dev)
    qd, kd, vd = synth.decode_batch(BT_DECODE, H, D, torch.bfloat16, seed=2, device=dev)
    st = synth.random_state(BT_DECODE, H, D, seed=1, device=dev, scale=0.1)
    od = torch.empty_like(qd)
    torch.cuda.synchronize()

    def step(evs=None):
        if evs is not None:
            evs[0].record()
        la.prefill(q, k, v, decay, out=out, final_state=fs)
        if evs is not None:
            evs[1].record()
        la.decode_step(qd, kd, vd, decay, st, out=od)
        if evs is not None:
            evs[2].record()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    K = args.steps
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(K)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(K):
        step(events[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    pre_ms = [e[0].elapsed_time(e[1]) for e in events]
    dec_ms = [e[1].elapsed_time(e[2]) for e in events]
    pre_avg = sum(pre_ms) / K
    dec_avg = sum(dec_ms) / K
    ms_per_step = wall * 1e3 / K

    tokens_per_step = T_PREFILL + BT_DECODE
    # The metric is prefill tokens/s: prefill tokens over the prefill kernel's own time (HIP
    # events on its stream).  The whole step's rate (prefill and decode tokens over the step's
    # wall time) is reported beside it as step_tokens_per_s.
    value = T_PREFILL / (pre_avg / 1e3)
    pf = prefill_flop(T_PREFILL, H, D)
    pb = prefill_bytes(T_PREFILL, H, D)
    db = decode_bytes(BT_DECODE, H, D)
    pre_tflops = pf / (pre_avg / 1e3) / 1e12
    pre_gbps = pb / (pre_avg / 1e3) / 1e9
    dec_gbps = db / (dec_avg / 1e3) / 1e9

    result = {
        "metric": METRIC,
        "value": value,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "step_tokens_per_s": tokens_per_step / (ms_per_step / 1e3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": "lightning prefill 1 x 65536 tokens x 64 heads x d128 bf16 "
                        "(lambda 0.9->0.9999, final fp32 states) + decode step 256 seqs x 64 "
                        "heads fp32 128x128 states",
            "prefill_tokens": T_PREFILL, "heads": H, "head_dim": D, "block": KERNEL_BLOCK,
            "decode_batch": BT_DECODE,
        },
        "prefill": {
            "ms": pre_avg, "ms_min": min(pre_ms),
            "tokens_per_s": T_PREFILL / (pre_avg / 1e3),
            "tflops": pre_tflops, "pct_bf16_mfma_peak": 100.0 * pre_tflops / BF16_PEAK_TFLOPS,
            # the FLOP the kernel itself issues at its own block size (intra 4 B d grows with B)
            "kernel_block": KERNEL_BLOCK,
            "kernel_flop_per_launch": prefill_flop(T_PREFILL, H, D, KERNEL_BLOCK),
            "kernel_block_tflops": prefill_flop(T_PREFILL, H, D, KERNEL_BLOCK) / (pre_avg / 1e3) / 1e12,
            "algorithmic_GBps": pre_gbps,
            "flop_per_launch": pf, "bytes_per_launch": pb,
        },
        "decode": {
            "ms": dec_avg, "ms_min": min(dec_ms), "GBps": dec_gbps,
            "pct_hbm_peak": 100.0 * dec_gbps / HBM_PEAK_GBPS, "bytes_per_launch": db,
        },
        "roofline": {
            "bound": "hbm", "kernel": PREFILL_KERNEL,
            "achieved": pre_gbps, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
            "frac": pre_gbps / HBM_PEAK_GBPS, "traffic": measured_traffic(),
            "achieved_source": "HIP events around the prefill launches of this run",
            "trace": committed_trace(pb),
        },
    }

    if not args.no_extras:
        del q, k, v, out
        legs = {
            "varlen_prefill": lambda: long_prefill_leg("varlen_16", dev),
            "long_prefill": lambda: long_prefill_leg("prefill_1m", dev),
            "few_chain_prefill": lambda: few_chain_prefill(dev),
            "backward": lambda: backward_leg(wl, dev),
            "few_chain_backward": lambda: few_chain_backward(dev),
            "decode_tokens": lambda: decode_tokens_leg(dev),
            "fp32_prefill": lambda: fp32_prefill_leg(dev),
            "measured_peaks": lambda: measured_peaks(dev),
        }
        for name in EXTRA_LEGS:
            if name in chosen:
                result[name] = legs[name]()
    if not args.no_cpu_baseline:
        q, k, v = wl.inputs(device=dev)
        result["cpu_baseline"] = cpu_baseline(q, k, v, wl, args.cpu_sample_tokens, tokens_per_step)
    print(json.dumps(result), flush=True)


def time_ms(fn, iters, warmup):
    """Average milliseconds per call from HIP events on the current stream (the library's
    kernels run on it)."""
    import torch

    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(iters):
        fn()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / iters


def backward_bytes(T, H, D, S=1):
    # read q, k, v, d_out and write dq, dk, dv (bf16) + write d_initial_state (fp32)
    return T * H * D * 2 * 7 + S * H * D * D * 4 + H * 4


def backward_leg(wl, dev, iters=10, warmup=2):
    """Backward of the 65,536 x 64 prefill (dq, dk, dv and the initial-state gradient), timed
    outside the timed steps."""
    import torch

    import long_context_attention_attn_amd as la
    from long_context_attention_attn_amd import synth

    q, k, v = wl.inputs(device=dev)
    do, _, _ = synth.qkv(wl.T, wl.H, wl.D, torch.bfloat16, seed=50, device=dev)
    dec = wl.decay().to(dev)
    ms = time_ms(lambda: la.backward(q, k, v, dec, do), iters, warmup)
    nbytes = backward_bytes(wl.T, wl.H, wl.D)
    # three scans: each reads three [T, H, D] tensors and writes one
    scan_bytes = 3 * prefill_bytes(wl.T, wl.H, wl.D)
    return {"tokens": wl.T, "heads": wl.H, "ms": ms, "tokens_per_s": wl.T / (ms / 1e3),
            "algorithmic_bytes": nbytes, "algorithmic_GBps": nbytes / (ms / 1e3) / 1e9,
            "scan_bytes": scan_bytes, "scan_GBps": scan_bytes / (ms / 1e3) / 1e9,
            "flop": 3 * prefill_flop(wl.T, wl.H, wl.D),
            "tflops": 3 * prefill_flop(wl.T, wl.H, wl.D) / (ms / 1e3) / 1e12}


def decode_tokens_leg(dev, iters=20, warmup=3):
    """m decode steps per sequence in one pass (state read and written once) for 256 sequences
    x 64 heads; m = 1 is the single-step kernel."""
    import torch

    import long_context_attention_attn_amd as la
    from long_context_attention_attn_amd import synth

    dec = synth.decay_geometric(H, 0.9, 0.9999).to(dev)
    st = synth.random_state(BT_DECODE, H, D, seed=1, device=dev, scale=0.1)
    res = []
    for m in (1, 2, 4, 8):
        q, k, v = synth.qkv(BT_DECODE * m, H, D, torch.bfloat16, seed=2, device=dev)
        if m == 1:
            fn = lambda: la.decode_step(q, k, v, dec, st)
        else:
            shp = (BT_DECODE, m, H, D)
            q4, k4, v4 = q.view(shp), k.view(shp), v.view(shp)
            fn = lambda: la.decode_tokens(q4, k4, v4, dec, st)
        ms = time_ms(fn, iters, warmup)
        nbytes = 2 * BT_DECODE * H * D * D * 4 + 4 * BT_DECODE * m * H * D * 2 + H * 4
        res.append({"m": m, "ms": ms, "tokens_per_s": BT_DECODE * m / (ms / 1e3),
                    "GBps": nbytes / (ms / 1e3) / 1e9, "bytes": nbytes})
    return res


def few_chain_prefill(dev, iters=20, warmup=3):
    """Prefill shapes with fewer (sequence, head, 32-column slice) chains than compute units --
    8,192 x 8 heads, 65,536 x 8 heads and 65,536 x 32 heads (one device's share of the 64-head
    layer under 8-way and 2-way head sharding) at d = 128, and the 64-head layer at d = 64 (two
    slices per head: 128 chains) -- timed with the plain scan and with the sequence split the
    library suggests."""
    import torch

    import long_context_attention_attn_amd as la
    from long_context_attention_attn_amd import _lib, synth

    res = []
    for T, Hc, Dh in ((8192, 8, D), (65536, 8, D), (65536, 32, D), (65536, 64, 64)):
        q, k, v = synth.qkv(T, Hc, Dh, torch.bfloat16, seed=0, device=dev)
        dec = synth.decay_geometric(Hc, 0.9, 0.9999).to(dev)
        o = torch.empty_like(q)
        f = torch.empty((1, Hc, Dh, Dh), dtype=torch.float32, device=dev)
        seg = _lib.prefill_split_blocks(T, 1, Hc, Dh, _lib.LA_BF16)
        plain = time_ms(lambda: la.prefill(q, k, v, dec, out=o, final_state=f), iters, warmup)
        split = time_ms(lambda: la.prefill(q, k, v, dec, out=o, final_state=f, split=seg or None),
                        iters, warmup)
        nbytes = prefill_bytes(T, Hc, Dh)
        res.append({"tokens": T, "heads": Hc, "head_dim": Dh, "seg_blocks": seg,
                    "plain_ms": plain, "split_ms": split, "speedup": plain / split,
                    "split_algorithmic_GBps": nbytes / (split / 1e3) / 1e9,
                    "split_hbm_frac": nbytes / (split / 1e3) / 1e9 / HBM_PEAK_GBPS,
                    "split_tokens_per_s": T / (split / 1e3)})
        del q, k, v, o
    return res


def few_chain_backward(dev, iters=10, warmup=2):
    """Backward of 65,536 tokens x 8 heads (one device's share of the 64-head layer under
    8-way head sharding): the three gradient scans plain and sequence-split."""
    import torch

    import long_context_attention_attn_amd as la
    from long_context_attention_attn_amd import _lib, synth

    T, Hc = 65536, 8
    q, k, v = synth.qkv(T, Hc, D, torch.bfloat16, seed=0, device=dev)
    do, _, _ = synth.qkv(T, Hc, D, torch.bfloat16, seed=50, device=dev)
    dec = synth.decay_geometric(Hc, 0.9, 0.9999).to(dev)
    seg = _lib.prefill_split_blocks(T, 1, Hc, D, _lib.LA_BF16)
    plain = time_ms(lambda: la.backward(q, k, v, dec, do), iters, warmup)
    split = time_ms(lambda: la.backward(q, k, v, dec, do, split=seg or None), iters, warmup)
    nbytes = backward_bytes(T, Hc, D)
    return {"tokens": T, "heads": Hc, "seg_blocks": seg, "plain_ms": plain, "split_ms": split,
            "speedup": plain / split, "split_algorithmic_GBps": nbytes / (split / 1e3) / 1e9,
            "split_tokens_per_s": T / (split / 1e3)}


def long_prefill_leg(name, dev, iters=5, warmup=2):
    """The other full-size prefill workloads at 64 heads x d128 bf16, timed with HIP events:
    16 packed sequences of 1,024-32,768 tokens (T = 272,568, state reset at every boundary) and
    one 1,048,576-token sequence.  Tokens/s, TFLOP/s at B = 64 accounting and algorithmic
    HBM GB/s against the 8 TB/s peak."""
    import torch

    import long_context_attention_attn_amd as la
    from long_context_attention_attn_amd import synth

    wl = synth.workloads()[name]
    q, k, v = wl.inputs(device=dev)
    decay = wl.decay().to(dev)
    cu = wl.cu_seqlens().to(dev) if wl.S > 1 else None
    out = torch.empty_like(q)
    fs = torch.empty((wl.S, wl.H, wl.D, wl.D), dtype=torch.float32, device=dev)
    ms = time_ms(lambda: la.prefill(q, k, v, decay, cu, out=out, final_state=fs), iters, warmup)
    del q, k, v, out, fs
    torch.cuda.empty_cache()
    nbytes = prefill_bytes(wl.T, wl.H, wl.D, wl.S)
    flop = prefill_flop(wl.T, wl.H, wl.D)
    gbps = nbytes / (ms / 1e3) / 1e9
    return {"workload": wl.note, "tokens": wl.T, "sequences": wl.S, "heads": wl.H, "ms": ms,
            "tokens_per_s": wl.T / (ms / 1e3), "tflops": flop / (ms / 1e3) / 1e12,
            "pct_bf16_mfma_peak": 100.0 * flop / (ms / 1e3) / 1e12 / BF16_PEAK_TFLOPS,
            "algorithmic_bytes": nbytes, "algorithmic_GBps": gbps,
            "hbm_frac": gbps / HBM_PEAK_GBPS}


def sources_sha256(paths):
    """sha256 over the concatenated bytes of the given repository files."""
    import hashlib

    h = hashlib.sha256()
    for p in paths:
        h.update(open(os.path.join(ROOT, p), "rb").read())
    return h.hexdigest()


def committed_trace(nbytes):
    """The prefill kernel's average duration in the committed rocprofv3 kernel trace
    (profiles/prefill_kernel_trace.json) with the fraction of the HBM roofline it gives and the
    shader clock the counter run measured; None when the kernel source changed since."""
    path = os.path.join(ROOT, "profiles", "prefill_kernel_trace.json")
    try:
        doc = json.load(open(path))
        sha = sources_sha256(doc["kernel_sources"])
    except (OSError, ValueError, KeyError, TypeError):
        return None
    if sha != doc.get("kernel_sources_sha256") or doc.get("kernel") != PREFILL_KERNEL:
        return None
    us = doc["avg_us"]
    gbps = nbytes / (us / 1e6) / 1e9
    return {"source": doc.get("summary"), "avg_us": us, "achieved": gbps,
            "frac": gbps / HBM_PEAK_GBPS, "shader_clock_mhz": doc.get("shader_clock_mhz")}


def measured_traffic():
    """HBM bytes per prefill launch from the committed counter runs (profiles/traffic.json),
    or None when the kernel source has changed since those counters were taken."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        doc = json.load(open(path))
        sha = sources_sha256(doc["kernel_sources"])
    except (OSError, ValueError, KeyError, TypeError):
        return None
    if sha != doc.get("kernel_sources_sha256") or doc.get("kernel") != PREFILL_KERNEL:
        return None
    return doc.get("traffic_bytes_per_launch")


def fp32_prefill_leg(dev, iters=5, warmup=2):
    """The fp32-storage prefill (fp32 matrix instructions) at 65,536 tokens x 64 heads x d128,
    against the 157.3 TFLOP/s fp32 matrix peak at B = 64 accounting."""
    import torch
    import long_context_attention_attn_amd as la
    from long_context_attention_attn_amd import synth

    T, H, D = T_PREFILL, 64, 128
    q, k, v = synth.qkv(T, H, D, torch.float32, seed=0, device=dev)
    decay = synth.decay_geometric(H, 0.9, 0.9999).to(dev)
    out = torch.empty_like(q)
    fs = torch.empty((1, H, D, D), dtype=torch.float32, device=dev)
    ms = time_ms(lambda: la.prefill(q, k, v, decay, out=out, final_state=fs), iters, warmup)
    tf = prefill_flop(T, H, D) / (ms / 1e3) / 1e12
    return {"workload": "prefill 1 x %d tokens x %d heads x d%d fp32" % (T, H, D), "ms": ms,
            "tokens_per_s": T / (ms / 1e3), "tflops": tf, "pct_fp32_matrix_peak": 100.0 * tf / 157.3}


def measured_peaks(dev):
    """Ceilings re-measured on this device beside the published ones: copies of 2 GiB (HBM
    read + write) by device memcpy and by an elementwise kernel, and large square library GEMMs
    (dense MFMA) in bf16 and in fp32: achievable rather than theoretical peaks."""
    import torch

    n = 1 << 31
    src = torch.ones(n // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    ms = time_ms(lambda: dst.copy_(src), 10, 2)  # device-to-device memcpy (blit kernel)
    ms_e = time_ms(lambda: torch.mul(src, 1.0, out=dst), 10, 2)  # elementwise read + write
    res = {"hbm_memcpy_GBps": 2 * n / (ms / 1e3) / 1e9,
           "hbm_elementwise_copy_GBps": 2 * n / (ms_e / 1e3) / 1e9,
           "hbm_spec_GBps": HBM_PEAK_GBPS}
    del src, dst
    m = 8192
    for dt, name in ((torch.bfloat16, "bf16"), (torch.float32, "fp32")):
        a = torch.randn(m, m, device=dev, dtype=dt)
        b = torch.randn(m, m, device=dev, dtype=dt)
        ms = time_ms(lambda: torch.mm(a, b), 10, 3)
        res[name + "_gemm_%d_TFLOPs" % m] = 2.0 * m ** 3 / (ms / 1e3) / 1e12
        del a, b
    res["bf16_spec_TFLOPs"] = BF16_PEAK_TFLOPS
    res["fp32_matrix_spec_TFLOPs"] = 157.3
    return res


def copy_probe(mib, steps, warmup):
    """A plain copy of `mib` MiB between two device buffers (read mib, write mib)."""
    import torch

    n = mib * (1 << 20)
    src = torch.ones(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(warmup):
        dst.copy_(src)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    print(json.dumps({"copy_probe_bytes_read": n, "copy_probe_bytes_written": n,
                      "ms": ms, "GBps": 2 * n / (ms / 1e3) / 1e9}), flush=True)


def cpu_baseline(q, k, v, wl, n_tok, tokens_per_step):
    """The fp64 oracle on the host cores for one step of the same workload: its recurrent form
    (O2) on the first n_tok tokens of the prefill input (all 64 heads), scaled to the 65,536
    tokens, plus its decode step (O4) on all 256 x 64 states of the decode shape (synthetic
    values: the timing does not depend on them).  value = tokens per step / oracle seconds per
    step, the GPU value's unit.  fp64 FLOP counted as 5 d^2 per token-head (decay, rank-1 update
    and q S)."""
    import torch

    import oracle
    from long_context_attention_attn_amd import synth
    from oracle import _f64  # noqa: PLC0415

    o = oracle.default()
    decay = wl.decay()
    dec64 = decay.double().numpy()
    # Inputs converted outside the timed regions (the oracle consumes fp64).
    qf, kf, vf = (_f64(x[:n_tok].cpu()) for x in (q, k, v))
    qd, kd, vd = (_f64(x) for x in synth.decode_batch(BT_DECODE, H, D, torch.bfloat16, seed=2))
    st = _f64(synth.random_state(BT_DECODE, H, D, seed=1, scale=0.1))
    threads = o.num_threads()
    t0 = time.perf_counter()
    o.recurrent(qf, kf, vf, dec64)
    dt_pre = time.perf_counter() - t0
    t0 = time.perf_counter()
    o.decode_step(qd, kd, vd, dec64, st)
    dt_dec = time.perf_counter() - t0
    step_s = dt_pre * (T_PREFILL / n_tok) + dt_dec
    flop_tok = 5 * D * D
    # One thread on 4 heads of the same prefill tokens (1/16 of the work), scaled to 64 heads.
    heads1 = 4
    o.set_num_threads(1)
    t1 = time.perf_counter()
    o.recurrent(qf[:, :heads1], kf[:, :heads1], vf[:, :heads1], dec64[:heads1])
    dt1 = (time.perf_counter() - t1) * (H / heads1)
    o.set_num_threads(threads)
    return {
        "value": tokens_per_step / step_s, "unit": "tokens/s", "cores": threads, "kind": "oracle",
        "sample": "fp64 recurrent form on the first %d of %d prefill tokens (all %d heads, "
                  "%.1f s, scaled to the full prefill) + fp64 decode step on %d x %d states "
                  "(%.2f s)" % (n_tok, T_PREFILL, H, dt_pre, BT_DECODE, H, dt_dec),
        "seconds_per_step": step_s,
        "prefill_tokens_per_s": n_tok / dt_pre,
        "prefill_fp64_gflops": n_tok * H * flop_tok / dt_pre / 1e9,
        "decode_ms": dt_dec * 1e3,
        "decode_fp64_gflops": BT_DECODE * H * flop_tok / dt_dec / 1e9,
        "single_thread": {"value": n_tok / dt1, "unit": "prefill tokens/s", "cores": 1,
                          "sample": "same tokens, heads 0-3, scaled x16 to 64 heads"},
        "cpu_model": _cpu_model(),
    }


def _cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


if __name__ == "__main__":
    main()
