"""Host-side checks of bench.py's contract (no GPU): the one-GPU guard and the algorithmic
FLOP and byte counts the reported rates divide by."""
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=60)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_prefill_flop_per_token_head():
    # 4 B d + 4 d^2 at B = 64, d = 128: 32,768 + 65,536 = 98,304 FLOP per token-head
    assert bench.prefill_flop(1, 1, 128) == 98304
    assert bench.prefill_flop(65536, 64, 128) == 65536 * 64 * 98304 == 412316860416
    # d = 64: 4*64*64 + 4*64*64
    assert bench.prefill_flop(1, 1, 64) == 32768


def test_prefill_bytes():
    # bf16 q, k, v read + out written = 1,024 B per token-head at d = 128, plus the fp32 final
    # state (64 KiB per head) and the decay vector
    assert bench.prefill_bytes(1, 1, 128, S=0) == 1024 + 4
    assert bench.prefill_bytes(65536, 64, 128) == 65536 * 64 * 1024 + 64 * 65536 + 64 * 4


def test_decode_bytes():
    # fp32 state read + write, bf16 q, k, v, o, fp32 decay: 2,164,261,120 B at 256 x 64 x 128
    assert bench.decode_bytes(256, 64, 128) == 2164261120


def test_unknown_extra_leg_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--extras", "nope"],
                       capture_output=True, text=True, timeout=60)
    assert r.returncode == 2
    assert "unknown extra leg" in r.stderr and "fp32_prefill" in r.stderr
