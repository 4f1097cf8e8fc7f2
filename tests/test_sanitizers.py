"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only, no device code
instrumented).

* The oracle (plain C) built by gcc with -fsanitize=address,undefined runs every pin.
* A private copy of the oracle with a planted out-of-bounds read is caught (the instrumentation
  is live, not silently absent).
* The C-ABI library is built by hipcc with the sanitizers on its host code only (each flag
  behind -Xarch_host; the gfx950 kernels are compiled as usual) and runs the ABI host tests:
  every validation path, status string and overlap rule.

Each run is a child Python process with the sanitizer runtime preloaded (the interpreter is
not instrumented); leak detection is off because the interpreter itself never frees its
arenas.
"""
import glob
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
TESTS = os.path.join(ROOT, "tests")
ORACLE_SRC = os.path.join(ROOT, "oracle", "la_oracle.c")
CSRC = os.path.join(ROOT, "long_context_attention_attn_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ENV = {"ASAN_OPTIONS": "detect_leaks=0:abort_on_error=0",
       "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1"}


def _gcc_runtime():
    r = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True)
    path = r.stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


def _clang_runtime():
    found = glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so")
    return found[0] if found else None


def _child(script, runtime, *args):
    env = dict(os.environ, LD_PRELOAD=runtime, **ENV)
    return subprocess.run([sys.executable, "-c", script] + list(args), capture_output=True,
                          text=True, env=env, timeout=600)


def _build_oracle(src, out):
    subprocess.run(["gcc", "-O1", "-g", "-std=c11", "-fPIC", "-shared", "-fopenmp",
                    "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
                    "-fno-omit-frame-pointer", "-I", os.path.dirname(ORACLE_SRC), "-o", out, src],
                   check=True)


PINS = """
import sys
sys.path[:0] = [%r, %r]
import oracle, oracle_pins
o = oracle.Oracle(sys.argv[1])
for pin in oracle_pins.ALL_PINS:
    pin(o)
print("pins ok", len(oracle_pins.ALL_PINS))
""" % (ROOT, TESTS)


@pytest.fixture(scope="module")
def gcc_asan():
    rt = _gcc_runtime()
    if rt is None or shutil.which("gcc") is None:
        pytest.skip("gcc's AddressSanitizer runtime is not installed")
    return rt


def test_oracle_pins_under_asan_ubsan(tmp_path, gcc_asan):
    lib = str(tmp_path / "liblaoracle_san.so")
    _build_oracle(ORACLE_SRC, lib)
    r = _child(PINS, gcc_asan, lib)
    assert r.returncode == 0, r.stderr[-4000:]
    assert "pins ok" in r.stdout
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr


def test_planted_overflow_is_caught(tmp_path, gcc_asan):
    src = open(ORACLE_SRC).read()
    good = "for (int32_t a = 0; a < D; ++a) acc += qt[a] * St[(size_t)a * D + c];"
    assert src.count(good) == 1
    bad = tmp_path / "la_oracle_oob.c"
    bad.write_text(src.replace(good, good.replace("a < D", "a <= D")))
    lib = str(tmp_path / "liblaoracle_oob.so")
    _build_oracle(str(bad), lib)
    script = """
import sys
sys.path[:0] = [%r]
import numpy as np
import oracle
o = oracle.Oracle(sys.argv[1])
x = np.ones((2, 3, 8))
o.decode_step(x, x, x, np.full(3, 0.5), np.zeros((2, 3, 8, 8)))
print("not caught")
""" % ROOT
    r = _child(script, gcc_asan, lib)
    assert r.returncode != 0 and "heap-buffer-overflow" in r.stderr, r.stderr[-2000:]


ABI = """
import sys
sys.path[:0] = [%r]
from long_context_attention_attn_amd import _lib
_lib._PATH = sys.argv[1]
import pytest
sys.exit(pytest.main(["-q", "-p", "no:cacheprovider", %r]))
""" % (ROOT, os.path.join(TESTS, "test_abi_host.py"))


def test_abi_host_checks_under_asan_ubsan(tmp_path):
    rt = _clang_runtime()
    if rt is None or not os.path.exists(HIPCC):
        pytest.skip("hipcc or clang's AddressSanitizer runtime is not installed")
    import torch

    if torch.cuda.is_available():
        pytest.skip("a GPU is visible: the host tests expect no device")
    from long_context_attention_attn_amd.build import SOURCES

    lib = str(tmp_path / "liblightning_attn_san.so")
    sources = [os.path.join(CSRC, f) for f in SOURCES]
    cmd = [HIPCC, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC", "-shared",
           "-mcode-object-version=5", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           # host code only: every sanitizer flag goes behind -Xarch_host
           "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=undefined",
           "-Xarch_host", "-fno-omit-frame-pointer", "-o", lib] + sources
    b = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
    assert b.returncode == 0, b.stderr[-4000:]
    r = _child(ABI, rt, lib)
    assert r.returncode == 0, (r.stdout[-3000:], r.stderr[-3000:])
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr
