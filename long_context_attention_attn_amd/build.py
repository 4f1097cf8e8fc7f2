"""Build liblightning_attn.so in-tree with hipcc for gfx950.

Usage:  python -m long_context_attention_attn_amd.build
Each .hip file is compiled to an object in parallel, then linked into one shared library next
to this file.  Flags: -O3, code-object v5, packed-fp32 instructions disabled
(-Xclang -target-feature -Xclang -packed-fp32-ops), MFMA accumulators in VGPRs.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "liblightning_attn.so")
BUILD_DIR = os.path.join(ROOT, "_build")
SOURCES = ["la_api.hip", "prefill_bf16.hip", "prefill_bf16_b128.hip", "prefill_f32.hip",
           "decode.hip", "split.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

COMMON = [
    "--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-mcode-object-version=5",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE, "-I", CSRC, "-Wall", "-Wno-unused-result",
    # keep MFMA accumulators in ordinary VGPRs (no AGPR<->VGPR copies around the VALU work
    # that reads them)
    "-mllvm", "-amdgpu-mfma-vgpr-form",
]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC] + COMMON + ["-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s\n%s" % (src, " ".join(cmd), r.stderr))
    return obj


def build(verbose: bool = False) -> str:
    """Compile every HIP source and link the shared library; returns its path."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 1, 16)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n%s\n%s" % (" ".join(cmd), r.stderr))
    os.replace(tmp, LIB)
    if verbose:
        print("built", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
