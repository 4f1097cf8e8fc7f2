"""Helpers shared by the GPU tests: device transfer, per-slice errors, case banners."""
from __future__ import annotations

import sys

import numpy as np
import torch

BF16_TOL = 2e-2  # relative L2 per (sequence, head) slice, bf16 storage / fp32 accumulation
F32_TOL = 1e-4   # relative L2 per (sequence, head) slice, fp32 storage and arithmetic


def banner(msg: str) -> None:
    print("[gpu-case] " + msg, flush=True)
    sys.stdout.flush()


def dev():
    return torch.device("cuda:0")


def to_np(x: torch.Tensor) -> np.ndarray:
    return x.detach().to("cpu").to(torch.float64).numpy()


def rel(a, b, abs_floor: float = 1e-6) -> float:
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    nb = np.linalg.norm(b)
    if nb == 0.0:
        return float(np.linalg.norm(a - b)) / abs_floor if np.linalg.norm(a - b) > abs_floor else 0.0
    return float(np.linalg.norm(a - b) / nb)


def slice_errors(got: np.ndarray, ref: np.ndarray, cu) -> np.ndarray:
    """Relative L2 error per (sequence, head) of [T, H, D] arrays; shape [S, H]."""
    cu = [int(x) for x in cu]
    S, H = len(cu) - 1, ref.shape[1]
    errs = np.zeros((S, H))
    for s in range(S):
        for h in range(H):
            errs[s, h] = rel(got[cu[s]:cu[s + 1], h], ref[cu[s]:cu[s + 1], h])
    return errs


def state_errors(got: np.ndarray, ref: np.ndarray) -> np.ndarray:
    """Relative L2 error per (sequence, head) of [S, H, D, D] states."""
    S, H = ref.shape[:2]
    return np.array([[rel(got[s, h], ref[s, h]) for h in range(H)] for s in range(S)])
