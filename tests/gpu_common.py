"""Helpers shared by the GPU parity tests (not collected as tests)."""

from __future__ import annotations

import sys

import numpy as np
import pytest

# bf16 in, fp32 accumulate, compared with the fp64 oracle on the same inputs
BF16_MAX_ABS = 2e-2
BF16_REL_L2 = 5e-3
# fp32 caches: fp32 dot products and softmax over at most a few thousand keys
FP32_MAX_ABS = 1e-4
FP32_REL_L2 = 1e-5
# LSE = m + ln l.  The bf16 kernel's l sums the bf16-rounded probabilities that
# also enter the PV product (each within a relative 2^-8 of its fp32 value, so
# O stays consistent with its own denominator): |ln l' - ln l| <= -ln(1 - 2^-8)
# < 3.92e-3, reached only when few keys carry the sum (it averages out over
# many).  fp32 caches sum fp32 probabilities: about 1e-6 over a few thousand
# keys, bounded here by 1e-4.
LSE_ABS_BF16 = 3.92e-3
LSE_ABS_FP32 = 1e-4


def torch_cuda():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch


def to64(t) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def to32(t) -> np.ndarray:
    return t.detach().float().cpu().numpy()


def rel_l2(a, ref) -> float:
    return float(np.linalg.norm((a - ref).ravel()) / max(np.linalg.norm(ref.ravel()), 1e-300))


def max_abs(a, ref) -> float:
    return float(np.max(np.abs(a - ref))) if a.size else 0.0


def assert_close(out, ref, bf16: bool, what: str):
    ma, rl = max_abs(out, ref), rel_l2(out, ref)
    tol_ma, tol_rl = (BF16_MAX_ABS, BF16_REL_L2) if bf16 else (FP32_MAX_ABS, FP32_REL_L2)
    assert ma <= tol_ma and rl <= tol_rl, f"{what}: max_abs {ma:.3e} (tol {tol_ma}), rel_l2 {rl:.3e} (tol {tol_rl})"
    return ma, rl


def say(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()
