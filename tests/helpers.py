"""Shared test helpers: tensor <-> numpy for the oracle, tolerances, GPU guard."""
from __future__ import annotations

import os
import sys

import numpy as np
import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

# Output tolerances for the FFN / combine (max-abs error over max |reference|):
# bf16 operands with fp32 accumulation and a bf16 intermediate, and true fp32.
TOL = {"bf16": 1e-2, "f32": 1e-5}
# gate weights: absolute
GATE_W_ATOL = 1e-6
# signature: relative
SIG_RTOL = 1e-6


def np_of(t: torch.Tensor) -> np.ndarray:
    """Host numpy copy; bf16 comes back as its raw uint16 bit patterns."""
    t = t.detach().contiguous().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def f64_of(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().to(torch.float64).numpy()


def rel_max_err(got: np.ndarray, ref: np.ndarray) -> float:
    scale = float(np.abs(ref).max())
    err = float(np.abs(np.asarray(got, dtype=np.float64) - ref).max()) if ref.size else 0.0
    return err / scale if scale > 0 else err


def require_gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU test run without a visible GPU")
    import top_expert_routing_amd as m
    m.load()          # raises if libmoe.so is missing: no fallback exists


def announce(msg: str) -> None:
    print(f"[case] {msg}", flush=True)
