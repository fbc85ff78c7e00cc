"""Shared helpers of the GPU parity tests (tolerances, comparisons, device setup)."""
from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

# Attention outputs: float32 max-abs 1e-4; bf16 max-abs 2e-2 and mean-abs 2e-3
# against the float64 oracle on the same stored inputs.
TOL = {"f32": dict(max_abs=1e-4, mean_abs=1e-4), "bf16": dict(max_abs=2e-2, mean_abs=2e-3)}
# LSE is float32 in both paths. bf16 inputs: the row sum adds bf16-rounded P
# (relative error <= 2^-9 per term), so |d LSE| <= ~2e-3; 5e-3 leaves margin.
LSE_TOL = {"f32": 1e-4, "bf16": 5e-3}


def device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def announce(msg: str):
    """Names the case on stdout before a GPU step, so a fault can be attributed."""
    print(f"\n[case] {msg}", flush=True)
    sys.stdout.flush()


def to_f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu").to(torch.float64).numpy()


def bits(t: torch.Tensor) -> np.ndarray:
    t = t.detach().to("cpu").contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.view(torch.int32).numpy().view(np.uint32)


def assert_attention_close(got: np.ndarray, want: np.ndarray, dtype: str, what: str):
    err = np.abs(got - want)
    mx, mean = float(err.max()), float(err.mean())
    rel = mx / max(float(np.abs(want).max()), 1e-30)
    tol = TOL[dtype]
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    assert mx <= tol["max_abs"] and mean <= tol["mean_abs"], (
        f"{what}: max-abs {mx:.3e} (tol {tol['max_abs']}), mean-abs {mean:.3e} "
        f"(tol {tol['mean_abs']}), max-abs/max|ref| {rel:.3e}")
    return mx, mean


def assert_lse_close(got: np.ndarray, want: np.ndarray, dtype: str, what: str):
    mx = float(np.abs(got - want).max())
    assert mx <= LSE_TOL[dtype], f"{what}: LSE max-abs {mx:.3e} (tol {LSE_TOL[dtype]})"
