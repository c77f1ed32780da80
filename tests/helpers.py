"""Shared helpers of the GPU parity tests (device upload, tolerance checks)."""
from __future__ import annotations

import sys

import numpy as np
import torch

# bars: bf16 I/O with fp32 accumulation, and the fp32 path
TOL_BF16_MAX, TOL_BF16_MEAN = 3e-2, 3e-3
TOL_FP32 = 1e-4


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def tdt(dtype: str):
    return torch.bfloat16 if dtype == "bf16" else torch.float32


def dev(a: np.ndarray, dtype: str) -> torch.Tensor:
    """Upload float32 values (already representable in `dtype`) exactly."""
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(tdt(dtype))
    return t.cuda()


def dev_params(p: dict, dtype: str) -> dict:
    return {k: dev(v, dtype) for k, v in p.items()}


def host64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def check(got: np.ndarray, ref: np.ndarray, dtype: str, what: str = ""):
    err = np.abs(np.asarray(got, np.float64) - np.asarray(ref, np.float64))
    assert np.isfinite(got).all(), f"{what}: non-finite output"
    mx, mean = float(err.max()) if err.size else 0.0, float(err.mean()) if err.size else 0.0
    say(f"  {what}: max-abs {mx:.3e} mean-abs {mean:.3e}")
    if dtype == "bf16":
        assert mx <= TOL_BF16_MAX and mean <= TOL_BF16_MEAN, f"{what}: max {mx:.3e} mean {mean:.3e}"
    else:
        assert mx <= TOL_FP32, f"{what}: max {mx:.3e}"
    return mx, mean
