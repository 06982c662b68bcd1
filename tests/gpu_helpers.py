"""Shared helpers for the GPU tests: device checks, host copies and the tolerance
rules the GPU results are held to against the CPU oracle."""
from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

# fp32 workloads: max |gpu - oracle| over every element
F32_ABS_TOL = 1e-5
# bf16 workloads: for every output row r, max_i |gpu - oracle| <= 2e-2 * max_i |oracle|
BF16_ROW_REL_TOL = 2e-2


def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def announce(msg: str) -> None:
    """Name the case before a GPU step, flushed, so a crash still tells which one."""
    print(f"[gpu case] {msg}", flush=True)
    sys.stdout.flush()


def host(t: torch.Tensor) -> np.ndarray:
    """Exact float64 copy of a device tensor (bf16 and fp32 widen exactly)."""
    return t.detach().to(torch.float32).cpu().numpy().astype(np.float64)


def check_f32_abs(gpu: np.ndarray, ref: np.ndarray, tol: float = F32_ABS_TOL) -> float:
    assert gpu.shape == ref.shape, (gpu.shape, ref.shape)
    assert np.all(np.isfinite(gpu)), "non-finite GPU output"
    err = float(np.max(np.abs(gpu - ref))) if gpu.size else 0.0
    assert err <= tol, f"max abs error {err:.3e} > {tol:.0e}"
    return err


def check_rows_rel(gpu: np.ndarray, ref: np.ndarray, row: int, tol: float = BF16_ROW_REL_TOL):
    """Per-row relative rule over rows of ``row`` consecutive elements (the last
    axis is split into rows of that width)."""
    assert gpu.shape == ref.shape, (gpu.shape, ref.shape)
    assert np.all(np.isfinite(gpu)), "non-finite GPU output"
    g = gpu.reshape(-1, row)
    r = ref.reshape(-1, row)
    err = np.max(np.abs(g - r), axis=1)
    scale = np.max(np.abs(r), axis=1)
    bad = err > tol * scale
    worst = float(np.max(err / np.maximum(scale, 1e-300)))
    assert not np.any(bad), (f"{int(bad.sum())} of {len(bad)} rows exceed {tol} x row max; "
                             f"worst ratio {worst:.3e}")
    return worst, float(np.max(np.abs(g - r)))
