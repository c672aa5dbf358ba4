"""Helpers for comparing the HIP path with the oracle (used by the GPU tests)."""
from __future__ import annotations

import sys

import numpy as np

# Bars (written here once, used by every parity test):
#   fp32 output: max |O - O*| <= 1e-5
#   bf16 / fp16 output: max |O - O*| <= 2e-2 and mean |O - O*| <= 2e-3
#   every dtype: max |lse - lse*| <= 1e-3
TOL = {
    "f32": dict(o_max=1e-5, o_mean=1e-5, lse_max=1e-3),
    "f16": dict(o_max=2e-2, o_mean=2e-3, lse_max=1e-3),
    "bf16": dict(o_max=2e-2, o_mean=2e-3, lse_max=1e-3),
}


def say(msg: str) -> None:
    """Name the case on the real stderr (not captured) before the GPU runs it."""
    sys.__stderr__.write(msg + "\n")
    sys.__stderr__.flush()


def errors(o_gpu, lse_gpu, o_ref, lse_ref) -> dict:
    o = np.asarray(o_gpu, dtype=np.float64)
    l = np.asarray(lse_gpu, dtype=np.float64)
    eo = np.abs(o - o_ref)
    el = np.abs(l - lse_ref)
    return dict(o_max=float(eo.max()), o_mean=float(eo.mean()), lse_max=float(el.max()),
                finite=bool(np.isfinite(o).all() and np.isfinite(l).all()))


def check(err: dict, dtype: str, what: str) -> None:
    tol = TOL[dtype]
    assert err["finite"], f"{what}: non-finite output"
    assert err["o_max"] <= tol["o_max"], f"{what}: max|dO| {err['o_max']:.3e} > {tol['o_max']}"
    assert err["o_mean"] <= tol["o_mean"], f"{what}: mean|dO| {err['o_mean']:.3e} > {tol['o_mean']}"
    assert err["lse_max"] <= tol["lse_max"], f"{what}: max|dlse| {err['lse_max']:.3e} > {tol['lse_max']}"


def sample_rows(N: int, rng: np.random.Generator, n_random: int = 48) -> np.ndarray:
    """Rows at tile edges (32, 64, 128 multiples and their neighbours), both ends, and random."""
    fixed = [0, 1, 2, 31, 32, 33, 63, 64, 65, 127, 128, 129, 255, 256, N // 2, N // 2 + 1,
             N - 129, N - 128, N - 127, N - 65, N - 64, N - 33, N - 32, N - 2, N - 1]
    rows = [r for r in fixed if 0 <= r < N] + list(rng.integers(0, N, size=n_random))
    return np.unique(np.array(rows, dtype=np.int64))
