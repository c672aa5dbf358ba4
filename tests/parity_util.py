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


# Backward bars.  Every gradient element is a sum of products in which one factor
# (P, or dS = P o (dP - D)) is rounded once to the input type before the matrix
# core multiplies it, and the result is rounded once more on the store, so its
# error is a few units of roundoff u of that type relative to the size of its row
# (u = 2^-8 for bf16, 2^-11 for fp16).  The error of each element is therefore
# measured against the RMS of its own row of the exact gradient (row sizes differ by
# orders of magnitude under the causal mask), with a floor of 1% of the whole
# tensor's RMS for rows whose exact gradient vanishes (dQ of the first causal
# query is exactly zero):
#   max over elements of |err| / (8 u base)  <= 1,   mean of |err| / base <= u,
# base = row RMS + 1% of the tensor RMS.
# dQ carries one more term.  D_i = dO_i . O_i is formed from the forward's output
# O, which is rounded to the input type, so D_i is off by up to
# u sum_c |dO_ic O_ic|; every dS_ij of the row moves by -P_ij times that, and dQ_i
# by -scale (sum_j P_ij k_j) times it.  Where dP_ij - D_i cancels (a causal row
# with two or three keys) this term is the larger one, so the dQ bar adds
#   t_ic = scale u (sum_c' |dO_ic' O*_ic'|) |(P K)_ic|
# to the allowance, with O* and P K taken from the oracle's forward.
BWD_U = {"bf16": 2.0 ** -8, "f16": 2.0 ** -11}


def bwd_errors(g_gpu, g_ref, u: float, extra=None) -> dict:
    """Errors of one gradient tensor [..., N, d] against the exact one (see above)."""
    g = np.asarray(g_gpu, dtype=np.float64)
    r = np.asarray(g_ref, dtype=np.float64)
    rms_all = float(np.sqrt(np.mean(r * r)))
    base = np.sqrt(np.mean(r * r, axis=-1, keepdims=True)) + 1e-2 * rms_all + 1e-300
    e = np.abs(g - r)
    allow = 8 * u * base + (0.0 if extra is None else extra)
    return dict(ratio=float((e / allow).max()), mean=float((e / base).mean()) / u,
                max_u=float((e / base).max()) / u, finite=bool(np.isfinite(g).all()),
                abs_max=float(e.max()), rms=rms_all)


def bwd_check(err: dict, what: str) -> None:
    assert err["finite"], f"{what}: non-finite gradient"
    assert err["ratio"] <= 1.0, f"{what}: error {err['ratio']:.3f} x the allowance"
    assert err["mean"] <= 1.0, f"{what}: mean row-relative error {err['mean']:.3f} u > 1 u"


def dq_extra(q, k, v, dout, scale: float, causal: bool, u: float, oracle_mod):
    """The dQ allowance t (above) from the oracle's forward of (Q, K, V) and of (Q, K, K)."""
    o_ref, _ = oracle_mod.attn_fwd(q, k, v, scale, causal)
    pk, _ = oracle_mod.attn_fwd(q, k, k, scale, causal)
    dof = np.asarray(dout.double().numpy() if hasattr(dout, "double") else dout, dtype=np.float64)
    dD = u * np.sum(np.abs(dof * o_ref), axis=-1, keepdims=True)
    return scale * dD * np.abs(pk)
