"""fp64 CPU attention oracle — TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  It shares no code with the HIP library
(``exact_attention_96_amd``) and neither imports the other.

The arithmetic lives in ``attn_oracle.c`` (plain C, OpenMP over rows): the
literal definition of scaled-dot-product attention with a causal lower-
triangle mask, softmax over keys and the per-row log-sum-exp, following
"Understand FlashAttention" (nothiny.github.io), sections "前向传播" and
"附：数值稳定的logsumexp(L)推导", and "PyTorch profiling part 3: attention",
section "朴素注意力" (naive attention); and its backward (dQ, dK, dV of a loss
with gradient dO) from "Understand FlashAttention", section "反向传播"; and the
general-mask form (boolean or additive mask, unequal query and key lengths,
safe softmax) from "PyTorch profiling part 3", sections "构建因果掩码" and
"安全 softmax"; and causal linear attention (phi(x) = elu(x) + 1 similarity,
causal dot product, normaliser) from the hqwc.cn notes on the fast-transformers
linear attention kernels, sections 0x0-0x2.  This module only marshals arrays.

Pins (tests/test_oracle.py) tie it to facts the pages and the mathematics fix;
every function here is pinned (none is "parity unpinned").
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(_HERE, "attn_oracle.c")
LIB = os.path.join(_HERE, "liboracle.so")


def build(verbose: bool = False, src: str = SRC, out: str = LIB, werror: bool = True) -> str:
    """Compile attn_oracle.c with gcc into a shared library (always recompiles).

    Plain -O2, no -ffast-math (keeps IEEE semantics and the written summation
    order) and no -march=native (the library must run on other x86 hosts).
    """
    tmp = out + ".tmp"
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp",
           "-Wall", "-Wextra"] + (["-Werror"] if werror else []) + [src, "-o", tmp, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


class OracleLib:
    """ctypes handle on one build of attn_oracle.c (the default one, or a test build)."""

    def __init__(self, path: str = LIB):
        if not os.path.exists(path):
            raise RuntimeError(f"oracle library missing: {path} (run oracle.build())")
        lib = ctypes.CDLL(path)
        dp = ctypes.POINTER(ctypes.c_double)
        i64 = ctypes.c_int64
        lib.oracle_attn_fwd_f64.argtypes = [dp, dp, dp, dp, dp, i64, i64, i64, i64,
                                            ctypes.c_double, ctypes.c_int]
        lib.oracle_attn_fwd_f64.restype = ctypes.c_int
        lib.oracle_attn_rows_f64.argtypes = [dp, dp, dp, i64, i64, ctypes.c_double,
                                             ctypes.c_int, ctypes.POINTER(i64), i64, dp, dp]
        lib.oracle_attn_rows_f64.restype = ctypes.c_int
        lib.oracle_attn_dense_f64.argtypes = [dp, dp, i64, i64, ctypes.c_double,
                                              ctypes.c_int, dp, dp]
        lib.oracle_attn_dense_f64.restype = ctypes.c_int
        lib.oracle_attn_bwd_f64.argtypes = [dp, dp, dp, dp, dp, dp, dp, i64, i64, i64, i64,
                                            ctypes.c_double, ctypes.c_int]
        lib.oracle_attn_bwd_f64.restype = ctypes.c_int
        lib.oracle_attn_masked_f64.argtypes = [dp, dp, dp, dp, i64, i64, dp, dp, i64, i64, i64, i64,
                                               i64, ctypes.c_double, ctypes.c_int]
        lib.oracle_attn_masked_f64.restype = ctypes.c_int
        lib.oracle_linattn_f64.argtypes = [dp, dp, dp, dp, i64, i64, i64, i64, ctypes.c_int,
                                           ctypes.c_double]
        lib.oracle_linattn_f64.restype = ctypes.c_int
        lib.oracle_num_threads.argtypes = []
        lib.oracle_num_threads.restype = ctypes.c_int
        self.lib = lib
        self.path = path

    def num_threads(self) -> int:
        return int(self.lib.oracle_num_threads())

    def attn_fwd(self, q, k, v, scale: float, causal: bool):
        """O, lse for q, k, v of shape [B, H, N, d] (any float dtype, widened exactly)."""
        q, k, v = _f64(q), _f64(k), _f64(v)
        if q.ndim != 4 or q.shape != k.shape or q.shape != v.shape:
            raise ValueError("q, k, v must share one [B, H, N, d] shape")
        B, H, N, d = q.shape
        o = np.empty_like(q)
        lse = np.empty((B, H, N), dtype=np.float64)
        rc = self.lib.oracle_attn_fwd_f64(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse),
                                          B, H, N, d, float(scale), int(bool(causal)))
        if rc:
            raise RuntimeError(f"oracle_attn_fwd_f64 failed with status {rc}")
        return o, lse

    def attn_rows(self, q, k, v, scale: float, causal: bool, rows):
        """O[rows], lse[rows] for ONE head: q, k, v of shape [N, d]."""
        q, k, v = _f64(q), _f64(k), _f64(v)
        if q.ndim != 2 or q.shape != k.shape or q.shape != v.shape:
            raise ValueError("q, k, v must share one [N, d] shape")
        N, d = q.shape
        rows = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
        o = np.empty((rows.size, d), dtype=np.float64)
        lse = np.empty((rows.size,), dtype=np.float64)
        rc = self.lib.oracle_attn_rows_f64(
            _ptr(q), _ptr(k), _ptr(v), N, d, float(scale), int(bool(causal)),
            rows.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)), rows.size, _ptr(o), _ptr(lse))
        if rc:
            raise RuntimeError(f"oracle_attn_rows_f64 failed with status {rc}")
        return o, lse

    def attn_dense(self, q, k, scale: float, causal: bool):
        """Dense S (scaled, masked to -inf) and P = softmax(S) for ONE head [N, d]."""
        q, k = _f64(q), _f64(k)
        if q.ndim != 2 or q.shape != k.shape:
            raise ValueError("q, k must share one [N, d] shape")
        N, d = q.shape
        S = np.empty((N, N), dtype=np.float64)
        P = np.empty((N, N), dtype=np.float64)
        rc = self.lib.oracle_attn_dense_f64(_ptr(q), _ptr(k), N, d, float(scale),
                                            int(bool(causal)), _ptr(S), _ptr(P))
        if rc:
            raise RuntimeError(f"oracle_attn_dense_f64 failed with status {rc}")
        return S, P

    def attn_bwd(self, q, k, v, dout, scale: float, causal: bool):
        """dQ, dK, dV of a loss whose gradient with respect to O is dout, all [B, H, N, d]
        ("Understand FlashAttention", section "反向传播", with the scale on dQ and dK)."""
        q, k, v, dout = _f64(q), _f64(k), _f64(v), _f64(dout)
        if q.ndim != 4 or any(t.shape != q.shape for t in (k, v, dout)):
            raise ValueError("q, k, v, dout must share one [B, H, N, d] shape")
        B, H, N, d = q.shape
        dq, dk, dv = np.empty_like(q), np.empty_like(q), np.empty_like(q)
        rc = self.lib.oracle_attn_bwd_f64(_ptr(q), _ptr(k), _ptr(v), _ptr(dout), _ptr(dq), _ptr(dk),
                                          _ptr(dv), B, H, N, d, float(scale), int(bool(causal)))
        if rc:
            raise RuntimeError(f"oracle_attn_bwd_f64 failed with status {rc}")
        return dq, dk, dv

    def attn_masked(self, q, k, v, scale: float, causal: bool, mask=None, kind: str = "bool"):
        """O [B, H, Nq, d], lse [B, H, Nq] with a general mask and Nq != Nk allowed.

        q: [B, H, Nq, d]; k, v: [B, H, Nk, d].  mask: None, or an array broadcastable to
        [B, H, Nq, Nk] whose leading two axes are B or 1: kind "bool" (nonzero = key visible,
        turned into an additive 0 / -inf bias as the math backend does, "PyTorch profiling
        part 3", section "构建因果掩码") or kind "add" (added to the scaled scores).
        causal: bottom-right aligned lower triangle (key j visible iff j <= i + Nk - Nq).
        Rows that see no key: o = 0, lse = -inf.
        """
        q, k, v = _f64(q), _f64(k), _f64(v)
        if q.ndim != 4 or k.ndim != 4 or k.shape != v.shape or q.shape[:2] != k.shape[:2] \
                or q.shape[3] != k.shape[3]:
            raise ValueError("q [B, H, Nq, d], k and v [B, H, Nk, d] expected")
        B, H, Nq, d = q.shape
        Nk = k.shape[2]
        bias_p, sb, sh = None, 0, 0
        if mask is not None:
            m = _f64(mask) if kind == "add" else None
            if kind == "bool":
                mb = np.asarray(mask.detach().cpu().numpy() if hasattr(mask, "detach") else mask)
                m = np.where(mb != 0, 0.0, -np.inf)
            elif kind != "add":
                raise ValueError("kind must be 'bool' or 'add'")
            if m.ndim != 4 or m.shape[2:] != (Nq, Nk) or m.shape[0] not in (1, B) \
                    or m.shape[1] not in (1, H):
                raise ValueError(f"mask of shape {m.shape} does not broadcast to {(B, H, Nq, Nk)}")
            m = np.ascontiguousarray(m, dtype=np.float64)
            sb = 0 if m.shape[0] == 1 else m.shape[1] * Nq * Nk
            sh = 0 if m.shape[1] == 1 else Nq * Nk
            bias_p = m
        o = np.empty((B, H, Nq, d), dtype=np.float64)
        lse = np.empty((B, H, Nq), dtype=np.float64)
        rc = self.lib.oracle_attn_masked_f64(
            _ptr(q), _ptr(k), _ptr(v), _ptr(bias_p) if bias_p is not None else None, sb, sh,
            _ptr(o), _ptr(lse), B, H, Nq, Nk, d, float(scale), int(bool(causal)))
        if rc:
            raise RuntimeError(f"oracle_attn_masked_f64 failed with status {rc}")
        return o, lse

    def linear_attn(self, q, k, v, feature_map: bool = True, eps: float = 1e-6):
        """Causal linear attention, out [B, H, N, M] for q, k [B, H, N, E], v [B, H, N, M].

        feature_map=False: the causal dot product out_j = sum_{t<=j} (q_j . k_t) v_t;
        True: phi = elu + 1 on q and k, and out_j = that product of phi(q), phi(k), v
        times 1 / (phi(q_j) . sum_{t<=j} phi(k_t) + eps).
        """
        q, k, v = _f64(q), _f64(k), _f64(v)
        if q.ndim != 4 or k.shape != q.shape or v.ndim != 4 or v.shape[:3] != q.shape[:3]:
            raise ValueError("q, k [B, H, N, E] and v [B, H, N, M] expected")
        B, H, N, E = q.shape
        M = v.shape[3]
        out = np.empty((B, H, N, M), dtype=np.float64)
        rc = self.lib.oracle_linattn_f64(_ptr(q), _ptr(k), _ptr(v), _ptr(out), B * H, N, E, M,
                                         int(bool(feature_map)), float(eps))
        if rc:
            raise RuntimeError(f"oracle_linattn_f64 failed with status {rc}")
        return out


def _f64(x) -> np.ndarray:
    """Exact widening of a torch tensor or array to a C-contiguous fp64 array."""
    if hasattr(x, "detach"):  # torch tensor (any float dtype, CPU or GPU)
        x = x.detach().to("cpu").double().numpy()
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


_default = None


def default() -> OracleLib:
    global _default
    if _default is None:
        _default = OracleLib(LIB)
    return _default


def num_threads() -> int:
    return default().num_threads()


def attn_fwd(q, k, v, scale: float, causal: bool):
    return default().attn_fwd(q, k, v, scale, causal)


def attn_rows(q, k, v, scale: float, causal: bool, rows):
    return default().attn_rows(q, k, v, scale, causal, rows)


def attn_dense(q, k, scale: float, causal: bool):
    return default().attn_dense(q, k, scale, causal)


def attn_bwd(q, k, v, dout, scale: float, causal: bool):
    return default().attn_bwd(q, k, v, dout, scale, causal)


def attn_masked(q, k, v, scale: float, causal: bool, mask=None, kind: str = "bool"):
    return default().attn_masked(q, k, v, scale, causal, mask, kind)


def linear_attn(q, k, v, feature_map: bool = True, eps: float = 1e-6):
    return default().linear_attn(q, k, v, feature_map, eps)
