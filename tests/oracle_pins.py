"""Pins for the fp64 oracle: facts fixed by the pages and by the mathematics.

Each ``pin_*`` takes an oracle handle (``oracle.OracleLib``) and raises
AssertionError when the oracle disagrees with the fact it pins.  The same
battery runs against the real oracle (tests/test_oracle.py) and against
deliberately broken builds of it (tests/test_oracle_mutants.py), which shows
that a plausible slip anywhere in the oracle fails at least one pin.

Sources (pages cited by title and section):
  [FA]  "Understand FlashAttention" (nothiny.github.io)
        - "数值稳定的 Softmax": softmax(x)_i = e^{x_i-m} / sum_j e^{x_j-m}
        - "关键统计量": per-row m (row max) and l (sum of e^{x-m})
        - "两块情况的完整推导", steps 1-8: the blockwise (online) recurrence
        - "前向传播": S = Q K^T, P = softmax(S), O = P V
        - "附：数值稳定的logsumexp(L)推导": L_i = log sum_j e^{S_ij} = m_i + log l_i
  [PT]  "PyTorch profiling part 3: attention" (Hugging Face blog, Chinese translation)
        - "朴素注意力": scores = q k^T, times scale, masked to -inf, softmax, times v
        - "缩放点积注意力" / "那么 math 后端有什么用？": torch's SDPA math path is a
          plain decomposition of the same operation (used as an independent library)
        - "构建因果掩码": the causal mask is the lower triangle (tril), key j <= query i
  [FA]  "反向传播": dV = P^T dO, dP = dO V^T, dS = P o (dP - rowsum(P o dP)),
        dQ = dS K, dK = dS^T Q (the backward pins below; S carries the scale)
  [PT]  "构建因果掩码" (a mask enters as an additive 0 / -inf bias after scaling) and
        "安全 softmax" (a row with every entry -inf yields zeros, not 0/0): the
        general-mask pins below; for Nq != Nk the causal triangle is anchored at the
        bottom-right corner (the queries are the last Nq positions of the keys)
"""
from __future__ import annotations

import json
import math
import os
from decimal import Decimal, getcontext

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "hand_examples.json")


def _close(a, b, tol, what):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, f"{what}: shape {a.shape} vs {b.shape}"
    both_inf = np.isinf(a) & np.isinf(b) & (np.sign(a) == np.sign(b))
    with np.errstate(invalid="ignore"):
        err = np.where(both_inf, 0.0, np.abs(a - b))
    worst = float(np.max(err)) if err.size else 0.0
    assert np.all(np.isfinite(err)) and worst <= tol, f"{what}: max err {worst:.3e} > {tol:.1e}"


def _one_head(orc, q, k, v, scale, causal):
    o, lse = orc.attn_fwd(q[None, None], k[None, None], v[None, None], scale, causal)
    return o[0, 0], lse[0, 0]


# ---------------------------------------------------------------- closed forms

def pin_golden_hand_examples(orc):
    """Hand-derived closed forms ([FA] 前向传播 + logsumexp appendix, [PT] 朴素注意力, 构建因果掩码)."""
    with open(GOLDEN) as f:
        data = json.load(f)
    for ex in data["examples"]:
        q, k, v = (np.array(ex[n], dtype=np.float64) for n in ("q", "k", "v"))
        o, lse = _one_head(orc, q, k, v, ex["scale"], ex["causal"])
        _close(o, np.array([[float(x) for x in r] for r in ex["o"]]), 1e-14, ex["name"] + " o")
        _close(lse, np.array([float(x) for x in ex["lse"]]), 1e-14, ex["name"] + " lse")


def _decimal_attention(q, k, v, scale, causal):
    """Brute force in 40-digit decimal arithmetic: the [PT] naive-attention steps."""
    getcontext().prec = 40
    N, d = len(q), len(q[0])
    sc = Decimal(scale)
    S, P, O, L = [], [], [], []
    for i in range(N):
        srow = []
        for j in range(N):
            if causal and j > i:
                srow.append(None)
            else:
                dot = sum(Decimal(q[i][c]) * Decimal(k[j][c]) for c in range(d))
                srow.append(dot * sc)
        m = max(x for x in srow if x is not None)
        w = [Decimal(0) if x is None else (x - m).exp() for x in srow]
        l = sum(w)
        prow = [x / l for x in w]
        orow = [sum(prow[j] * Decimal(v[j][c]) for j in range(N)) for c in range(d)]
        S.append(srow)
        P.append(prow)
        O.append(orow)
        L.append(m + l.ln())
    return S, P, O, L


def pin_bruteforce_decimal(orc):
    """Tiny integer inputs (scores exact in fp64) against a 40-digit brute force."""
    rng = np.random.default_rng(1234)
    for trial in range(40):
        N = int(rng.integers(1, 5))
        d = int(rng.integers(1, 3))
        hi = 2 if trial < 30 else 30  # the last trials have logits up to ~900
        q = rng.integers(-hi, hi + 1, size=(N, d)).astype(np.float64)
        k = rng.integers(-hi, hi + 1, size=(N, d)).astype(np.float64)
        v = rng.integers(-2, 3, size=(N, d)).astype(np.float64)
        causal = bool(trial % 2)
        scale = 0.5
        S_ref, P_ref, O_ref, L_ref = _decimal_attention(q.tolist(), k.tolist(), v.tolist(),
                                                        scale, causal)
        S, P = orc.attn_dense(q, k, scale, causal)
        for i in range(N):
            for j in range(N):
                want = -math.inf if S_ref[i][j] is None else float(S_ref[i][j])
                assert S[i, j] == want, f"S[{i},{j}] = {S[i, j]} != {want} (trial {trial})"
        _close(P, np.array([[float(x) for x in r] for r in P_ref]), 1e-15, f"P trial {trial}")
        o, lse = _one_head(orc, q, k, v, scale, causal)
        _close(o, np.array([[float(x) for x in r] for r in O_ref]), 1e-14, f"O trial {trial}")
        _close(lse, np.array([float(x) for x in L_ref]), 1e-13, f"lse trial {trial}")


def pin_two_keys_sigmoid(orc):
    """N = 2: row 1 is a two-way softmax, o_1 = sig(s11-s10) v1 + sig(s10-s11) v0,
    lse_1 = log(e^{s10} + e^{s11}) ([FA] logsumexp appendix)."""
    rng = np.random.default_rng(7)
    for causal in (False, True):
        q, k, v = rng.standard_normal((3, 2, 5))
        scale = 0.37
        o, lse = _one_head(orc, q, k, v, scale, causal)
        s10, s11 = scale * (q[1] @ k[0]), scale * (q[1] @ k[1])
        sig = 1.0 / (1.0 + math.exp(-(s11 - s10)))
        _close(o[1], sig * v[1] + (1 - sig) * v[0], 1e-14, "o_1")
        mx = max(s10, s11)
        _close(lse[1], mx + math.log(math.exp(s10 - mx) + math.exp(s11 - mx)), 1e-14, "lse_1")
        if causal:  # row 0 sees key 0 alone
            assert np.array_equal(o[0], v[0]) and lse[0] == scale * (q[0] @ k[0])


def pin_zero_query(orc):
    """Q = 0 makes every allowed score 0: uniform weights over exactly the allowed keys.
    Causal: o_i = mean(v_0..v_i), lse_i = log(i+1); non-causal: mean(V), log N."""
    rng = np.random.default_rng(11)
    N, d = 37, 5
    q = np.zeros((N, d))
    k = rng.standard_normal((N, d))
    v = rng.standard_normal((N, d))
    o, lse = _one_head(orc, q, k, v, 0.125, True)
    _close(o, np.cumsum(v, axis=0) / np.arange(1, N + 1)[:, None], 1e-14, "causal mean")
    _close(lse, np.log(np.arange(1, N + 1)), 1e-14, "causal log(i+1)")
    o, lse = _one_head(orc, q, k, v, 0.125, False)
    _close(o, np.broadcast_to(v.mean(axis=0), (N, d)), 1e-14, "mean")
    _close(lse, np.full(N, math.log(N)), 1e-14, "log N")


def pin_causal_row0_and_single_key(orc):
    """Causal row 0 attends to key 0 only: o_0 = v_0 exactly, lse_0 = s_00 exactly.
    N = 1 (either mode) is the same situation."""
    rng = np.random.default_rng(3)
    q, k, v = rng.standard_normal((3, 9, 4))
    o, lse = _one_head(orc, q, k, v, 0.5, True)
    assert np.array_equal(o[0], v[0]), "causal o_0 != v_0"
    assert lse[0] == (q[0] @ k[0]) * 0.5, "causal lse_0 != s_00"
    for causal in (False, True):
        o, lse = _one_head(orc, q[:1], k[:1], v[:1], 0.5, causal)
        assert np.array_equal(o[0], v[0]) and lse[0] == (q[0] @ k[0]) * 0.5


# ---------------------------------------------------------------- invariants

def pin_normalization(orc):
    """Softmax rows sum to 1 ([FA] 数值稳定的 Softmax); a constant V gives that constant;
    sum_j e^{S_ij - L_i} = 1 ([FA] 为什么保存 logsumexp: P_ij = e^{S_ij - L_i})."""
    rng = np.random.default_rng(5)
    for causal in (False, True):
        N, d = 50, 8
        q, k = rng.standard_normal((2, N, d)) * 2
        S, P = orc.attn_dense(q, k, 0.3, causal)
        _close(P.sum(axis=1), np.ones(N), 1e-14 * N, "row sums")
        if causal:
            assert np.all(P[np.triu_indices(N, 1)] == 0.0), "masked weights not zero"
        c = rng.standard_normal(d)
        v = np.broadcast_to(c, (N, d)).copy()
        o, lse = _one_head(orc, q, k, v, 0.3, causal)
        _close(o, v, 1e-14, "constant V")
        _close(np.exp(S - lse[:, None]).sum(axis=1), np.ones(N), 1e-13, "sum e^{S-L}")
        vr = rng.standard_normal((N, d))
        o, _ = _one_head(orc, q, k, vr, 0.3, causal)
        _close(o, P @ vr, 1e-13, "O = P V")


def _blockwise(q, k, v, scale, causal, bounds):
    """[FA] 两块情况的完整推导 applied block after block (steps 1-7 per key block,
    step 8 once), written independently of the oracle, all query rows at once."""
    N, d = q.shape
    m = np.full(N, -np.inf)
    l = np.zeros(N)
    acc = np.zeros((N, d))
    rows = np.arange(N)[:, None]
    for a, b in bounds:
        S = (q @ k[a:b].T) * scale
        if causal:
            S = np.where(np.arange(a, b)[None, :] > rows, -np.inf, S)
        m_new = np.maximum(m, S.max(axis=1))
        m_use = np.where(np.isinf(m_new), 0.0, m_new)
        alpha = np.exp(m - m_use)
        p = np.exp(S - m_use[:, None])
        l = alpha * l + p.sum(axis=1)
        acc = alpha[:, None] * acc + p @ v[a:b]
        m = m_new
    return acc / l[:, None], m + np.log(l)


def pin_online_recurrence(orc):
    """The blockwise m/l/O rescaling equals the full softmax ([FA] steps 5-8), for
    random block partitions (size-1 blocks included) and large dynamic range."""
    rng = np.random.default_rng(99)
    for trial in range(12):
        N = int(rng.integers(1, 90))
        d = int(rng.integers(1, 20))
        q, k, v = rng.standard_normal((3, N, d))
        k[rng.random(N) < 0.1] *= 8.0  # spiky keys: the running max jumps
        if trial % 3 == 0:
            cuts = np.arange(1, N)  # every block has one key
        else:
            cuts = np.sort(rng.choice(np.arange(1, N), size=min(N - 1, int(rng.integers(0, 8))),
                                      replace=False)) if N > 1 else np.array([], dtype=int)
        edges = [0] + [int(c) for c in cuts] + [N]
        bounds = list(zip(edges[:-1], edges[1:]))
        causal = bool(trial % 2)
        o_ref, lse_ref = _blockwise(q, k, v, 0.7, causal, bounds)
        o, lse = _one_head(orc, q, k, v, 0.7, causal)
        _close(o, o_ref, 1e-12, f"online O trial {trial}")
        _close(lse, lse_ref, 1e-12, f"online lse trial {trial}")


def pin_shift_invariance(orc):
    """Adding the same constant to every score of a row leaves P (hence O) unchanged and
    shifts L by that constant ([FA] 数值稳定的 Softmax)."""
    rng = np.random.default_rng(21)
    N, d = 40, 6
    q, k, v = rng.standard_normal((3, N, d))
    c = 3.25
    q2 = np.concatenate([q, np.ones((N, 1))], axis=1)
    k2 = np.concatenate([k, np.full((N, 1), c)], axis=1)
    v2 = np.concatenate([v, np.full((N, 1), -2.0)], axis=1)
    for causal in (False, True):
        o, lse = _one_head(orc, q, k, v, 0.5, causal)
        o2, lse2 = _one_head(orc, q2, k2, v2, 0.5, causal)
        _close(o2[:, :d], o, 1e-13, "shift O")
        _close(o2[:, d], np.full(N, -2.0), 1e-14, "shift constant column")
        _close(lse2, lse + 0.5 * c, 1e-13, "shift lse")


def pin_permutation(orc):
    """Non-causal: permuting K and V rows together leaves O and L unchanged; permuting
    Q rows permutes O rows.  Causal: row i equals the last row of the non-causal
    problem restricted to keys 0..i (the lower-triangle mask, [PT] 构建因果掩码)."""
    rng = np.random.default_rng(8)
    N, d = 33, 7
    q, k, v = rng.standard_normal((3, N, d))
    o, lse = _one_head(orc, q, k, v, 0.4, False)
    pk = rng.permutation(N)
    o2, lse2 = _one_head(orc, q, k[pk], v[pk], 0.4, False)
    _close(o2, o, 1e-13, "perm KV O")
    _close(lse2, lse, 1e-13, "perm KV lse")
    pq = rng.permutation(N)
    o3, lse3 = _one_head(orc, q[pq], k, v, 0.4, False)
    _close(o3, o[pq], 1e-15, "perm Q O")
    _close(lse3, lse[pq], 1e-15, "perm Q lse")
    oc, lsec = _one_head(orc, q, k, v, 0.4, True)
    for i in (0, 1, 5, 17, N - 1):
        oi, li = _one_head(orc, q[: i + 1], k[: i + 1], v[: i + 1], 0.4, False)
        _close(oc[i], oi[i], 1e-15, f"causal prefix row {i}")
        _close(lsec[i], li[i], 1e-15, f"causal prefix lse {i}")


def pin_scale_and_linearity(orc):
    """The scale multiplies q.k: (2q, scale/2) and (4k, scale/4) give identical results
    (exact powers of two).  O is linear in V."""
    rng = np.random.default_rng(13)
    N, d = 29, 6
    q, k, v, v2 = rng.standard_normal((4, N, d))
    for causal in (False, True):
        o, lse = _one_head(orc, q, k, v, 0.3, causal)
        oa, la = _one_head(orc, 2 * q, k, v, 0.15, causal)
        ob, lb = _one_head(orc, q, 4 * k, v, 0.075, causal)
        _close(oa, o, 1e-15, "2q")
        _close(la, lse, 1e-15, "2q lse")
        _close(ob, o, 1e-15, "4k")
        _close(lb, lse, 1e-15, "4k lse")
        o2, _ = _one_head(orc, q, k, v2, 0.3, causal)
        o3, _ = _one_head(orc, q, k, 1.5 * v - 0.25 * v2, 0.3, causal)
        _close(o3, 1.5 * o - 0.25 * o2, 1e-13, "linear in V")
        # doubling the scale is not the same as doubling V: the weights sharpen
        o4, _ = _one_head(orc, q, k, v, 0.6, causal)
        assert np.max(np.abs(o4 - o)) > 1e-3


def pin_torch_sdpa(orc):
    """Cross-check with torch's own CPU fp64 SDPA math path and torch.logsumexp, an
    independent decomposition of the same operation ([PT] math backend)."""
    import torch
    import torch.nn.functional as F
    rng = np.random.default_rng(17)
    for (B, H, N, d) in [(1, 1, 1, 1), (2, 3, 7, 16), (1, 2, 64, 64), (1, 1, 130, 128)]:
        for causal in (False, True):
            q, k, v = (rng.standard_normal((B, H, N, d)) for _ in range(3))
            scale = 1.0 / math.sqrt(d)
            o, lse = orc.attn_fwd(q, k, v, scale, causal)
            tq, tk, tv = (torch.from_numpy(x) for x in (q, k, v))
            ref = F.scaled_dot_product_attention(tq, tk, tv, is_causal=causal, scale=scale)
            s = torch.matmul(tq, tk.transpose(-1, -2)) * scale
            if causal:
                s = s.masked_fill(torch.ones(N, N, dtype=torch.bool).triu(1), float("-inf"))
            _close(o, ref.numpy(), 1e-12, f"sdpa O {B,H,N,d,causal}")
            _close(lse, torch.logsumexp(s, dim=-1).numpy(), 1e-12, f"sdpa lse {B,H,N,d,causal}")


def pin_rows_api(orc):
    """Row-by-row evaluation returns exactly the rows of the full evaluation."""
    rng = np.random.default_rng(4)
    N, d = 70, 9
    q, k, v = rng.standard_normal((3, N, d))
    rows = np.array([0, 1, 33, 69, 5, 5])
    for causal in (False, True):
        o, lse = _one_head(orc, q, k, v, 0.25, causal)
        orow, lrow = orc.attn_rows(q, k, v, 0.25, causal, rows)
        assert np.array_equal(orow, o[rows]) and np.array_equal(lrow, lse[rows])


def pin_heads_independent(orc):
    """Each (b, h) head is its own problem: a batched call equals per-head calls."""
    rng = np.random.default_rng(6)
    B, H, N, d = 2, 3, 19, 4
    q, k, v = rng.standard_normal((3, B, H, N, d))
    for causal in (False, True):
        o, lse = orc.attn_fwd(q, k, v, 0.5, causal)
        for b in range(B):
            for h in range(H):
                oh, lh = _one_head(orc, q[b, h], k[b, h], v[b, h], 0.5, causal)
                assert np.array_equal(o[b, h], oh) and np.array_equal(lse[b, h], lh)


# ---------------------------------------------------------------- backward

def _loss(orc, q, k, v, g, scale, causal):
    """L = sum(O * g): its gradient with respect to O is g."""
    o, _ = orc.attn_fwd(q, k, v, scale, causal)
    return float(np.sum(o * g))


def pin_bwd_finite_differences(orc):
    """Every entry of dQ, dK, dV equals the central difference of L = sum(O g) computed
    with the forward oracle (a derivative fixed by the forward alone)."""
    rng = np.random.default_rng(23)
    B, H, N, d = 1, 2, 5, 3
    h = 1e-5
    for causal in (False, True):
        q, k, v, g = (rng.standard_normal((B, H, N, d)) for _ in range(4))
        grads = orc.attn_bwd(q, k, v, g, 0.8, causal)
        for which, grad in enumerate(grads):
            num = np.empty_like(grad)
            for idx in np.ndindex(grad.shape):
                args = [q, k, v]
                plus = [a.copy() for a in args]
                minus = [a.copy() for a in args]
                plus[which][idx] += h
                minus[which][idx] -= h
                num[idx] = (_loss(orc, *plus, g, 0.8, causal) - _loss(orc, *minus, g, 0.8, causal)) / (2 * h)
            _close(grad, num, 1e-8, f"finite differences {'qkv'[which]} causal={causal}")


def pin_bwd_constant_values(orc):
    """Equal V rows make O independent of the weights, so dQ = dK = 0; dV still
    carries P^T dO ([FA] 反向传播: dS_ij = P_ij (dP_ij - sum_k P_ik dP_ik) with dP_ij
    the same for every j)."""
    rng = np.random.default_rng(24)
    B, H, N, d = 1, 2, 11, 6
    q, k, g = (rng.standard_normal((B, H, N, d)) for _ in range(3))
    v = np.broadcast_to(rng.standard_normal(d), (B, H, N, d)).copy()
    for causal in (False, True):
        dq, dk, dv = orc.attn_bwd(q, k, v, g, 0.6, causal)
        _close(dq, np.zeros_like(dq), 1e-13, "constant V: dQ")
        _close(dk, np.zeros_like(dk), 1e-13, "constant V: dK")
        assert np.max(np.abs(dv)) > 1e-2


def pin_bwd_sums(orc):
    """Rows of P sum to 1, so sum_j dV_j = sum_i dO_i; rows of dS sum to 0, so
    sum_j dK_j = 0 (both hold causal or not)."""
    rng = np.random.default_rng(25)
    B, H, N, d = 2, 2, 13, 5
    for causal in (False, True):
        q, k, v, g = (rng.standard_normal((B, H, N, d)) for _ in range(4))
        dq, dk, dv = orc.attn_bwd(q, k, v, g, 0.45, causal)
        _close(dv.sum(axis=2), g.sum(axis=2), 1e-12, "sum of dV rows")
        _close(dk.sum(axis=2), np.zeros((B, H, d)), 1e-12, "sum of dK rows")


def pin_bwd_closed_forms(orc):
    """Causal row 0 sees key 0 only: P_00 = 1, dS_0. = 0, so dQ_0 = 0 exactly.  Scale 0:
    dQ = dK = 0 exactly, and P is uniform over the allowed keys, so
    dV_j = sum_{i >= j} dO_i / (i + 1) (causal) or mean_i dO_i (not causal)."""
    rng = np.random.default_rng(26)
    B, H, N, d = 1, 1, 9, 4
    q, k, v, g = (rng.standard_normal((B, H, N, d)) for _ in range(4))
    dq, _, _ = orc.attn_bwd(q, k, v, g, 0.9, True)
    assert np.all(dq[0, 0, 0] == 0.0)
    for causal in (False, True):
        dq, dk, dv = orc.attn_bwd(q, k, v, g, 0.0, causal)
        assert np.all(dq == 0.0) and np.all(dk == 0.0)
        if causal:
            w = np.array([[1.0 / (i + 1) if j <= i else 0.0 for j in range(N)] for i in range(N)])
        else:
            w = np.full((N, N), 1.0 / N)
        _close(dv[0, 0], w.T @ g[0, 0], 1e-14, f"scale 0 dV causal={causal}")


def pin_bwd_torch_autograd(orc):
    """Cross-check with torch autograd through its CPU fp64 SDPA math path, an
    independent implementation of the same derivative ([PT] math backend)."""
    import torch
    import torch.nn.functional as F
    rng = np.random.default_rng(27)
    for (B, H, N, d) in [(1, 1, 1, 1), (2, 3, 7, 16), (1, 2, 40, 64)]:
        for causal in (False, True):
            q, k, v, g = (rng.standard_normal((B, H, N, d)) for _ in range(4))
            scale = 1.0 / math.sqrt(d)
            dq, dk, dv = orc.attn_bwd(q, k, v, g, scale, causal)
            tq, tk, tv = (torch.from_numpy(x.copy()).requires_grad_(True) for x in (q, k, v))
            out = F.scaled_dot_product_attention(tq, tk, tv, is_causal=causal, scale=scale)
            out.backward(torch.from_numpy(g))
            for mine, ref, name in ((dq, tq.grad, "dQ"), (dk, tk.grad, "dK"), (dv, tv.grad, "dV")):
                _close(mine, ref.numpy(), 1e-12, f"autograd {name} {B,H,N,d,causal}")


def pin_bwd_heads_independent(orc):
    """A batched backward equals per-head backward calls."""
    rng = np.random.default_rng(28)
    B, H, N, d = 2, 2, 8, 3
    q, k, v, g = rng.standard_normal((4, B, H, N, d))
    dq, dk, dv = orc.attn_bwd(q, k, v, g, 0.5, True)
    for b in range(B):
        for hh in range(H):
            one = orc.attn_bwd(q[b:b + 1, hh:hh + 1], k[b:b + 1, hh:hh + 1], v[b:b + 1, hh:hh + 1],
                               g[b:b + 1, hh:hh + 1], 0.5, True)
            for full, part in zip((dq, dk, dv), one):
                assert np.array_equal(full[b, hh], part[0, 0])


# ---------------------------------------------------------------- general masks

def pin_masked_reduces_to_plain(orc):
    """No mask and Nq = Nk: the same numbers as the plain (pinned) forward."""
    rng = np.random.default_rng(40)
    for causal in (False, True):
        q, k, v = rng.standard_normal((3, 2, 3, 9, 5))
        o, lse = orc.attn_masked(q, k, v, 0.4, causal)
        o2, lse2 = orc.attn_fwd(q, k, v, 0.4, causal)
        _close(o, o2, 1e-15, f"no mask O causal={causal}")
        _close(lse, lse2, 1e-15, f"no mask lse causal={causal}")


def pin_masked_tril_is_causal(orc):
    """A boolean lower-triangle mask ([PT] 构建因果掩码: ones -> tril) and the equivalent
    additive 0 / -inf bias both equal the plain causal forward."""
    rng = np.random.default_rng(41)
    q, k, v = rng.standard_normal((3, 2, 2, 10, 4))
    tril = np.tril(np.ones((10, 10), dtype=np.uint8))[None, None]
    o_ref, lse_ref = orc.attn_fwd(q, k, v, 0.7, True)
    o, lse = orc.attn_masked(q, k, v, 0.7, False, tril, "bool")
    _close(o, o_ref, 1e-15, "tril bool O")
    _close(lse, lse_ref, 1e-15, "tril bool lse")
    bias = np.where(tril != 0, 0.0, -np.inf)
    o, lse = orc.attn_masked(q, k, v, 0.7, False, bias, "add")
    _close(o, o_ref, 1e-15, "tril additive O")
    _close(lse, lse_ref, 1e-15, "tril additive lse")


def pin_masked_bottom_right(orc):
    """Nq < Nk, causal: the Nq queries are the last Nq positions, so they equal the last
    Nq rows of the square causal problem whose earlier query rows are arbitrary.
    Nq > Nk: the first Nq - Nk queries see no key (o = 0, lse = -inf) and the last Nk
    rows equal the square causal problem on them."""
    rng = np.random.default_rng(42)
    B, H, d = 1, 2, 6
    for Nq, Nk in ((1, 9), (4, 11), (11, 11)):
        q_full, k, v = rng.standard_normal((3, B, H, Nk, d))
        q = q_full[:, :, Nk - Nq:]
        o_ref, lse_ref = orc.attn_fwd(q_full, k, v, 0.5, True)
        o, lse = orc.attn_masked(q, k, v, 0.5, True)
        _close(o, o_ref[:, :, Nk - Nq:], 1e-15, f"bottom-right O {Nq, Nk}")
        _close(lse, lse_ref[:, :, Nk - Nq:], 1e-15, f"bottom-right lse {Nq, Nk}")
    Nq, Nk = 7, 3
    q = rng.standard_normal((B, H, Nq, d))
    k, v = rng.standard_normal((2, B, H, Nk, d))
    o, lse = orc.attn_masked(q, k, v, 0.5, True)
    assert np.all(o[:, :, :Nq - Nk] == 0.0) and np.all(lse[:, :, :Nq - Nk] == -np.inf)
    o_ref, lse_ref = orc.attn_fwd(q[:, :, Nq - Nk:], k, v, 0.5, True)
    _close(o[:, :, Nq - Nk:], o_ref, 1e-15, "Nq > Nk O")
    _close(lse[:, :, Nq - Nk:], lse_ref, 1e-15, "Nq > Nk lse")


def pin_masked_safe_softmax(orc):
    """[PT] 安全 softmax: a row with every key hidden gives o = 0 and lse = -inf exactly
    (no NaN); the other rows equal the problem without those rows."""
    rng = np.random.default_rng(43)
    B, H, Nq, Nk, d = 1, 2, 6, 8, 5
    q = rng.standard_normal((B, H, Nq, d))
    k, v = rng.standard_normal((2, B, H, Nk, d))
    mask = rng.random((B, H, Nq, Nk)) < 0.6
    mask[:, :, [1, 4]] = False
    mask[:, :, [0, 2, 3, 5], 0] = True
    o, lse = orc.attn_masked(q, k, v, 0.8, False, mask, "bool")
    assert np.all(o[:, :, [1, 4]] == 0.0) and np.all(lse[:, :, [1, 4]] == -np.inf)
    keep = [0, 2, 3, 5]
    o2, lse2 = orc.attn_masked(q[:, :, keep], k, v, 0.8, False, mask[:, :, keep], "bool")
    _close(o[:, :, keep], o2, 1e-15, "unmasked rows O")
    _close(lse[:, :, keep], lse2, 1e-15, "unmasked rows lse")
    assert np.isfinite(o).all()


def pin_masked_single_key(orc):
    """One visible key per row: the softmax weight is exactly 1, so o_i = v_j and
    lse_i = scale q_i . k_j + bias_ij."""
    rng = np.random.default_rng(44)
    B, H, Nq, Nk, d = 1, 1, 5, 7, 3
    q = rng.integers(-3, 4, (B, H, Nq, d)).astype(np.float64)
    k, v = rng.integers(-3, 4, (2, B, H, Nk, d)).astype(np.float64)
    pick = rng.integers(0, Nk, Nq)
    bias = np.full((1, 1, Nq, Nk), -np.inf)
    bias[0, 0, np.arange(Nq), pick] = 0.25 * np.arange(Nq)
    o, lse = orc.attn_masked(q, k, v, 0.5, False, bias, "add")
    for i, j in enumerate(pick):
        assert np.array_equal(o[0, 0, i], v[0, 0, j])
        assert lse[0, 0, i] == 0.5 * float(q[0, 0, i] @ k[0, 0, j]) + 0.25 * i


def pin_masked_row_constant_bias(orc):
    """A finite bias constant along each row leaves P and O unchanged ([FA] 数值稳定的
    Softmax: shift invariance) and adds the constant to lse."""
    rng = np.random.default_rng(45)
    B, H, Nq, Nk, d = 2, 2, 5, 9, 4
    q = rng.standard_normal((B, H, Nq, d))
    k, v = rng.standard_normal((2, B, H, Nk, d))
    c = rng.standard_normal((B, H, Nq, 1)) * 3
    for causal in (False, True):
        o, lse = orc.attn_masked(q, k, v, 0.6, causal, np.broadcast_to(c, (B, H, Nq, Nk)), "add")
        o2, lse2 = orc.attn_masked(q, k, v, 0.6, causal)
        _close(o, o2, 1e-13, f"row bias O causal={causal}")
        _close(lse, lse2 + c[..., 0], 1e-13, f"row bias lse causal={causal}")


def pin_masked_broadcast(orc):
    """A mask shared over batches or heads equals the same mask repeated."""
    rng = np.random.default_rng(46)
    B, H, Nq, Nk, d = 2, 3, 4, 6, 5
    q = rng.standard_normal((B, H, Nq, d))
    k, v = rng.standard_normal((2, B, H, Nk, d))
    for shape in ((1, 1), (B, 1), (1, H)):
        m = rng.standard_normal(shape + (Nq, Nk))
        o, lse = orc.attn_masked(q, k, v, 0.3, True, m, "add")
        o2, lse2 = orc.attn_masked(q, k, v, 0.3, True, np.broadcast_to(m, (B, H, Nq, Nk)).copy(), "add")
        assert np.array_equal(o, o2) and np.array_equal(lse, lse2)
    mb = rng.standard_normal((B, 1, Nq, Nk))
    mh = rng.standard_normal((1, H, Nq, Nk))
    o, _ = orc.attn_masked(q, k, v, 0.3, False, mb, "add")
    o2, _ = orc.attn_masked(q, k, v, 0.3, False, mh, "add")
    assert np.max(np.abs(o - o2)) > 1e-3


def pin_masked_torch_sdpa(orc):
    """torch's CPU fp64 SDPA with a boolean or float attn_mask and torch.logsumexp of the
    biased scores ([PT] math backend; its bool mask marks the keys that take part)."""
    import torch
    import torch.nn.functional as F
    rng = np.random.default_rng(47)
    for (B, H, Nq, Nk, d) in [(1, 1, 1, 5, 8), (2, 2, 9, 13, 16), (1, 2, 33, 20, 64)]:
        q = rng.standard_normal((B, H, Nq, d))
        k, v = rng.standard_normal((2, B, H, Nk, d))
        mb = rng.random((B, H, Nq, Nk)) < 0.7
        mb[..., rng.integers(0, Nk)] = True
        bias = rng.standard_normal((1, H, Nq, Nk))
        scale = 1.0 / math.sqrt(d)
        tq, tk, tv = (torch.from_numpy(x) for x in (q, k, v))
        s = torch.matmul(tq, tk.transpose(-1, -2)) * scale
        for kind, m, tm, sb in (("bool", mb, torch.from_numpy(mb), s.masked_fill(~torch.from_numpy(mb), float("-inf"))),
                                ("add", bias, torch.from_numpy(bias), s + torch.from_numpy(bias))):
            o, lse = orc.attn_masked(q, k, v, scale, False, m, kind)
            ref = F.scaled_dot_product_attention(tq, tk, tv, attn_mask=tm, scale=scale)
            _close(o, ref.numpy(), 1e-12, f"sdpa masked O {kind} {B,H,Nq,Nk,d}")
            _close(lse, torch.logsumexp(sb, dim=-1).numpy(), 1e-12, f"sdpa masked lse {kind}")


# ---------------------------------------------------------------- causal linear attention
# (hqwc.cn notes on the fast-transformers kernels, sections 0x0-0x2)

def _lin_recurrence(q, k, v, feature_map, eps):
    """The running-state form the page's CPU code uses (a separately written route):
    S += k_t v_t^T, z += k_t, then out_t = q_t S (/ (q_t . z + eps))."""
    phi = (lambda x: np.where(x > 0, x + 1.0, np.exp(np.minimum(x, 0.0)))) if feature_map else (lambda x: x)
    q, k = phi(q), phi(k)
    B, H, N, E = q.shape
    M = v.shape[3]
    out = np.empty((B, H, N, M))
    for b in range(B):
        for h in range(H):
            S = np.zeros((E, M))
            z = np.zeros(E)
            for t in range(N):
                S += np.outer(k[b, h, t], v[b, h, t])
                z += k[b, h, t]
                o = q[b, h, t] @ S
                out[b, h, t] = o / (q[b, h, t] @ z + eps) if feature_map else o
    return out


def pin_linear_recurrence(orc):
    """The definition (oracle) equals the running-state recurrence (page section 0x2's CPU
    loop: outer product into the state, then the query times the state), both forms."""
    rng = np.random.default_rng(61)
    for (B, H, N, E, M) in [(1, 1, 1, 3, 2), (2, 3, 17, 8, 5), (1, 2, 40, 16, 32)]:
        q, k = rng.standard_normal((2, B, H, N, E))
        v = rng.standard_normal((B, H, N, M))
        for fm in (False, True):
            _close(orc.linear_attn(q, k, v, fm, 1e-6), _lin_recurrence(q, k, v, fm, 1e-6), 1e-11,
                   f"linear recurrence fm={fm} {B,H,N,E,M}")


def pin_linear_torch_einsum(orc):
    """torch CPU fp64 with the page's module written as library calls: Z = 1/(einsum(Q,
    K.cumsum) + eps), the causal product as tril(Q K^T) V, phi = F.elu + 1."""
    import torch
    import torch.nn.functional as F
    rng = np.random.default_rng(62)
    B, H, N, E, M = 2, 2, 33, 16, 24
    q, k = rng.standard_normal((2, B, H, N, E))
    v = rng.standard_normal((B, H, N, M))
    tq, tk, tv = (torch.from_numpy(x) for x in (q, k, v))
    fq, fk = F.elu(tq) + 1, F.elu(tk) + 1
    prod = torch.matmul(torch.tril(torch.matmul(fq, fk.transpose(-1, -2))), tv)
    z = 1.0 / (torch.einsum("bhle,bhle->bhl", fq, fk.cumsum(2)) + 1e-6)
    _close(orc.linear_attn(q, k, v, True, 1e-6), (prod * z[..., None]).numpy(), 1e-12, "linear torch module")
    raw = torch.matmul(torch.tril(torch.matmul(tq, tk.transpose(-1, -2))), tv)
    _close(orc.linear_attn(q, k, v, False), raw.numpy(), 1e-12, "linear torch product")


def pin_linear_closed_forms(orc):
    """Row 0 sees key 0 alone: raw out_0 = (q_0 . k_0) v_0; with the feature map
    out_0 = s v_0 / (s + eps), s = phi(q_0) . phi(k_0).  phi(x) = x + 1 for x > 0 and
    e^x for x <= 0 (elu(x) = e^x - 1 there)."""
    q = np.array([[[[0.5, -1.0]]]])
    k = np.array([[[[2.0, -0.25]]]])
    v = np.array([[[[3.0, -1.0, 0.5]]]])
    s_raw = 0.5 * 2.0 + (-1.0) * (-0.25)
    _close(orc.linear_attn(q, k, v, False)[0, 0, 0], s_raw * v[0, 0, 0], 1e-15, "raw row 0")
    s = (0.5 + 1.0) * (2.0 + 1.0) + math.exp(-1.0) * math.exp(-0.25)
    _close(orc.linear_attn(q, k, v, True, 1e-6)[0, 0, 0], s * v[0, 0, 0] / (s + 1e-6), 1e-15, "phi row 0")


def pin_linear_constant_values(orc):
    """Constant values c: every output row is c * S / (S + eps) with S = phi(q_j) . sum
    phi(k_t) > 0, i.e. c up to eps; and eps = 0 gives c exactly (normalised weights)."""
    rng = np.random.default_rng(63)
    q, k = rng.standard_normal((2, 1, 2, 50, 8))
    v = np.full((1, 2, 50, 5), 0.75)
    _close(orc.linear_attn(q, k, v, True, 0.0), v, 1e-14, "constant values, eps 0")
    out = orc.linear_attn(q, k, v, True, 1e-6)
    assert np.all(out <= 0.75) and np.all(out > 0.75 * (1 - 1e-4)), "constant values, eps 1e-6"


def pin_linear_causal_prefix(orc):
    """Row j depends on tokens 0..j only: truncating the sequence after row j, or
    changing later tokens, leaves rows 0..j unchanged (bit for bit)."""
    rng = np.random.default_rng(64)
    q, k = rng.standard_normal((2, 1, 1, 30, 6))
    v = rng.standard_normal((1, 1, 30, 4))
    full = orc.linear_attn(q, k, v, True)
    pre = orc.linear_attn(q[:, :, :12], k[:, :, :12], v[:, :, :12], True)
    assert np.array_equal(full[:, :, :12], pre), "causal prefix"
    k2, v2 = k.copy(), v.copy()
    k2[:, :, 12:] += 5.0
    v2[:, :, 12:] -= 3.0
    assert np.array_equal(orc.linear_attn(q, k2, v2, True)[:, :, :12], full[:, :, :12]), "later tokens"
    assert np.max(np.abs(orc.linear_attn(q, k2, v2, True)[:, :, 12:] - full[:, :, 12:])) > 1e-3


def pin_linear_brute_force_integers(orc):
    """Small integer inputs: the raw product is exact in fp64 and equals a pure-Python
    triple loop bit for bit."""
    rng = np.random.default_rng(65)
    q = rng.integers(-3, 4, (1, 2, 7, 3)).astype(np.float64)
    k = rng.integers(-3, 4, (1, 2, 7, 3)).astype(np.float64)
    v = rng.integers(-3, 4, (1, 2, 7, 2)).astype(np.float64)
    out = orc.linear_attn(q, k, v, False)
    for h in range(2):
        for j in range(7):
            for m in range(2):
                want = sum(sum(q[0, h, j, e] * k[0, h, t, e] for e in range(3)) * v[0, h, t, m]
                           for t in range(j + 1))
                assert out[0, h, j, m] == want, f"integer brute force h={h} j={j} m={m}"


def pin_linear_heads_independent(orc):
    """Each (batch, head) is its own sequence: computing one head alone gives its rows."""
    rng = np.random.default_rng(66)
    q, k = rng.standard_normal((2, 2, 3, 9, 4))
    v = rng.standard_normal((2, 3, 9, 5))
    full = orc.linear_attn(q, k, v, True)
    for (b, h) in [(0, 0), (1, 2), (0, 1)]:
        one = orc.linear_attn(q[b:b + 1, h:h + 1], k[b:b + 1, h:h + 1], v[b:b + 1, h:h + 1], True)
        assert np.array_equal(one[0, 0], full[b, h]), f"head {b},{h}"


def pin_linear_linear_in_values(orc):
    """The output is linear in V: out(a V1 + V2) = a out(V1) + out(V2)."""
    rng = np.random.default_rng(67)
    q, k = rng.standard_normal((2, 1, 1, 20, 6))
    v1, v2 = rng.standard_normal((2, 1, 1, 20, 3))
    lhs = orc.linear_attn(q, k, 2.5 * v1 + v2, True)
    rhs = 2.5 * orc.linear_attn(q, k, v1, True) + orc.linear_attn(q, k, v2, True)
    _close(lhs, rhs, 1e-12, "linear in V")


ALL_PINS = [v for n, v in sorted(globals().items()) if n.startswith("pin_")]
