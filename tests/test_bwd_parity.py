"""GPU parity of the backward (attn_bwd through the C ABI) against the fp64 oracle.

The GPU runs the forward and then the backward on seeded inputs; the oracle
computes the exact gradients of the same inputs (widened exactly to fp64).
Bars are derived in parity_util (row-relative, from the roundoff of the input
type, plus the dQ term from D formed with the rounded forward output).
"""
import math

import numpy as np
import pytest
import torch

import exact_attention_96_amd as ea
import oracle
from exact_attention_96_amd.workloads import WORKLOADS, make_inputs, random_grad, random_qkv
from parity_util import BWD_U, bwd_check, bwd_errors, dq_extra, say

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.fixture(scope="module", autouse=True)
def gpu():
    assert torch.cuda.is_available(), "these tests need an MI355X"
    name = torch.cuda.get_device_properties(0).gcnArchName
    assert name.startswith("gfx950"), f"built for gfx950, found {name}"


def f32(x: float) -> float:
    return float(np.float32(x))


def gpu_grads(q, k, v, do, causal, scale, delta=None):
    qd, kd, vd, dod = (t.to(DEV) for t in (q, k, v, do))
    o, lse = ea.attn_fwd(qd, kd, vd, causal=causal, scale=scale)
    dq, dk, dv = ea.attn_bwd(qd, kd, vd, o, lse, dod, causal=causal, scale=scale, delta=delta)
    torch.cuda.synchronize()
    return o, lse, dq, dk, dv


def bwd_parity(q, k, v, do, causal, scale, dtype, what):
    say(f"[bwd parity] {what}: shape={tuple(q.shape)} dtype={dtype} causal={causal} scale={scale}")
    _, _, dq, dk, dv = gpu_grads(q, k, v, do, causal, scale)
    ref = oracle.attn_bwd(q, k, v, do, scale, causal)
    u = BWD_U[dtype]
    extra = (dq_extra(q, k, v, do, scale, causal, u, oracle), None, None)
    out = {}
    for name, g, r, x in zip(("dq", "dk", "dv"), (dq, dk, dv), ref, extra):
        err = bwd_errors(g.float().cpu().numpy(), r, u, x)
        say(f"    {name}: {err['ratio']:.3f} x allowance, max {err['max_u']:.2f} u, mean "
            f"{err['mean']:.3f} u, abs_max {err['abs_max']:.3e}, rms {err['rms']:.3e}")
        bwd_check(err, f"{what} {name}")
        out[name] = err
    return out


CASES = [
    # (B, H, N, d, dtype, causal, seed): ragged N (not a multiple of 32 or 128), both head sizes
    (1, 2, 700, 128, "bf16", True, 11),
    (1, 2, 389, 128, "bf16", False, 12),
    (2, 2, 1000, 64, "bf16", True, 13),
    (1, 3, 256, 64, "bf16", False, 14),
    (1, 2, 513, 128, "f16", True, 15),
    (2, 2, 300, 64, "f16", False, 16),
    (1, 1, 1, 64, "bf16", True, 17),
    (1, 1, 2, 128, "bf16", True, 18),
    (1, 2, 33, 64, "f16", False, 19),
    (1, 1, 129, 128, "bf16", False, 20),
]


@pytest.mark.parametrize("B,H,N,d,dtype,causal,seed", CASES,
                         ids=[f"b{c[0]}h{c[1]}n{c[2]}d{c[3]}_{c[4]}_{'causal' if c[5] else 'full'}"
                              for c in CASES])
def test_bwd_shapes(B, H, N, d, dtype, causal, seed):
    q, k, v = random_qkv(B, H, N, d, dtype, seed)
    do = random_grad(B, H, N, d, dtype, seed + 1000)
    bwd_parity(q, k, v, do, causal, f32(1 / math.sqrt(d)), dtype, f"bwd {dtype} N={N} d={d}")


def test_bwd_causal_long_sequence_d64():
    """Two heads of the bf16 causal N=2048 d=64 workload at full length."""
    w = WORKLOADS["c2"].with_(B=1, H=2)
    q, k, v = make_inputs(w)
    do = random_grad(w.B, w.H, w.N, w.d, w.dtype, 2002)
    bwd_parity(q, k, v, do, True, w.scale, w.dtype, "bwd c2-shape heads")


def test_bwd_spiky_keys_f16():
    """The fp16 non-causal workload's recipe (std 0.5, 1% of K rows times 8), two heads."""
    w = WORKLOADS["c4"].with_(B=1, H=2)
    q, k, v = make_inputs(w)
    do = random_grad(w.B, w.H, w.N, w.d, w.dtype, 4004, std=0.5)
    bwd_parity(q, k, v, do, False, w.scale, w.dtype, "bwd c4-recipe heads")


def test_bwd_scale_not_default():
    q, k, v = random_qkv(1, 2, 200, 64, "bf16", 21, std=0.5)
    do = random_grad(1, 2, 200, 64, "bf16", 1021)
    bwd_parity(q, k, v, do, True, 0.3, "bf16", "bwd scale 0.3")


def test_bwd_delta_is_row_dot_of_do_and_o():
    """The workspace holds D_i = dO_i . O_i ("Understand FlashAttention", section
    "反向传播"), from the forward's rounded O: within 2u of sum |dO O*| of the exact O*."""
    B, H, N, d = 1, 2, 300, 128
    q, k, v = random_qkv(B, H, N, d, "bf16", 22)
    do = random_grad(B, H, N, d, "bf16", 1022)
    scale = f32(1 / math.sqrt(d))
    say(f"[bwd delta] shape={(B, H, N, d)}")
    delta = torch.empty((B, H, N), dtype=torch.float32, device=DEV)
    gpu_grads(q, k, v, do, True, scale, delta=delta)
    o_ref, _ = oracle.attn_fwd(q, k, v, scale, True)
    dof = do.double().numpy()
    D_ref = np.sum(dof * o_ref, axis=-1)
    bound = 2 * 2.0 ** -8 * np.sum(np.abs(dof * o_ref), axis=-1) + 1e-5
    err = np.abs(delta.cpu().numpy() - D_ref)
    assert (err <= bound).all(), f"max excess {(err - bound).max():.3e}"


def test_bwd_bitwise_reproducible():
    q, k, v = random_qkv(1, 2, 450, 128, "bf16", 23)
    do = random_grad(1, 2, 450, 128, "bf16", 1023)
    say("[bwd repro] b1h2n450d128 bf16 causal")
    a = gpu_grads(q, k, v, do, True, f32(1 / math.sqrt(128)))
    b = gpu_grads(q, k, v, do, True, f32(1 / math.sqrt(128)))
    for x, y in zip(a[2:], b[2:]):
        assert torch.equal(x, y)


def test_bwd_rejects_f32():
    x = torch.zeros((1, 1, 8, 64), dtype=torch.float32, device=DEV)
    lse = torch.zeros((1, 1, 8), dtype=torch.float32, device=DEV)
    with pytest.raises(ea.AttnError) as e:
        ea.attn_bwd(x, x, x, x, lse, x)
    assert e.value.status == ea.ATTN_EUNSUPPORTED
