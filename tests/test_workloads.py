"""Seeded input generators (host logic, CPU only)."""
import torch

from exact_attention_96_amd.workloads import WORKLOADS, make_inputs, random_qkv


def test_shapes_dtypes_and_determinism():
    for key in ("c1", "c4"):
        w = WORKLOADS[key]
        q, k, v = make_inputs(w)
        assert q.shape == k.shape == v.shape == (w.B, w.H, w.N, w.d)
        assert q.dtype == w.torch_dtype and q.is_contiguous()
        q2, k2, v2 = make_inputs(w)
        assert torch.equal(q, q2) and torch.equal(k, k2) and torch.equal(v, v2)
        q3, _, _ = make_inputs(w, seed=w.seed + 100)
        assert not torch.equal(q, q3)


def test_spiky_rows():
    w = WORKLOADS["c4"]
    _, k, _ = make_inputs(w)
    rows = k.float().reshape(-1, w.d).abs().amax(dim=1)
    n_spiky = round(0.01 * w.B * w.H * w.N)
    assert n_spiky == 1311
    # std 0.5 rows essentially never exceed 4 in magnitude; spiky rows are x8
    big = int((rows > 4.5).sum())
    assert n_spiky * 0.9 <= big <= n_spiky


def test_flop_and_byte_counts():
    w = WORKLOADS["c3"]
    assert w.flops == 4 * 2 * 32 * 8192 * 8192 * 128 / 2
    assert w.io_bytes == 4 * 2 * 32 * 8192 * 128 * 2 + 4 * 2 * 32 * 8192
    assert abs(w.scale - 0.08838834764831845) < 1e-8


def test_random_qkv():
    q, k, v = random_qkv(1, 2, 33, 64, "bf16", seed=5)
    assert q.dtype == torch.bfloat16 and q.shape == (1, 2, 33, 64)
