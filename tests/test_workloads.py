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


def test_unequal_lengths_generator():
    from exact_attention_96_amd.workloads import random_qkv_lens
    q, k, v = random_qkv_lens(2, 3, 17, 40, 64, "f16", seed=9)
    assert q.shape == (2, 3, 17, 64) and k.shape == v.shape == (2, 3, 40, 64)
    assert q.dtype == torch.float16
    q2, k2, v2 = random_qkv_lens(2, 3, 17, 40, 64, "f16", seed=9)
    assert torch.equal(q, q2) and torch.equal(k, k2) and torch.equal(v, v2)


def test_mask_patterns():
    """Each pattern is a contiguous bool [Bm, Hm, Nq, Nk] with the structure it names."""
    from exact_attention_96_amd.workloads import random_mask
    Nq, Nk = 100, 300
    shapes = (2, 3, Nq, Nk)
    for kind, kw in (("bernoulli", dict(p=0.3)), ("window", dict(w=50)), ("padding", {}),
                     ("blocks", dict(p=0.5)), ("empty_rows", {})):
        m = random_mask(kind, 2, 3, Nq, Nk, seed=1, **kw)
        assert m.shape == shapes and m.dtype == torch.bool and m.is_contiguous(), kind
        assert torch.equal(m, random_mask(kind, 2, 3, Nq, Nk, seed=1, **kw)), kind  # seeded
    # window: key j visible to query i iff i + Nk - Nq - w < j <= i + Nk - Nq
    m = random_mask("window", 1, 1, Nq, Nk, seed=0, w=50)[0, 0]
    i, j = 10, 10 + Nk - Nq
    assert m[i, j] and m[i, j - 49] and not m[i, j - 50] and not m[i, j + 1]
    assert int(m.sum(dim=1).max()) == 50
    # padding: a key prefix per (b, h), the same for every query
    m = random_mask("padding", 2, 3, Nq, Nk, seed=2)
    lens = m[:, :, 0].sum(-1)
    assert (lens >= 1).all() and torch.equal(m, m[:, :, :1].expand_as(m))
    assert torch.equal(m[..., 0, :], torch.arange(Nk).view(1, 1, Nk) < lens[..., None])
    # blocks: constant on 64 x 64 blocks
    m = random_mask("blocks", 1, 1, 128, 128, seed=3, p=0.5)[0, 0]
    assert torch.equal(m[:64, :64], m[0, 0].expand(64, 64))
    # empty rows: some rows see no key at all
    m = random_mask("empty_rows", 1, 1, 400, 300, seed=4)[0, 0]
    assert int((m.sum(1) == 0).sum()) > 0


def test_masked_and_linear_workloads():
    from exact_attention_96_amd.workloads import LINEAR_WORKLOADS, MASKED_WORKLOADS
    m1 = MASKED_WORKLOADS["m1"]
    assert (m1.B, m1.H, m1.Nq, m1.Nk, m1.d, m1.dtype, m1.causal) == (2, 32, 8192, 8192, 128, "bf16", False)
    m3 = MASKED_WORKLOADS["m3"]
    assert m3.mask_kind is None and m3.causal and (m3.Nq, m3.Nk) == (2048, 8192)
    l1 = LINEAR_WORKLOADS["l1"]
    assert l1.io_bytes == 4 * 2 * 32 * 8192 * (2 * 64 + 2 * 64)
    assert l1.flops == 2 * 32 * 8192 * (4.0 * 64 * 64 + 3.0 * 64)
    small = l1.__class__("t", 1, 2, 33, 16, 32, seed=5)
    q, k, v = small.inputs()
    assert q.shape == k.shape == (1, 2, 33, 16) and v.shape == (1, 2, 33, 32) and q.dtype == torch.float32
