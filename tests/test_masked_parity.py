"""GPU parity of attn_fwd_masked (unequal query/key lengths, boolean masks) and
attn_mask_pack against the fp64 oracle's general-mask form, through the C ABI.

The oracle (oracle.attn_masked) applies the mask as an additive 0 / -inf bias after
scaling, anchors the causal triangle at the bottom-right corner (key j visible to
query i iff j <= i + Nk - Nq) and gives a row that sees no key o = 0, lse = -inf.
Such rows must come back exactly so from the GPU; every other row meets the bars
of parity_util.TOL.
"""
import numpy as np
import pytest
import torch

import exact_attention_96_amd as ea
import oracle
from exact_attention_96_amd.workloads import WORKLOADS, make_inputs, random_mask, random_qkv_lens
from parity_util import check, errors, sample_rows, say

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.fixture(scope="module", autouse=True)
def gpu():
    assert torch.cuda.is_available(), "these tests need an MI355X"
    assert torch.cuda.get_device_properties(0).gcnArchName.startswith("gfx950")


def run(q, k, v, mask, causal, scale):
    qd, kd, vd = (t.to(DEV) for t in (q, k, v))
    md = None if mask is None else mask.to(DEV)
    o, lse = ea.attn_fwd_masked(qd, kd, vd, mask=md, causal=causal, scale=scale)
    torch.cuda.synchronize()
    return o.float().cpu().numpy(), lse.cpu().numpy()


def compare(o, lse, o_ref, lse_ref, dtype, what):
    """Rows the oracle leaves empty must be exactly 0 / -inf; the rest meet the bars."""
    empty = np.isneginf(lse_ref)
    assert np.isneginf(lse[empty]).all(), f"{what}: an empty row has a finite lse"
    assert (o[empty] == 0).all(), f"{what}: an empty row has a nonzero output"
    live = ~empty
    if live.any():
        err = errors(o[live], lse[live], o_ref[live], lse_ref[live])
        check(err, dtype, what)


def parity(q, k, v, mask, causal, scale, dtype, what):
    say(f"[masked] {what}: q={tuple(q.shape)} k={tuple(k.shape)} dtype={dtype} causal={causal} "
        f"mask={None if mask is None else tuple(mask.shape)}")
    o, lse = run(q, k, v, mask, causal, scale)
    o_ref, lse_ref = oracle.attn_masked(q, k, v, scale, causal, mask)
    compare(o, lse, o_ref, lse_ref, dtype, what)
    return o, lse


# (Nq, Nk): equal, Nq < Nk with offsets that are and are not multiples of 32 (the
# diagonal of a wave's 32 rows then crosses a 64-key unit), Nq > Nk (the first
# Nq - Nk causal rows see no key), single rows, ragged tails.
LENGTHS = [(1, 1), (1, 300), (65, 64), (100, 300), (128, 256), (256, 288), (300, 1000),
           (513, 129), (1000, 333), (777, 777)]
KINDS = [("bf16", 128), ("bf16", 64), ("f16", 64), ("f16", 128), ("f32", 64)]


@pytest.mark.parametrize("kind", KINDS, ids=lambda t: f"{t[0]}-d{t[1]}")
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("lens", LENGTHS, ids=lambda t: f"nq{t[0]}-nk{t[1]}")
def test_lengths(lens, causal, kind):
    Nq, Nk = lens
    dtype, d = kind
    q, k, v = random_qkv_lens(1, 2, Nq, Nk, d, dtype, seed=Nq * 7 + Nk)
    parity(q, k, v, None, causal, float(np.float32(d ** -0.5)), dtype, f"lengths {Nq}x{Nk}")


MASKS = [("bernoulli", dict(p=0.5)), ("bernoulli", dict(p=0.03)), ("window", dict(w=100)),
         ("padding", {}), ("blocks", dict(p=0.3)), ("empty_rows", {})]


@pytest.mark.parametrize("kind", [("bf16", 128), ("f16", 64), ("f32", 128)], ids=lambda t: f"{t[0]}-d{t[1]}")
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("mk", MASKS, ids=lambda t: t[0] + "".join(f"-{k}{v}" for k, v in t[1].items()))
def test_masks(mk, causal, kind):
    dtype, d = kind
    name, kw = mk
    B, H, Nq, Nk = 2, 3, 300, 389
    q, k, v = random_qkv_lens(B, H, Nq, Nk, d, dtype, seed=11)
    mask = random_mask(name, B, H, Nq, Nk, seed=12, **kw)
    parity(q, k, v, mask, causal, float(np.float32(d ** -0.5)), dtype, f"mask {name}")


@pytest.mark.parametrize("bm,hm", [(1, 1), (2, 1), (1, 3)])
def test_mask_broadcast(bm, hm):
    """A mask shared across the batch or the heads (word stride 0 on that axis)."""
    q, k, v = random_qkv_lens(2, 3, 200, 700, 128, "bf16", seed=21)
    mask = random_mask("bernoulli", bm, hm, 200, 700, seed=22, p=0.4)
    parity(q, k, v, mask, True, float(np.float32(128 ** -0.5)), "bf16", f"broadcast {bm}x{hm}")


def test_every_row_empty():
    q, k, v = random_qkv_lens(1, 2, 100, 100, 64, "bf16", seed=31)
    mask = torch.zeros((1, 1, 100, 100), dtype=torch.bool)
    o, lse = run(q, k, v, mask, False, 0.125)
    assert (o == 0).all() and np.isneginf(lse).all()


def test_spiky_keys_under_a_mask():
    """fp16 with 1 % of key rows scaled by 8 (the many-block short-sequence recipe):
    the running max jumps while some keys are hidden."""
    w = WORKLOADS["c4"].with_(B=2, H=4)
    q, k, v = make_inputs(w)
    mask = random_mask("bernoulli", 2, 1, w.N, w.N, seed=41, p=0.7)
    parity(q, k, v, mask, False, w.scale, "f16", "spiky keys, bernoulli mask")


def test_unmasked_equal_lengths_match_attn_fwd_bitwise():
    """Without a mask and with Nq = Nk the two entry points run the same kernel."""
    q, k, v = random_qkv_lens(2, 2, 1000, 1000, 128, "bf16", seed=51)
    qd, kd, vd = (t.to(DEV) for t in (q, k, v))
    for causal in (False, True):
        o1, l1 = ea.attn_fwd(qd, kd, vd, causal=causal)
        o2, l2 = ea.attn_fwd_masked(qd, kd, vd, causal=causal)
        torch.cuda.synchronize()
        assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_explicit_lower_triangle_matches_causal():
    """A materialised lower-triangle mask (the math backend's causal mask) gives the
    causal result: against the oracle, and within the bars of the causal kernel."""
    q, k, v = random_qkv_lens(1, 4, 777, 777, 128, "bf16", seed=61)
    tril = torch.ones((777, 777), dtype=torch.bool).tril().view(1, 1, 777, 777)
    o, lse = parity(q, k, v, tril, False, float(np.float32(128 ** -0.5)), "bf16", "explicit tril")
    o_ref, lse_ref = oracle.attn_fwd(q, k, v, float(np.float32(128 ** -0.5)), True)
    check(errors(o, lse, o_ref, lse_ref), "bf16", "explicit tril vs the causal oracle")


def test_deterministic():
    q, k, v = random_qkv_lens(2, 2, 300, 500, 64, "f16", seed=71)
    mask = random_mask("bernoulli", 1, 2, 300, 500, seed=72, p=0.5)
    a = run(q, k, v, mask, True, 0.125)
    b = run(q, k, v, mask, True, 0.125)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


@pytest.mark.parametrize("heads,rows,nk", [(1, 1, 1), (1, 3, 64), (2, 5, 65), (1, 7, 300), (3, 64, 1000),
                                           (2, 300, 200), (1, 513, 4200)])
def test_mask_pack_bits(heads, rows, nk):
    """attn_mask_pack against bit packing and tile summaries done on the host (bit-exact).
    Sparse masks, so that empty units and empty tiles occur."""
    g = torch.Generator().manual_seed(rows * 1000 + nk)
    m = torch.randint(0, 3, (heads, 1, rows, nk), generator=g, dtype=torch.uint8)  # 0, 1, 2 (nonzero = on)
    m *= (torch.rand((heads, 1, rows, nk), generator=g) < 0.002).to(torch.uint8)
    packed = ea.pack_mask(m.to(DEV))
    bits = packed.bits.cpu().numpy().view(np.uint64)
    tiles = packed.tiles.cpu().numpy().view(np.uint64)
    W = (nk + 63) // 64
    on = np.zeros((heads, rows, W * 64), dtype=np.uint64)
    on[:, :, :nk] = (m.numpy()[:, 0] != 0)
    want = np.zeros((heads, rows, W), dtype=np.uint64)
    for j in range(W * 64):
        want[:, :, j // 64] |= on[:, :, j] << np.uint64(j % 64)
    assert np.array_equal(bits[:, 0], want)
    nt, tw = (rows + 255) // 256, (W + 63) // 64
    unit_any = np.zeros((heads, nt, tw * 64), dtype=np.uint64)
    for t in range(nt):
        unit_any[:, t, :W] = (want[:, 256 * t:256 * t + 256] != 0).any(axis=1)
    want_t = np.zeros((heads, nt, tw), dtype=np.uint64)
    for u in range(tw * 64):
        want_t[:, :, u // 64] |= unit_any[:, :, u] << np.uint64(u % 64)
    assert np.array_equal(tiles[:, 0], want_t)


@pytest.mark.parametrize("kind,kw", [("blocks", dict(p=0.2)), ("window", dict(w=300)),
                                     ("bernoulli", dict(p=0.001)), ("padding", {})])
@pytest.mark.parametrize("causal", [False, True])
def test_unit_skipping_changes_nothing(kind, kw, causal):
    """With the tile summary the kernel skips units no row of a query tile sees; a
    skipped unit would only have added exact zeros, so the results are bitwise those
    of the same kernel walking every unit (and both match the oracle)."""
    q, k, v = random_qkv_lens(2, 2, 700, 1500, 128, "bf16", seed=81)
    mask = random_mask(kind, 2, 1, 700, 1500, seed=82, **kw)
    parity(q, k, v, mask, causal, float(np.float32(128 ** -0.5)), "bf16", f"skipping {kind}")
    qd, kd, vd = (t.to(DEV) for t in (q, k, v))
    packed = ea.pack_mask(mask.to(DEV))
    o1, l1 = ea.attn_fwd_masked(qd, kd, vd, mask_bits=packed, causal=causal)
    o2, l2 = ea.attn_fwd_masked(qd, kd, vd, mask_bits=packed.bits, causal=causal)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_full_size_sliding_window():
    """The headline shape (2 x 32 x 8192 x 128, bf16) with a causal sliding window of
    1024 keys given as a mask, in the benchmark's launch: sampled rows of three heads
    against the oracle, row by row."""
    w = WORKLOADS["c3"]
    q, k, v = make_inputs(w)
    N = w.N
    mask = random_mask("window", 1, 1, N, N, seed=0, w=1024)
    say(f"[masked] full size {tuple(q.shape)} window 1024")
    o, lse = run(q, k, v, mask, True, w.scale)
    rng = np.random.default_rng(5)
    for (b, h) in [(0, 0), (1, 31), (1, 7)]:
        rows = sample_rows(N, rng, n_random=24)
        sub = mask[:, :, rows]
        o_ref, lse_ref = oracle.attn_masked(q[b:b + 1, h:h + 1, rows], k[b:b + 1, h:h + 1],
                                            v[b:b + 1, h:h + 1], w.scale, False, sub)
        compare(o[b, h, rows], lse[b, h, rows], o_ref[0, 0], lse_ref[0, 0], "bf16",
                f"window head ({b},{h})")
    assert np.isfinite(o).all() and np.isfinite(lse).all()


@pytest.mark.parametrize("scale", [0.0, -0.2, 1.0])
@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("f16", 64), ("f32", 64)])
def test_masked_scales(scale, dtype, d):
    """Scale 0 (every visible key weighs the same: o is the mean of the visible values,
    lse the log of their count), a negative scale and a large one, under a mask."""
    q, k, v = random_qkv_lens(2, 2, 200, 333, d, dtype, seed=91)
    mask = random_mask("bernoulli", 1, 2, 200, 333, seed=92, p=0.3)
    parity(q, k, v, mask, True, scale, dtype, f"masked scale {scale}")


def test_side_stream():
    """attn_mask_pack and attn_fwd_masked on a side stream (torch's current stream there)."""
    q, k, v = random_qkv_lens(1, 3, 257, 500, 128, "f16", seed=101)
    mask = random_mask("bernoulli", 1, 1, 257, 500, seed=102, p=0.5)
    s = torch.cuda.Stream()
    say("[masked] f16 on a side stream")
    with torch.cuda.stream(s):
        qd, kd, vd, md = (t.to(DEV, non_blocking=False) for t in (q, k, v, mask))
        s.synchronize()
        o, lse = ea.attn_fwd_masked(qd, kd, vd, mask=md, causal=True, scale=0.0884)
    s.synchronize()
    o_ref, lse_ref = oracle.attn_masked(q, k, v, 0.0884, True, mask)
    compare(o.float().cpu().numpy(), lse.cpu().numpy(), o_ref, lse_ref, "f16", "side stream")


def test_binding_rejects_bad_arguments():
    q = torch.zeros(1, 2, 8, 64, device=DEV, dtype=torch.bfloat16)
    k = torch.zeros(1, 2, 12, 64, device=DEV, dtype=torch.bfloat16)
    with pytest.raises(ValueError):       # k and v of different lengths
        ea.attn_fwd_masked(q, k, k[:, :, :10])
    with pytest.raises(TypeError):        # mixed dtypes
        ea.attn_fwd_masked(q, k, k.half())
    with pytest.raises(ValueError):       # mask of the wrong shape
        ea.attn_fwd_masked(q, k, k, mask=torch.ones(1, 2, 8, 11, dtype=torch.bool, device=DEV))
    with pytest.raises(ValueError):       # mask and packed bits together
        m = torch.ones(1, 1, 8, 12, dtype=torch.bool, device=DEV)
        ea.attn_fwd_masked(q, k, k, mask=m, mask_bits=ea.pack_mask(m))
    with pytest.raises(TypeError):        # a float mask is not a boolean mask
        ea.pack_mask(torch.ones(1, 1, 8, 12, device=DEV))
    with pytest.raises(ea.AttnError) as e:
        z = torch.zeros(1, 1, 8, 96, device=DEV, dtype=torch.bfloat16)
        ea.attn_fwd_masked(z, z, z)
    assert e.value.status == ea.ATTN_EUNSUPPORTED
