"""GPU parity of attn_linear_fwd (causal linear attention, fp32) against the fp64
oracle (oracle.linear_attn), through the C ABI.

Bar (written here; a first-order rounding bound of the GPU's evaluation order,
u = 2^-24).  The kernel carries the state S_j = sum_{t<=j} k_t v_t^T in fp32 in token
order (j + 1 rounded additions) and reads out q_j . S_j with at most E more, so for the
causal dot product
    |o - o*|_jm <= (j + E + 2) u A_jm,   A_jm = sum_e |q_je| sum_{t<=j} |k_te| |v_tm|
(A from the oracle on |q|, |k|, |v|).  With the feature map, phi(q), phi(k) carry at
most 2 u of their own (expf within 2 ulp, x + 1 one rounding), the denominator is a sum
of positive terms (relative error <= (j + E + 6) u) and the division adds u:
    |o - o*|_jm <= (j + E + 8) u (A_jm / den_j + |o*_jm|),
A and den from the oracle on phi(q), phi(k) (phi evaluated in fp64 here).
The chunked form (a workspace) sums a chunk of at most 64 tokens, then the chunk
sums over the chunks, then adds the in-chunk products (a 64-term sum of E-term
products), so it gets 2 * 64 more rounded additions in the same bound.
Both forms run on every case.
"""
import numpy as np
import pytest
import torch

import exact_attention_96_amd as ea
import oracle
from parity_util import say

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
U = 2.0 ** -24


@pytest.fixture(scope="module", autouse=True)
def gpu():
    assert torch.cuda.is_available(), "these tests need an MI355X"
    assert torch.cuda.get_device_properties(0).gcnArchName.startswith("gfx950")


def inputs(B, H, N, E, M, seed, std=1.0):
    g = torch.Generator().manual_seed(seed)
    q = torch.randn((B, H, N, E), generator=g) * std
    k = torch.randn((B, H, N, E), generator=g) * std
    v = torch.randn((B, H, N, M), generator=g)
    return q, k, v


def phi64(x):
    x = np.asarray(x, dtype=np.float64)
    return np.where(x > 0, x + 1.0, np.exp(np.minimum(x, 0.0)))


def bound(q, k, v, fm, eps, o_ref, chunked):
    N, E = q.shape[2], q.shape[3]
    j = np.arange(N, dtype=np.float64).reshape(1, 1, N, 1) + (128 if chunked else 0)
    if not fm:
        A = oracle.linear_attn(np.abs(q.double().numpy()), np.abs(k.double().numpy()),
                               np.abs(v.double().numpy()), False)
        return (j + E + 2) * U * A
    fq, fk = phi64(q), phi64(k)
    A = oracle.linear_attn(fq, fk, np.abs(v.double().numpy()), False)
    den = np.einsum("bhne,bhne->bhn", fq, np.cumsum(fk, axis=2))[..., None] + eps
    return (j + E + 8) * U * (A / den + np.abs(o_ref))


def check(q, k, v, fm, eps, what, chunked=True):
    say(f"[linear] {what}: q={tuple(q.shape)} v={tuple(v.shape)} feature_map={fm} chunked={chunked}")
    o = ea.attn_linear_fwd(q.to(DEV), k.to(DEV), v.to(DEV), feature_map=fm, eps=eps, chunked=chunked)
    torch.cuda.synchronize()
    o = o.cpu().double().numpy()
    o_ref = oracle.linear_attn(q, k, v, fm, eps)
    err = np.abs(o - o_ref)
    bar = bound(q, k, v, fm, eps, o_ref, chunked)
    ratio = float((err / bar).max())
    say(f"[linear]   max err {err.max():.3e}, max err / bound {ratio:.4f}")
    assert np.isfinite(o).all(), f"{what}: non-finite output"
    assert ratio <= 1.0, f"{what}: error {ratio:.3f} x the bound"
    return o, o_ref, err


SHAPES = [(1, 1, 1, 16, 16), (1, 2, 31, 32, 16), (2, 2, 100, 64, 64), (1, 3, 257, 128, 32),
          (2, 1, 1000, 64, 48), (1, 1, 33, 16, 128), (1, 2, 700, 128, 64), (1, 1, 129, 32, 80),
          (1, 2, 64, 128, 128)]


@pytest.mark.parametrize("chunked", [True, False], ids=["chunked", "scan"])
@pytest.mark.parametrize("fm", [False, True])
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_shapes(shape, fm, chunked):
    q, k, v = inputs(*shape, seed=sum(shape))
    check(q, k, v, fm, 1e-6, f"shape {shape}", chunked)


@pytest.mark.parametrize("chunked", [True, False], ids=["chunked", "scan"])
def test_normalised_output_accuracy(chunked):
    """With the feature map the output is a weighted mean of values: at N = 2048 its
    error stays within the fp32 bar used for softmax attention (1e-5)."""
    q, k, v = inputs(1, 2, 2048, 64, 64, seed=7)
    _, _, err = check(q, k, v, True, 1e-6, "N 2048 normalised", chunked)
    assert err.max() <= 1e-5


@pytest.mark.parametrize("chunked", [True, False], ids=["chunked", "scan"])
def test_wide_inputs(chunked):
    """Queries and keys scaled by 4: phi's exponential branch reaches e^-16 and its linear
    branch 17, so the weights span ~10 decades."""
    q, k, v = inputs(1, 2, 300, 64, 32, seed=8, std=4.0)
    check(q, k, v, True, 1e-6, "wide inputs", chunked)


def test_large_value_width():
    """E = 128 with M = 256: eight value-column blocks, four per wave, in the chunked
    matrix-core form."""
    q, k, v = inputs(1, 1, 200, 128, 256, seed=12)
    check(q, k, v, True, 1e-6, "E 128 M 256", True)


def test_lds_chunk_limit_falls_back_to_the_scan():
    """E = 16 with M = 512 does not fit the LDS chunk tiles of that width: the call with
    a workspace runs the scan and meets the scan's (tighter) bound."""
    q, k, v = inputs(1, 1, 200, 16, 512, seed=13)
    check(q, k, v, True, 1e-6, "E 16 M 512", False)
    o = ea.attn_linear_fwd(q.to(DEV), k.to(DEV), v.to(DEV), chunked=True).cpu()
    o_scan = ea.attn_linear_fwd(q.to(DEV), k.to(DEV), v.to(DEV), chunked=False).cpu()
    assert torch.equal(o, o_scan)


def test_constant_values_and_zero_queries():
    q, k, v = inputs(1, 1, 500, 32, 16, seed=9)
    v = torch.full_like(v, -1.25)
    o = ea.attn_linear_fwd(q.to(DEV), k.to(DEV), v.to(DEV), feature_map=True, eps=0.0).cpu()  # chunked
    assert torch.allclose(o, v, atol=2e-6, rtol=0)  # normalised weights of a constant
    o = ea.attn_linear_fwd(torch.zeros_like(q).to(DEV), k.to(DEV), v.to(DEV), feature_map=False).cpu()
    assert torch.equal(o, torch.zeros_like(o))       # q = 0: the product is exactly 0


@pytest.mark.parametrize("chunked", [True, False], ids=["chunked", "scan"])
def test_causal_prefix_and_determinism(chunked):
    q, k, v = inputs(2, 2, 600, 64, 32, seed=10)
    a = ea.attn_linear_fwd(q.to(DEV), k.to(DEV), v.to(DEV), chunked=chunked).cpu()
    b = ea.attn_linear_fwd(q.to(DEV), k.to(DEV), v.to(DEV), chunked=chunked).cpu()
    assert torch.equal(a, b)
    # a prefix of whole chunks (256 = 4 x 64) gives the same rows bit for bit in both forms
    pre = ea.attn_linear_fwd(q[:, :, :256].contiguous().to(DEV), k[:, :, :256].contiguous().to(DEV),
                             v[:, :, :256].contiguous().to(DEV), chunked=chunked).cpu()
    assert torch.equal(pre, a[:, :, :256])


@pytest.mark.parametrize("chunked", [True, False], ids=["chunked", "scan"])
def test_full_size_workload(chunked):
    """The benchmark shape (2 x 32 x 8192, E = M = 64, feature map): two heads in full
    against the oracle, in the benchmark's launch."""
    B, H, N, E, M = 2, 32, 8192, 64, 64
    q, k, v = inputs(B, H, N, E, M, seed=11)
    say(f"[linear] full size {(B, H, N, E, M)} chunked={chunked}")
    o = ea.attn_linear_fwd(q.to(DEV), k.to(DEV), v.to(DEV), chunked=chunked).cpu()
    assert torch.isfinite(o).all()
    for (b, h) in [(0, 0), (1, 31)]:
        sl = (slice(b, b + 1), slice(h, h + 1))
        o_ref = oracle.linear_attn(q[sl], k[sl], v[sl], True, 1e-6)
        err = np.abs(o[sl].double().numpy() - o_ref)
        bar = bound(q[sl], k[sl], v[sl], True, 1e-6, o_ref, chunked)
        say(f"[linear]   head ({b},{h}): max err {err.max():.3e}, max err / bound {(err / bar).max():.4f}")
        assert (err / bar).max() <= 1.0


# One-pass form (E and M in {32, 64} with a workspace): spans of 128 tokens, groups of 4
# spans; heads padded to a multiple of 8 on the grid.  These shapes cross groups (the
# inclusive-prefix chain), end in a ragged span, and pad the heads.
ONE_PASS = [(1, 3, 2500, 32, 64), (2, 5, 1100, 64, 32), (1, 1, 1025, 32, 32), (1, 2, 4096 + 7, 64, 64)]


@pytest.mark.parametrize("fm", [False, True])
@pytest.mark.parametrize("shape", ONE_PASS, ids=lambda s: "x".join(map(str, s)))
def test_one_pass_spans_and_groups(shape, fm):
    q, k, v = inputs(*shape, seed=sum(shape) + 3)
    check(q, k, v, fm, 1e-6, f"one-pass {shape}", True)


@pytest.mark.parametrize("shape", [(1, 1, 1, 32, 32), (1, 1, 127, 64, 32), (1, 1, 128, 32, 64),
                                   (1, 1, 129, 64, 64), (4, 64, 256, 64, 64)],
                         ids=lambda s: "x".join(map(str, s)))
def test_one_pass_edges(shape):
    """One token; one span short of, exactly and one past 128 tokens (a single span, then a
    ragged second one); and 256 heads of two spans (a grid of 512 workgroups, every head
    class full)."""
    q, k, v = inputs(*shape, seed=sum(shape) + 5)
    check(q, k, v, True, 1e-6, f"one-pass edge {shape}", True)


@pytest.mark.parametrize("fm", [False, True])
def test_one_pass_products_keep_fp32_accuracy(fm):
    """The one-pass form's products run on bf16 matrix cores from three-part splits of
    each fp32 operand.  Values on a large common offset (1000 + N(0, 1)) need all 24 bits
    of each operand: with two parts (16 bits) the normalised outputs, weighted means near
    1000, would be off by ~2^-16 of their size (1.5e-5); with three they stay at fp32 level
    (below 2e-6 relative, asserted) and within the fp32 bound.  Queries and keys at std 3
    widen the range of phi as well."""
    q, k, v = inputs(1, 2, 700, 64, 64, seed=31, std=3.0)
    v = v + 1000.0
    o, o_ref, err = check(q, k, v, fm, 1e-6, "one-pass, values offset by 1000", True)
    if fm:  # a weighted mean of values near 1000: fp32-level relative accuracy
        assert (err / np.abs(o_ref)).max() <= 2e-6


def test_one_pass_repeats_bitwise_and_ignores_stale_workspace():
    """The look-back reads earlier spans in a fixed order, so repeated calls give the same
    bits whatever their timing; a workspace left by another call (other sizes, other
    epochs) or filled with arbitrary bytes gives the same result as a fresh one."""
    B, H, N, E, M = 1, 3, 2500, 32, 64
    q, k, v = (t.to(DEV) for t in inputs(B, H, N, E, M, seed=21))
    n = ea.linear_workspace_bytes(B, H, N, E, M)
    ws = torch.zeros(n, dtype=torch.uint8, device=DEV)
    ref = ea.attn_linear_fwd(q, k, v, workspace=ws).cpu()
    for _ in range(3):
        assert torch.equal(ea.attn_linear_fwd(q, k, v, workspace=ws).cpu(), ref)
    # another problem on the same workspace, then this one again
    q2, k2, v2 = (t.to(DEV) for t in inputs(2, 2, 900, E, M, seed=22))
    ea.attn_linear_fwd(q2, k2, v2, workspace=ws[:ea.linear_workspace_bytes(2, 2, 900, E, M)])
    assert torch.equal(ea.attn_linear_fwd(q, k, v, workspace=ws).cpu(), ref)
    # arbitrary bytes
    g = torch.Generator(device="cpu").manual_seed(5)
    ws.copy_(torch.randint(0, 256, (n,), generator=g, dtype=torch.uint8).to(DEV))
    assert torch.equal(ea.attn_linear_fwd(q, k, v, workspace=ws).cpu(), ref)
    ws.fill_(0xFF)
    assert torch.equal(ea.attn_linear_fwd(q, k, v, workspace=ws).cpu(), ref)


def test_side_stream_and_caller_workspace():
    """Both forms on a side stream; the chunked one on a workspace the caller passes."""
    q, k, v = inputs(1, 2, 300, 32, 32, seed=13)
    o_ref = oracle.linear_attn(q, k, v, True, 1e-6)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        qd, kd, vd = (t.to(DEV) for t in (q, k, v))
        ws = torch.empty(ea.linear_workspace_bytes(1, 2, 300, 32, 32), dtype=torch.uint8, device=DEV)
        s.synchronize()
        a = ea.attn_linear_fwd(qd, kd, vd, workspace=ws)
        b = ea.attn_linear_fwd(qd, kd, vd, chunked=False)
    s.synchronize()
    for o, chunked in ((a, True), (b, False)):
        err = np.abs(o.cpu().double().numpy() - o_ref)
        assert (err / bound(q, k, v, True, 1e-6, o_ref, chunked)).max() <= 1.0


def test_binding_rejects_bad_arguments():
    q = torch.zeros(1, 1, 8, 64, device=DEV)
    with pytest.raises(ValueError):       # not float32
        ea.attn_linear_fwd(q.half(), q.half(), q.half())
    with pytest.raises(ValueError):       # k shaped differently from q
        ea.attn_linear_fwd(q, q[..., :32].contiguous(), q)
    with pytest.raises(ValueError):       # workspace too small
        ea.attn_linear_fwd(q, q, q, workspace=torch.empty(16, dtype=torch.uint8, device=DEV))
    with pytest.raises(ea.AttnError) as e:
        z = torch.zeros(1, 1, 8, 48, device=DEV)
        ea.attn_linear_fwd(z, z, z)
    assert e.value.status == ea.ATTN_EUNSUPPORTED
