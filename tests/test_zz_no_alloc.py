"""GPU: the backward entry point that allocates nothing (attn_bwd_noalloc, for
callers that cannot allocate device memory) against attn_bwd with a caller's
workspace, through the C ABI: two calls in a row, the second on a smaller
problem, each bitwise equal to attn_bwd on the same inputs (the same kernels run;
only where the per-row term D lives differs)."""
import math

import pytest
import torch

import exact_attention_96_amd as ea
from exact_attention_96_amd.workloads import random_grad, random_qkv
from parity_util import say

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.fixture(scope="module", autouse=True)
def gpu():
    assert torch.cuda.is_available(), "these tests need an MI355X"


CASES = [  # (B, H, N, d, dtype, causal, seed): the second is smaller than the first
    (2, 4, 1000, 128, "bf16", True, 61),
    (1, 3, 257, 64, "f16", False, 62),
]


def test_noalloc_backward_matches_attn_bwd():
    stream = torch.cuda.current_stream().cuda_stream
    for (B, H, N, d, dtype, causal, seed) in CASES:
        say(f"[noalloc] B={B} H={H} N={N} d={d} {dtype} causal={causal}")
        q, k, v = (t.to(DEV) for t in random_qkv(B, H, N, d, dtype, seed=seed))
        do = random_grad(B, H, N, d, dtype, seed + 100).to(DEV)
        scale = 1.0 / math.sqrt(d)
        o, lse = ea.attn_fwd(q, k, v, causal=causal, scale=scale)
        code = ea.ATTN_BF16 if dtype == "bf16" else ea.ATTN_F16
        ref = [torch.empty_like(q) for _ in range(3)]
        delta = torch.empty((B, H, N), dtype=torch.float32, device=DEV)
        st = ea.attn_bwd_ptr(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                             do.data_ptr(), *(t.data_ptr() for t in ref), delta.data_ptr(), B, H, N, d,
                             scale, int(causal), code, stream)
        assert st == ea.ATTN_OK
        got = [torch.full_like(q, float("nan")) for _ in range(3)]
        st = ea.attn_bwd_noalloc_ptr(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                                     do.data_ptr(), *(t.data_ptr() for t in got), B, H, N, d, scale,
                                     int(causal), code, stream)
        assert st == ea.ATTN_OK
        torch.cuda.synchronize()
        for name, r, g in zip(("dq", "dk", "dv"), ref, got):
            assert torch.isfinite(g.float()).all(), f"{name}: non-finite"
            assert torch.equal(r, g), f"{name}: differs from attn_bwd"


def test_noalloc_backward_binding():
    B, H, N, d = 1, 2, 300, 64
    q, k, v = (t.to(DEV) for t in random_qkv(B, H, N, d, "bf16", seed=71))
    do = random_grad(B, H, N, d, "bf16", 171).to(DEV)
    o, lse = ea.attn_fwd(q, k, v, causal=True)
    outs = [torch.empty_like(q) for _ in range(3)]
    ea.attn_bwd_noalloc(q, k, v, o, lse, do, *outs, causal=True)
    ref = ea.attn_bwd(q, k, v, o, lse, do, causal=True)
    torch.cuda.synchronize()
    assert all(torch.equal(a, b) for a, b in zip(outs, ref))
