"""Seeded synthetic attention inputs.

This module only draws random tensors; it holds none of the attention
arithmetic.  The oracle and the HIP path both consume what it returns, so a
parity check always compares the two on identical inputs.

Recipe (one CPU generator per call, seeded):
  Q, K, V are drawn in that order, each ``torch.randn(B, H, N, d, float32) * std``;
  for the "spiky" workload, ``round(0.01 * B*H*N)`` key rows picked by
  ``torch.randperm(B*H*N)`` over the flattened (b, h, n) rows are then
  multiplied by 8 (exact in every dtype used, being a power of two), which makes
  the running row maximum jump and exercises the rescaling of the online
  softmax; finally each tensor is rounded to the working dtype (round to
  nearest even).  The scale is 1/sqrt(d) rounded to fp32, the value of the
  naive-attention module of "PyTorch profiling part 3: attention" (section
  "朴素注意力").

The pages publish no benchmark dataset; these workloads stand in for the
attention shapes they discuss (long causal sequences, short many-head
batches).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, replace

import numpy as np
import torch

DTYPES = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    N: int
    d: int
    dtype: str          # "f32" | "f16" | "bf16"
    causal: bool
    std: float = 1.0
    spiky_frac: float = 0.0   # fraction of key rows multiplied by 8
    seed: int = 0

    @property
    def torch_dtype(self) -> torch.dtype:
        return DTYPES[self.dtype]

    @property
    def scale(self) -> float:
        """1/sqrt(d) rounded to fp32 (the value the kernel receives)."""
        return float(np.float32(1.0 / math.sqrt(self.d)))

    @property
    def flops(self) -> float:
        """Algorithmic FLOPs: 4*B*H*N^2*d, halved when causal."""
        f = 4.0 * self.B * self.H * self.N * self.N * self.d
        return f / 2 if self.causal else f

    @property
    def elt(self) -> int:
        return torch.tensor([], dtype=self.torch_dtype).element_size()

    @property
    def io_bytes(self) -> int:
        """Algorithmic bytes: read Q, K, V once, write O once (dtype) and lse once (fp32)."""
        return 4 * self.B * self.H * self.N * self.d * self.elt + 4 * self.B * self.H * self.N

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


# The five workloads (seeds 1..5).  "c3" is the headline one.
WORKLOADS = {
    "c1": Workload("c1_f32_noncausal_b1h1n128d64", 1, 1, 128, 64, "f32", False, seed=1),
    "c2": Workload("c2_bf16_causal_b4h16n2048d64", 4, 16, 2048, 64, "bf16", True, seed=2),
    "c3": Workload("c3_bf16_causal_b2h32n8192d128", 2, 32, 8192, 128, "bf16", True, seed=3),
    "c4": Workload("c4_f16_noncausal_b16h16n512d64_spiky", 16, 16, 512, 64, "f16", False,
                   std=0.5, spiky_frac=0.01, seed=4),
    "c5": Workload("c5_bf16_causal_b1h8n32768d128", 1, 8, 32768, 128, "bf16", True, seed=5),
}
HEADLINE = "c3"


def make_inputs(w: Workload, seed: int | None = None):
    """Q, K, V (CPU tensors in w's dtype, shape [B, H, N, d]) for workload w."""
    g = torch.Generator(device="cpu")
    g.manual_seed(w.seed if seed is None else seed)
    shape = (w.B, w.H, w.N, w.d)
    q = torch.randn(shape, dtype=torch.float32, generator=g) * w.std
    k = torch.randn(shape, dtype=torch.float32, generator=g) * w.std
    v = torch.randn(shape, dtype=torch.float32, generator=g) * w.std
    if w.spiky_frac > 0:
        rows = w.B * w.H * w.N
        n_spiky = int(round(w.spiky_frac * rows))
        idx = torch.randperm(rows, generator=g)[:n_spiky]
        k.view(rows, w.d)[idx] *= 8.0
    dt = w.torch_dtype
    return q.to(dt), k.to(dt), v.to(dt)


def random_qkv(B: int, H: int, N: int, d: int, dtype: str, seed: int, std: float = 1.0):
    """Q, K, V for an ad-hoc shape (parity sweeps), same recipe as make_inputs."""
    w = Workload("adhoc", B, H, N, d, dtype, False, std=std, seed=seed)
    return make_inputs(w)


def random_grad(B: int, H: int, N: int, d: int, dtype: str, seed: int, std: float = 1.0):
    """Upstream gradient dO (CPU tensor [B, H, N, d] in `dtype`): i.i.d. N(0, std^2),
    the gradient of a random linear loss sum(O * G)."""
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    dt = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[dtype]
    return (torch.randn((B, H, N, d), dtype=torch.float32, generator=g) * std).to(dt)


def random_qkv_lens(B: int, H: int, Nq: int, Nk: int, d: int, dtype: str, seed: int, std: float = 1.0):
    """Q [B, H, Nq, d] and K, V [B, H, Nk, d] (CPU, `dtype`): drawn in the order Q, K, V
    from one seeded generator as randn * std, then rounded to the dtype."""
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    q = torch.randn((B, H, Nq, d), dtype=torch.float32, generator=g) * std
    k = torch.randn((B, H, Nk, d), dtype=torch.float32, generator=g) * std
    v = torch.randn((B, H, Nk, d), dtype=torch.float32, generator=g) * std
    dt = DTYPES[dtype]
    return q.to(dt), k.to(dt), v.to(dt)


def random_mask(kind: str, Bm: int, Hm: int, Nq: int, Nk: int, seed: int, **kw) -> torch.Tensor:
    """A boolean mask [Bm, Hm, Nq, Nk] (CPU; True = key visible) of a given pattern:

    "bernoulli"  each entry visible with probability kw["p"] (default 0.5);
    "window"     key j visible to query i iff i + Nk - Nq - kw["w"] < j <= i + Nk - Nq
                 (a sliding window of w keys ending at the bottom-right diagonal);
    "padding"    per (b, h) a random key length L in [1, Nk]: key j visible iff j < L
                 (a padded batch);
    "blocks"     64 x 64 blocks visible with probability kw["p"] (default 0.3), the rest
                 hidden (block-sparse);
    "empty_rows" bernoulli(0.5) with a random tenth of the rows hidden entirely.
    """
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    shape = (Bm, Hm, Nq, Nk)
    if kind == "bernoulli":
        return torch.rand(shape, generator=g) < kw.get("p", 0.5)
    if kind == "window":
        i = torch.arange(Nq).view(Nq, 1) + (Nk - Nq)
        j = torch.arange(Nk).view(1, Nk)
        m = (j <= i) & (j > i - kw["w"])
        return m.expand(shape).contiguous()
    if kind == "padding":
        lens = torch.randint(1, Nk + 1, (Bm, Hm, 1, 1), generator=g)
        return (torch.arange(Nk).view(1, 1, 1, Nk) < lens).expand(shape).contiguous()
    if kind == "blocks":
        nb = ((Nq + 63) // 64, (Nk + 63) // 64)
        blk = torch.rand((Bm, Hm) + nb, generator=g) < kw.get("p", 0.3)
        m = blk.repeat_interleave(64, dim=2).repeat_interleave(64, dim=3)
        return m[:, :, :Nq, :Nk].contiguous()
    if kind == "empty_rows":
        m = torch.rand(shape, generator=g) < 0.5
        rows = torch.rand((Bm, Hm, Nq, 1), generator=g) < 0.1
        return (m & ~rows).contiguous()
    raise ValueError(f"unknown mask kind {kind!r}")


@dataclass(frozen=True)
class MaskedWorkload:
    """A workload of attn_fwd_masked: q [B, H, Nq, d], k and v [B, H, Nk, d] drawn by
    random_qkv_lens, and a mask [1, 1, Nq, Nk] shared by every head drawn by
    random_mask(mask_kind, ...) (None: no mask)."""
    name: str
    B: int
    H: int
    Nq: int
    Nk: int
    d: int
    dtype: str
    causal: bool
    mask_kind: str | None = None
    mask_w: int = 0          # window length for mask_kind "window"
    seed: int = 0

    @property
    def scale(self) -> float:
        return float(np.float32(1.0 / math.sqrt(self.d)))

    @property
    def elt(self) -> int:
        return torch.tensor([], dtype=DTYPES[self.dtype]).element_size()

    @property
    def io_bytes(self) -> int:
        """Read Q, K, V once, write O and lse once (the packed mask is counted apart)."""
        return (2 * self.B * self.H * (self.Nq + self.Nk) * self.d * self.elt
                + 4 * self.B * self.H * self.Nq)

    def inputs(self):
        q, k, v = random_qkv_lens(self.B, self.H, self.Nq, self.Nk, self.d, self.dtype, self.seed)
        mask = None
        if self.mask_kind is not None:
            mask = random_mask(self.mask_kind, 1, 1, self.Nq, self.Nk, self.seed + 1, w=self.mask_w)
        return q, k, v, mask


# Masked and unequal-length workloads at the headline head shape (B=2, H=32, d=128, bf16).
MASKED_WORKLOADS = {
    # the causal mask materialised as a boolean lower triangle (the math backend's form)
    "m1": MaskedWorkload("m1_bf16_tril_mask_b2h32n8192d128", 2, 32, 8192, 8192, 128, "bf16", False,
                         mask_kind="window", mask_w=8192, seed=101),
    # a causal sliding window of 1024 keys given as a mask
    "m2": MaskedWorkload("m2_bf16_window1024_b2h32n8192d128", 2, 32, 8192, 8192, 128, "bf16", True,
                         mask_kind="window", mask_w=1024, seed=102),
    # chunked prefill: the last 2048 of 8192 positions, causal from the bottom-right corner
    "m3": MaskedWorkload("m3_bf16_causal_nq2048_nk8192_b2h32d128", 2, 32, 2048, 8192, 128, "bf16",
                         True, seed=103),
}


@dataclass(frozen=True)
class LinearWorkload:
    """A workload of attn_linear_fwd (causal linear attention, fp32): q, k [B, H, N, E]
    and v [B, H, N, M] drawn in that order as randn from one seeded generator."""
    name: str
    B: int
    H: int
    N: int
    E: int
    M: int
    feature_map: bool = True
    eps: float = 1e-6
    seed: int = 0

    @property
    def io_bytes(self) -> int:
        """Read q, k, v once and write o once (fp32)."""
        return 4 * self.B * self.H * self.N * (2 * self.E + 2 * self.M)

    @property
    def flops(self) -> float:
        """Per token: state update and readout, 2 E M each; key sum and denominator, 3 E."""
        return float(self.B * self.H * self.N) * (4.0 * self.E * self.M + 3.0 * self.E)

    def inputs(self):
        g = torch.Generator(device="cpu")
        g.manual_seed(self.seed)
        q = torch.randn((self.B, self.H, self.N, self.E), generator=g)
        k = torch.randn((self.B, self.H, self.N, self.E), generator=g)
        v = torch.randn((self.B, self.H, self.N, self.M), generator=g)
        return q, k, v


# Causal linear attention at the headline sequence shape (B=2, H=32, N=8192), E = M = 64.
LINEAR_WORKLOADS = {
    "l1": LinearWorkload("l1_f32_causal_linear_b2h32n8192e64m64", 2, 32, 8192, 64, 64, seed=201),
}
