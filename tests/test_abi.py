"""The C-ABI library: loads, exports what include/attn.h declares, rejects bad
arguments before touching the GPU (CPU only: no compute call is made)."""
import os
import re

import pytest

import exact_attention_96_amd as ea
from exact_attention_96_amd import _binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "attn.h")


def declared_symbols():
    with open(HEADER) as f:
        text = f.read()
    return sorted(set(re.findall(r"ATTN_API\s+[\w\s\*]*?\b(attn_\w+)\s*\(", text)))


def test_header_declares_the_entry_points():
    assert declared_symbols() == ["attn_abi_version", "attn_bwd", "attn_bwd_noalloc", "attn_fwd", "attn_fwd_masked",
                                  "attn_linear_fwd", "attn_linear_workspace_bytes", "attn_mask_pack",
                                  "attn_strerror"]


def test_library_exports_every_declared_symbol():
    lib = _binding.lib()
    for name in declared_symbols():
        assert hasattr(lib, name), f"{name} not exported by {_binding.LIB_PATH}"


def test_library_exports_nothing_else():
    import subprocess
    out = subprocess.run(["nm", "-D", "--defined-only", _binding.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    funcs = sorted({ln.split()[-1] for ln in out.splitlines() if " T " in ln})
    assert funcs == declared_symbols()


def test_abi_version_matches_header():
    with open(HEADER) as f:
        m = re.search(r"#define ATTN_ABI_VERSION (\d+)", f.read())
    assert ea.abi_version() == int(m.group(1))


def test_strerror():
    assert ea.strerror(0) == "success"
    assert "invalid" in ea.strerror(1)
    assert "unsupported" in ea.strerror(2)
    assert "HIP" in ea.strerror(3)
    assert "scratch" in ea.strerror(4)
    assert ea.strerror(12345) == "unknown status"


# Fake, well separated, 16-byte aligned addresses: every case below is rejected by
# the host checks, which run before any HIP call.
Q, K, V, O, L = (i << 40 for i in range(1, 6))
GOOD = dict(q=Q, k=K, v=V, o=O, lse=L, B=2, H=3, N=100, d=64, scale=0.125, causal=1, dtype=2,
            stream=0)


def call(**kw):
    a = dict(GOOD)
    a.update(kw)
    return ea.attn_fwd_ptr(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["H"], a["N"],
                           a["d"], a["scale"], a["causal"], a["dtype"], a["stream"])


@pytest.mark.parametrize("kw", [
    dict(q=0), dict(k=0), dict(v=0), dict(o=0), dict(lse=0),
    dict(B=0), dict(H=0), dict(N=0), dict(d=0), dict(B=-1), dict(N=-5),
    dict(dtype=3), dict(dtype=-1), dict(causal=2), dict(causal=-1),
    dict(scale=float("nan")), dict(scale=float("inf")),
    dict(q=Q + 8), dict(k=K + 2), dict(v=V + 4), dict(o=O + 8), dict(lse=L + 2),
    dict(o=Q), dict(o=K + 16), dict(o=V + 1600), dict(lse=Q + 64), dict(lse=O + 4),
    dict(o=Q - 16),  # o ends inside q
], ids=lambda kw: ",".join(f"{k}={v}" for k, v in kw.items()))
def test_invalid_arguments(kw):
    assert call(**kw) == ea.ATTN_EINVAL


@pytest.mark.parametrize("kw", [dict(d=32), dict(d=96), dict(d=256), dict(d=65),
                                dict(B=65536, H=65536, N=1, d=64)])
def test_unsupported(kw):
    assert call(**kw) == ea.ATTN_EUNSUPPORTED


def test_lse_just_after_o_is_fine_to_check():
    # o occupies B*H*N*d*2 bytes; lse placed right after it does not overlap o.
    nbytes = 2 * 3 * 100 * 64 * 2
    assert call(dtype=7, lse=O + nbytes) == ea.ATTN_EINVAL  # rejected for the dtype only


# attn_bwd: the same host checks, with its extra buffers.
DO, DQ, DK, DV, DL = (i << 40 for i in range(6, 11))
GOOD_BWD = dict(q=Q, k=K, v=V, o=O, lse=L, dout=DO, dq=DQ, dk=DK, dv=DV, delta=DL, B=2, H=3, N=100,
                d=64, scale=0.125, causal=1, dtype=2, stream=0)
BWD_ORDER = ["q", "k", "v", "o", "lse", "dout", "dq", "dk", "dv", "delta", "B", "H", "N", "d",
             "scale", "causal", "dtype", "stream"]


def call_bwd(**kw):
    a = dict(GOOD_BWD)
    a.update(kw)
    return ea.attn_bwd_ptr(*(a[n] for n in BWD_ORDER))


@pytest.mark.parametrize("kw", [
    dict(q=0), dict(o=0), dict(lse=0), dict(dout=0), dict(dq=0), dict(dk=0), dict(dv=0),
    dict(delta=0), dict(B=0), dict(N=-1), dict(d=0), dict(dtype=5), dict(causal=3),
    dict(scale=float("nan")), dict(dout=DO + 8), dict(dq=DQ + 4), dict(dv=DV + 2),
    dict(delta=DL + 1), dict(lse=L + 2),
    dict(dq=Q), dict(dk=O + 32), dict(dv=DO - 16), dict(delta=L), dict(delta=DQ + 64),
    dict(dk=DQ + 16), dict(dv=DK), dict(dq=DL - 16),
], ids=lambda kw: ",".join(f"{k}={v}" for k, v in kw.items()))
def test_bwd_invalid_arguments(kw):
    assert call_bwd(**kw) == ea.ATTN_EINVAL


@pytest.mark.parametrize("kw", [dict(dtype=0), dict(d=32), dict(d=96), dict(d=256),
                                dict(B=65536, H=65536, N=1, d=64)])
def test_bwd_unsupported(kw):
    assert call_bwd(**kw) == ea.ATTN_EUNSUPPORTED


NOALLOC_ORDER = [n for n in BWD_ORDER if n != "delta"]


def call_bwd_noalloc(**kw):
    a = dict(GOOD_BWD)
    a.update(kw)
    return ea.attn_bwd_noalloc_ptr(*(a[n] for n in NOALLOC_ORDER))


@pytest.mark.parametrize("kw", [
    dict(q=0), dict(lse=0), dict(dout=0), dict(dq=0), dict(dv=0), dict(B=0), dict(d=0), dict(dtype=5),
    dict(causal=3), dict(scale=float("inf")), dict(dk=DK + 8), dict(lse=L + 2), dict(dq=Q), dict(dv=DK),
], ids=lambda kw: ",".join(f"{k}={v}" for k, v in kw.items()))
def test_bwd_noalloc_invalid_arguments(kw):
    assert call_bwd_noalloc(**kw) == ea.ATTN_EINVAL


@pytest.mark.parametrize("kw", [dict(dtype=0), dict(d=96), dict(B=65536, H=65536, N=1, d=64)])
def test_bwd_noalloc_unsupported(kw):
    assert call_bwd_noalloc(**kw) == ea.ATTN_EUNSUPPORTED


@pytest.mark.parametrize("shape", [dict(B=1, H=1, N=(1 << 22) + 1), dict(B=2, H=64, N=32769),
                                   dict(B=64, H=64, N=1025)])
def test_bwd_noalloc_rejects_rows_beyond_its_scratch(shape):
    """B*H*N above 2^22 rows: a status of its own, before any HIP call (CPU-safe)."""
    assert call_bwd_noalloc(**shape) == ea.ATTN_ESCRATCH


def test_bwd_outputs_right_after_inputs_are_fine():
    # dq placed right after dout (tensor bytes 2*3*100*64*2) does not overlap it.
    nbytes = 2 * 3 * 100 * 64 * 2
    assert call_bwd(dq=DO + nbytes, dtype=9) == ea.ATTN_EINVAL  # rejected for the dtype only


# attn_fwd_masked and attn_mask_pack: host checks only (fake addresses, nothing launched).
MB, MT = 11 << 40, 12 << 40
GOOD_M = dict(q=Q, k=K, v=V, mask=MB, tiles=MT, sb=3, sh=1, o=O, lse=L, B=2, H=3, Nq=100, Nk=300, d=64,
              scale=0.125, causal=1, dtype=2, stream=0)
M_ORDER = ["q", "k", "v", "mask", "tiles", "sb", "sh", "o", "lse", "B", "H", "Nq", "Nk", "d", "scale",
           "causal", "dtype", "stream"]
MASK_BYTES = 6 * 100 * 5 * 8    # 6 mask heads of 100 rows of 5 words
TILE_BYTES = 6 * 1 * 1 * 8      # 6 mask heads of 1 tile of 1 word


def call_m(**kw):
    a = dict(GOOD_M)
    a.update(kw)
    return ea.attn_fwd_masked_ptr(*(a[n] for n in M_ORDER))


@pytest.mark.parametrize("kw", [
    dict(q=0), dict(k=0), dict(v=0), dict(o=0), dict(lse=0),
    dict(B=0), dict(H=0), dict(Nq=0), dict(Nk=0), dict(Nk=-3), dict(d=0),
    dict(dtype=3), dict(causal=2), dict(scale=float("nan")),
    dict(q=Q + 8), dict(k=K + 4), dict(o=O + 2), dict(lse=L + 1), dict(mask=MB + 4),
    dict(tiles=MT + 4), dict(mask=0),        # tiles without a mask
    dict(sb=-1), dict(sh=-5),
    dict(o=Q), dict(o=K + 16), dict(lse=V + 64), dict(lse=O + 16),
    dict(o=MB), dict(lse=MB + MASK_BYTES - 8),   # inside the mask words read
    dict(lse=MT + TILE_BYTES - 4),               # inside the tile summary
    dict(o=V - 16),                              # o ends inside v (v holds Nk rows)
], ids=lambda kw: ",".join(f"{k}={v}" for k, v in kw.items()))
def test_masked_invalid_arguments(kw):
    assert call_m(**kw) == ea.ATTN_EINVAL


@pytest.mark.parametrize("kw", [dict(d=32), dict(d=96), dict(B=65536, H=65536, Nq=1, Nk=1, d=64, sb=0, sh=0),
                                dict(sb=1 << 32), dict(Nq=1 << 20, Nk=1 << 20, sb=0, sh=0),
                                dict(Nk=4097 * 64, Nq=1, sb=0, sh=0)])  # unit list too long for LDS
def test_masked_unsupported(kw):
    assert call_m(**kw) == ea.ATTN_EUNSUPPORTED


def test_masked_without_mask_ignores_strides():
    # no mask and no tiles: the strides are not examined (a bad dtype is what is reported)
    assert call_m(mask=0, tiles=0, sb=-1, sh=-1, dtype=9) == ea.ATTN_EINVAL


def test_masked_lse_right_after_mask_is_fine_to_check():
    # mask heads 0 .. (B-1) sb + (H-1) sh = 5 are read; lse right after them does not overlap
    assert call_m(lse=MB + MASK_BYTES, dtype=7) == ea.ATTN_EINVAL  # rejected for the dtype only
    assert call_m(lse=MT + TILE_BYTES, dtype=7) == ea.ATTN_EINVAL


@pytest.mark.parametrize("args", [
    (0, MB, MT, 4, 100, 100), (Q, 0, MT, 4, 100, 100), (Q, MB, MT, 0, 100, 100),
    (Q, MB, MT, 4, 0, 100), (Q, MB, MT, 4, 100, 0), (Q, MB + 4, MT, 4, 100, 100),
    (Q, MB, MT + 2, 4, 100, 100),
    (Q, Q + 8, MT, 4, 100, 100),      # bits inside the mask bytes
    (Q, MB, MB + 64, 4, 100, 100),    # tiles inside the bits
])
def test_mask_pack_invalid_arguments(args):
    assert ea.attn_mask_pack_ptr(*args, 0) == ea.ATTN_EINVAL


# attn_linear_fwd: host checks only (fake addresses, nothing launched).
WS = 13 << 40
GOOD_L = dict(q=Q, k=K, v=V, o=O, B=2, H=3, N=100, E=64, M=64, fm=1, eps=1e-6, stream=0, ws=WS,
              ws_bytes=2 * 3 * 2 * (64 * 64 + 64) * 4)
L_ORDER = ["q", "k", "v", "o", "B", "H", "N", "E", "M", "fm", "eps", "stream", "ws", "ws_bytes"]


def call_l(**kw):
    a = dict(GOOD_L)
    a.update(kw)
    return ea.attn_linear_fwd_ptr(*(a[n] for n in L_ORDER))


@pytest.mark.parametrize("kw", [
    dict(q=0), dict(k=0), dict(v=0), dict(o=0), dict(B=0), dict(H=-1), dict(N=0), dict(E=0), dict(M=0),
    dict(fm=2), dict(eps=-1e-6), dict(eps=float("nan")), dict(q=Q + 4), dict(v=V + 8), dict(o=O + 12),
    dict(o=Q), dict(o=K + 64), dict(o=V - 16),
    dict(ws=WS + 8), dict(ws_bytes=1000), dict(ws=Q + 64), dict(ws=O - 256),
], ids=lambda kw: ",".join(f"{k}={v}" for k, v in kw.items()))
def test_linear_invalid_arguments(kw):
    assert call_l(**kw) == ea.ATTN_EINVAL


@pytest.mark.parametrize("kw", [dict(E=48), dict(E=256), dict(M=40), dict(M=8)])
def test_linear_unsupported(kw):
    assert call_l(ws=0, **kw) == ea.ATTN_EUNSUPPORTED


def _scan_workspace(BH, N, E, M):
    """The one-pass form's layout (E, M in {32, 64}): per head, a flag and an aggregate
    (state and key sum, E M + E floats) per span of 128 tokens, and a flag and an
    inclusive prefix per group of 4 spans; four parts, each 256-byte aligned."""
    up = lambda x: (x + 255) // 256 * 256
    S = (N + 127) // 128
    SG = (S + 3) // 4
    ent = E * M + E
    off = up(BH * S * 8)
    off = up(off + BH * SG * 8)
    off = up(off + BH * S * ent * 4)
    return up(off + BH * SG * ent * 4)


def test_linear_workspace_bytes():
    # the larger of the chunked form's [B H][chunks of 64][E M + E] fp32 and, where it
    # applies, the one-pass form's layout
    chunked = 2 * 3 * 2 * (64 * 64 + 64) * 4
    assert ea.linear_workspace_bytes(2, 3, 100, 64, 64) == max(chunked, _scan_workspace(6, 100, 64, 64))
    assert _scan_workspace(6, 100, 64, 64) > chunked  # one span, its aggregate and prefix
    big = 2 * 32 * 128 * (64 * 64 + 64) * 4
    assert ea.linear_workspace_bytes(2, 32, 8192, 64, 64) == max(big, _scan_workspace(64, 8192, 64, 64)) == big
    assert ea.linear_workspace_bytes(1, 2, 300, 32, 64) == max(1 * 2 * 5 * (32 * 64 + 32) * 4,
                                                                _scan_workspace(2, 300, 32, 64))
    assert ea.linear_workspace_bytes(1, 1, 64, 16, 16) == 1 * 1 * 1 * (16 * 16 + 16) * 4
    assert ea.linear_workspace_bytes(1, 1, 64, 128, 48) == 1 * 1 * 1 * (128 * 48 + 128) * 4
    assert ea.linear_workspace_bytes(0, 1, 64, 16, 16) == -1
