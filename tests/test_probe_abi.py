"""The measurement probes' library (libattn_probe.so): loads, exports exactly what
include/attn_probe.h declares, rejects bad arguments before any HIP call (CPU only:
no kernel is launched)."""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "attn_probe.h")
LIB_PATH = os.path.join(ROOT, "exact_attention_96_amd", "libattn_probe.so")


def declared_symbols():
    with open(HEADER) as f:
        text = f.read()
    return sorted(set(re.findall(r"ATTN_PROBE_API\s+[\w\s\*]*?\b(attn_probe_\w+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB_PATH):
        pytest.fail(f"{LIB_PATH} is missing: build it first (python -m exact_attention_96_amd.build)")
    lib = ctypes.CDLL(LIB_PATH)
    vp, ci = ctypes.c_void_p, ctypes.c_int
    lib.attn_probe_mfma_bf16.argtypes = [vp, vp, ci, ci, vp]
    lib.attn_probe_lds_read.argtypes = [vp, ci, ci, ci, vp]
    return lib


def test_header_declares_the_probes():
    assert declared_symbols() == ["attn_probe_lds_read", "attn_probe_mfma_bf16"]


def test_library_exports_exactly_the_declared_symbols(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", LIB_PATH], capture_output=True, text=True,
                         check=True).stdout
    funcs = sorted({ln.split()[-1] for ln in out.splitlines() if " T " in ln})
    assert funcs == declared_symbols()


# a fake device address: every call below is rejected before it is used
FAKE = 1 << 40


@pytest.mark.parametrize("ops,out,blocks,iters,rc", [
    (None, FAKE, 1, 1, -1), (FAKE, None, 1, 1, -1),
    (FAKE, FAKE, 0, 1, -2), (FAKE, FAKE, 1, 0, -2), (FAKE, FAKE, -5, 10, -2),
])
def test_mfma_probe_rejects(lib, ops, out, blocks, iters, rc):
    assert lib.attn_probe_mfma_bf16(ops, out, blocks, iters, None) == rc


@pytest.mark.parametrize("out,blocks,iters,mode,rc", [
    (None, 1, 1, 0, -1), (FAKE, 0, 1, 0, -2), (FAKE, 1, 0, 2, -2), (FAKE, 1, 1, 3, -3), (FAKE, 1, 1, -1, -3),
])
def test_lds_probe_rejects(lib, out, blocks, iters, mode, rc):
    assert lib.attn_probe_lds_read(out, blocks, iters, mode, None) == rc
