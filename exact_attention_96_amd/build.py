"""Builds libattn.so (the HIP kernels and the C ABI) in-tree for gfx950, and
libattn_probe.so (the measurement harness's rate probes, include/attn_probe.h).

    python -m exact_attention_96_amd.build [-v]

Always recompiles.  The libraries are written next to this file, where the
Python binding and bench.py load them from.
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libattn.so")
SOURCES = [os.path.join(CSRC, "attn_api.hip")]
PROBE_LIB = os.path.join(PKG, "libattn_probe.so")
PROBE_SOURCES = [os.path.join(PKG, "probe", "probe.hip")]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

HIP_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    "-Wall",
    "-Werror",
    # never emit packed fp32 VALU ops (v_pk_add/mul/fma_f32)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-fvisibility=hidden",
]


def build(verbose: bool = False, extra_flags: list[str] | None = None, out: str = LIB,
          sources: list[str] | None = None) -> str:
    tmp = out + ".tmp"
    cmd = [HIPCC, *HIP_FLAGS, *(extra_flags or []), "-I", INCLUDE, "-I", CSRC, *(sources or SOURCES), "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    # the host compilation pass does not know the gfx feature name; that note is harmless
    noise = "'-packed-fp32-ops' is not a recognized feature for this target"
    err = "\n".join(ln for ln in res.stderr.splitlines() if noise not in ln)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{err}")
    if verbose and err.strip():
        print(err, file=sys.stderr)
    os.replace(tmp, out)
    return out


def build_probe(verbose: bool = False) -> str:
    return build(verbose, out=PROBE_LIB, sources=PROBE_SOURCES)


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
    print(build_probe(verbose="-v" in sys.argv))
