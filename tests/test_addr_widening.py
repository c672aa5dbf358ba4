"""CPU check of how the kernels move a 64-bit address through 32-bit lane moves.

The matrix-core forward passes the caller's mask base to its 4-byte LDS-DMA loads
through v_readfirstlane, one 32-bit word at a time; the builtin takes and returns a
signed int.  A signed widening of the low word once sign-extended a base with bit
31 set into the high word, and the first masked launch faulted the GPU.  This test
compiles the kernels' own split/join helpers (csrc/addr.hpp) for the host and checks
them on addresses with bit 31 and bit 63 set, and checks that the signed widening
(planted in a copy) fails the same cases.
"""
import os
import shutil
import subprocess
import textwrap

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "exact_attention_96_amd", "csrc")

PROGRAM = textwrap.dedent(r"""
    #include <stdint.h>
    #include <stdio.h>
    #include "addr.hpp"
    #ifdef SIGNED_WIDENING
    static uint64_t join(int lo, int hi) { return (uint64_t)(int64_t)lo | ((uint64_t)(uint32_t)hi << 32); }
    #else
    static uint64_t join(int lo, int hi) { return attn::addr_join(lo, hi); }
    #endif
    int main() {
        const uint64_t cases[] = {
            0x0ull, 0x1000ull, 0x7fffffffull, 0x80000000ull, 0x80001230ull, 0xfffffff0ull,
            0x00007f1280000000ull, 0x00007fff8badf000ull, 0x0000000180000010ull,
            0x8000000000000000ull, 0x8000000080000000ull, 0xffffffffffffffffull,
            0xffff800000000000ull, 0x123456789abcdef0ull};
        int bad = 0;
        for (uint64_t a : cases) {
            const uint64_t b = join(attn::addr_lo_word(a), attn::addr_hi_word(a));
            if (b != a) { printf("mismatch %016llx -> %016llx\n", (unsigned long long)a, (unsigned long long)b); ++bad; }
        }
        printf("bad %d\n", bad);
        return bad != 0;
    }
""")


def _build_and_run(tmp_path, defines=()):
    src = tmp_path / "addr_check.cpp"
    src.write_text(PROGRAM)
    exe = tmp_path / ("addr_check" + ("_mut" if defines else ""))
    cmd = ["g++", "-std=c++17", "-O2", "-Wall", "-Werror", "-I", CSRC, *[f"-D{d}" for d in defines],
           str(src), "-o", str(exe)]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    return subprocess.run([str(exe)], capture_output=True, text=True)


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")
def test_address_words_rejoin_exactly(tmp_path):
    r = _build_and_run(tmp_path)
    assert r.returncode == 0, r.stdout


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")
def test_signed_widening_is_caught(tmp_path):
    r = _build_and_run(tmp_path, ("SIGNED_WIDENING",))
    assert r.returncode != 0
    assert "mismatch 0000000080000000" in r.stdout
    assert "mismatch 00007f1280000000" in r.stdout
