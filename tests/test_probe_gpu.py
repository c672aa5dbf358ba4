"""The measurement probes (libattn_probe.so) compute what they claim, through the C ABI:
the matrix-core probe's sums for constant operands, and for each LDS read form the word
each lane last read, predicted on the host from the fill pattern (for the transposing
read, from its 4 x 16 transpose of 16-bit elements per 16-lane group)."""
import ctypes
import os

import numpy as np
import pytest

torch = pytest.importorskip("torch")

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB_PATH = os.path.join(ROOT, "exact_attention_96_amd", "libattn_probe.so")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def lib():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    lib = ctypes.CDLL(LIB_PATH)
    vp, ci = ctypes.c_void_p, ctypes.c_int
    lib.attn_probe_mfma_bf16.argtypes = [vp, vp, ci, ci, vp]
    lib.attn_probe_lds_read.argtypes = [vp, ci, ci, ci, vp]
    return lib


@pytest.mark.parametrize("iters", [1, 7, 64])
def test_mfma_probe_sums(lib, iters):
    # all operands 1.0: each product adds 16 to every accumulator entry, each of the four
    # chains takes two products an iteration, and a thread sums its 4 x 16 entries
    blocks = 3
    ops = torch.ones(256 * 8 * 8, dtype=torch.bfloat16, device="cuda:0")
    out = torch.full((blocks * 256,), float("nan"), dtype=torch.float32, device="cuda:0")
    rc = lib.attn_probe_mfma_bf16(ops.data_ptr(), out.data_ptr(), blocks, iters, torch.cuda.current_stream().cuda_stream)
    assert rc == 0
    torch.cuda.synchronize()
    assert torch.all(out == 4 * 16 * 2 * 16 * iters)


def _lds_words():
    # the fill: 32-bit word i of a workgroup's 64 KiB holds i * 2654435761 mod 2^32
    i = np.arange(65536 // 4, dtype=np.uint64)
    return ((i * np.uint64(2654435761)) % np.uint64(1 << 32)).astype(np.uint32)


def _expected_last_words(mode, iters):
    words = _lds_words()
    piece = 16 if mode == 0 else 8
    window = 64 * piece
    nwin = 65536 // window
    halves = words.view(np.uint16)  # little endian: element 2 i is the low half of word i
    exp = np.zeros(512, dtype=np.uint32)
    for t in range(512):
        w, lane = t // 64, t % 64
        win = (w * 8 + (iters - 1) * 8 + 7) % nwin  # the last read of the last iteration
        base = win * window
        if mode == 0:  # word 1 of the lane's 16 bytes
            exp[t] = words[(base + lane * 16) // 4 + 1]
        elif mode == 1:  # word 1 of the lane's 8 bytes
            exp[t] = words[(base + lane * 8) // 4 + 1]
        else:
            # 16-lane group g reads 128 contiguous bytes (lane j: elements 4 j .. 4 j + 3);
            # lane i receives, for t = 0..3, element (i % 4) of lane 4 t + i / 4's piece;
            # word 1 of the result packs t = 2 (low half) and t = 3
            g, i = lane // 16, lane % 16
            gbase = (base + g * 128) // 2  # in 16-bit elements
            def elem(tt):
                return int(halves[gbase + 4 * (4 * tt + i // 4) + (i % 4)])
            exp[t] = np.uint32(elem(2) | (elem(3) << 16))
    return exp


@pytest.mark.parametrize("mode", [0, 1, 2])
@pytest.mark.parametrize("iters", [1, 5])
def test_lds_probe_reads(lib, mode, iters):
    blocks = 2
    out = torch.zeros(blocks * 512, dtype=torch.int32, device="cuda:0")
    rc = lib.attn_probe_lds_read(out.data_ptr(), blocks, iters, mode, torch.cuda.current_stream().cuda_stream)
    assert rc == 0
    torch.cuda.synchronize()
    got = out.cpu().numpy().view(np.uint32).reshape(blocks, 512)
    exp = _expected_last_words(mode, iters)
    for b in range(blocks):
        assert np.array_equal(got[b], exp), f"mode {mode}: first mismatch at thread {np.argmax(got[b] != exp)}"
