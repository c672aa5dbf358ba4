"""ctypes binding of libattn.so (argument marshalling only).

Every step of the forward and backward runs in the HIP library; this module
checks the tensors, allocates the outputs with torch and passes raw device
pointers and torch's current HIP stream to ``attn_fwd``, ``attn_fwd_masked``,
``attn_mask_pack`` and ``attn_bwd`` (declared in include/attn.h).
There is no fallback: a missing library or a failed call raises.
"""
from __future__ import annotations

import ctypes
import math
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libattn.so")

ATTN_F32, ATTN_F16, ATTN_BF16 = 0, 1, 2
ATTN_OK, ATTN_EINVAL, ATTN_EUNSUPPORTED, ATTN_EHIP, ATTN_ESCRATCH = 0, 1, 2, 3, 4

_lib = None


class AttnError(RuntimeError):
    def __init__(self, status: int, msg: str, call: str = "attn_fwd"):
        super().__init__(f"{call} failed: status {status} ({msg})")
        self.status = status


def lib() -> ctypes.CDLL:
    """The loaded HIP library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"HIP library not built: {LIB_PATH} is missing "
                "(run `python -m exact_attention_96_amd.build`)")
        L = ctypes.CDLL(LIB_PATH)
        vp = ctypes.c_void_p
        ci = ctypes.c_int
        L.attn_fwd.argtypes = [vp, vp, vp, vp, vp, ci, ci, ci, ci, ctypes.c_float, ci, ci, vp]
        L.attn_fwd.restype = ci
        L.attn_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, ci, ci, ci, ci, ctypes.c_float,
                               ci, ci, vp]
        L.attn_bwd.restype = ci
        L.attn_bwd_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, ci, ci, ci, ci, ctypes.c_float, ci, ci,
                                       vp]
        L.attn_bwd_noalloc.restype = ci
        ll = ctypes.c_longlong
        L.attn_fwd_masked.argtypes = [vp, vp, vp, vp, vp, ll, ll, vp, vp, ci, ci, ci, ci, ci,
                                      ctypes.c_float, ci, ci, vp]
        L.attn_fwd_masked.restype = ci
        L.attn_mask_pack.argtypes = [vp, vp, vp, ll, ci, ci, vp]
        L.attn_linear_fwd.argtypes = [vp, vp, vp, vp, ci, ci, ci, ci, ci, ci, ctypes.c_float, vp, ll, vp]
        L.attn_linear_fwd.restype = ci
        L.attn_linear_workspace_bytes.argtypes = [ci, ci, ci, ci, ci]
        L.attn_linear_workspace_bytes.restype = ll
        L.attn_mask_pack.restype = ci
        L.attn_strerror.argtypes = [ci]
        L.attn_strerror.restype = ctypes.c_char_p
        L.attn_abi_version.argtypes = []
        L.attn_abi_version.restype = ci
        _lib = L
    return _lib


def strerror(status: int) -> str:
    return lib().attn_strerror(int(status)).decode()


def abi_version() -> int:
    return int(lib().attn_abi_version())


def attn_fwd_ptr(q: int, k: int, v: int, o: int, lse: int, B: int, H: int, N: int, d: int,
                 scale: float, causal: int, dtype: int, stream: int) -> int:
    """Raw call with integer device addresses; returns the status code."""
    return int(lib().attn_fwd(q, k, v, o, lse, B, H, N, d, ctypes.c_float(scale),
                              causal, dtype, stream))


def attn_fwd_masked_ptr(q: int, k: int, v: int, mask_bits: int | None, mask_tiles: int | None,
                        mask_stride_b: int, mask_stride_h: int, o: int, lse: int, B: int, H: int,
                        Nq: int, Nk: int, d: int, scale: float, causal: int, dtype: int,
                        stream: int) -> int:
    """Raw call with integer device addresses (None or 0: no mask / no tile summary)."""
    return int(lib().attn_fwd_masked(q, k, v, mask_bits or None, mask_tiles or None, mask_stride_b,
                                     mask_stride_h, o, lse, B, H, Nq, Nk, d, ctypes.c_float(scale),
                                     causal, dtype, stream))


def attn_mask_pack_ptr(mask: int, bits: int, tiles: int | None, heads: int, Nq: int, Nk: int,
                       stream: int) -> int:
    """Raw call with integer device addresses (tiles None or 0: no summary)."""
    return int(lib().attn_mask_pack(mask, bits, tiles or None, heads, Nq, Nk, stream))


def attn_linear_fwd_ptr(q: int, k: int, v: int, o: int, B: int, H: int, N: int, E: int, M: int,
                        feature_map: int, eps: float, stream: int, workspace: int | None = None,
                        workspace_bytes: int = 0) -> int:
    """Raw call with integer device addresses; returns the status code."""
    return int(lib().attn_linear_fwd(q, k, v, o, B, H, N, E, M, feature_map, ctypes.c_float(eps),
                                     workspace or None, workspace_bytes, stream))


def linear_workspace_bytes(B: int, H: int, N: int, E: int, M: int) -> int:
    return int(lib().attn_linear_workspace_bytes(B, H, N, E, M))


def attn_linear_fwd(q, k, v, feature_map: bool = True, eps: float = 1e-6, out=None, chunked: bool = True,
                    workspace=None):
    """Causal linear attention forward on the GPU (fp32).

    q, k: [B, H, N, E]; v: [B, H, N, M]; float32, contiguous, one HIP device.
    feature_map=True: phi = elu + 1 on q and k and the normaliser 1 / (phi(q_j) .
    sum_{t<=j} phi(k_t) + eps); False: the causal dot product of q and k as given.
    chunked=True runs a block form on a workspace (allocated here with torch unless one
    is passed: a uint8 tensor of at least linear_workspace_bytes, needing no
    initialisation): the one-pass form for E and M in {32, 64}, the chunked form
    otherwise; False the scan.
    Returns o [B, H, N, M] float32, enqueued on torch's current stream.
    """
    import torch
    for name, t in (("q", q), ("k", k), ("v", v)):
        if not isinstance(t, torch.Tensor):
            raise TypeError(f"{name} must be a torch.Tensor")
        if t.device.type != "cuda" or t.device != q.device:
            raise ValueError(f"{name} must be on q's HIP device")
        if not t.is_contiguous() or t.dtype != torch.float32 or t.dim() != 4:
            raise ValueError(f"{name} must be a contiguous 4-d float32 tensor")
    if k.shape != q.shape or v.shape[:3] != q.shape[:3]:
        raise ValueError(f"q, k [B, H, N, E] and v [B, H, N, M] expected, got {tuple(q.shape)}, "
                         f"{tuple(k.shape)}, {tuple(v.shape)}")
    B, H, N, E = q.shape
    M = v.shape[3]
    if out is None:
        out = torch.empty_like(v)
    if out.shape != v.shape or out.dtype != torch.float32 or not out.is_contiguous() or out.device != q.device:
        raise ValueError("out must be a contiguous float32 tensor like v")
    ws_ptr, ws_bytes = None, 0
    if chunked:
        need = linear_workspace_bytes(B, H, N, E, M)
        if workspace is None:
            workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
        if not isinstance(workspace, torch.Tensor) or workspace.device != q.device or not workspace.is_contiguous() \
                or workspace.numel() * workspace.element_size() < need:
            raise ValueError(f"workspace must be a contiguous tensor of at least {need} bytes on q's device")
        ws_ptr, ws_bytes = workspace.data_ptr(), workspace.numel() * workspace.element_size()
    with torch.cuda.device(q.device):
        stream = torch.cuda.current_stream(q.device).cuda_stream
        st = attn_linear_fwd_ptr(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), B, H, N, E, M,
                                 int(bool(feature_map)), float(eps), stream, ws_ptr, ws_bytes)
    if st != ATTN_OK:
        raise AttnError(st, strerror(st), "attn_linear_fwd")
    return out


def attn_bwd_ptr(q: int, k: int, v: int, o: int, lse: int, dout: int, dq: int, dk: int, dv: int,
                 delta: int, B: int, H: int, N: int, d: int, scale: float, causal: int, dtype: int,
                 stream: int) -> int:
    """Raw call with integer device addresses; returns the status code."""
    return int(lib().attn_bwd(q, k, v, o, lse, dout, dq, dk, dv, delta, B, H, N, d,
                              ctypes.c_float(scale), causal, dtype, stream))


def attn_bwd_noalloc_ptr(q: int, k: int, v: int, o: int, lse: int, dout: int, dq: int, dk: int, dv: int,
                         B: int, H: int, N: int, d: int, scale: float, causal: int, dtype: int,
                         stream: int) -> int:
    """Raw call of the no-allocation backward with integer device addresses; returns
    the status code."""
    return int(lib().attn_bwd_noalloc(q, k, v, o, lse, dout, dq, dk, dv, B, H, N, d,
                                      ctypes.c_float(scale), causal, dtype, stream))


def _dtype_code(t) -> int:
    import torch
    codes = {torch.float32: ATTN_F32, torch.float16: ATTN_F16, torch.bfloat16: ATTN_BF16}
    if t.dtype not in codes:
        raise TypeError(f"unsupported dtype {t.dtype}; expected float32, float16 or bfloat16")
    return codes[t.dtype]


def attn_fwd(q, k, v, causal: bool = False, scale: float | None = None, out=None, lse=None):
    """Attention forward on the GPU.

    q, k, v: torch tensors [B, H, N, d] on one HIP device, same dtype
    (float32, float16 or bfloat16), contiguous.  Returns (o, lse): o like q,
    lse float32 [B, H, N] with lse = ln sum_j e^{s_ij}.  ``scale`` defaults to
    1/sqrt(d) rounded to fp32.  The call is enqueued on torch's current stream.
    """
    import torch
    for name, t in (("q", q), ("k", k), ("v", v)):
        if not isinstance(t, torch.Tensor):
            raise TypeError(f"{name} must be a torch.Tensor")
        if t.device.type != "cuda":
            raise ValueError(f"{name} must be on a HIP device, got {t.device}")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    if q.dim() != 4 or k.shape != q.shape or v.shape != q.shape:
        raise ValueError(f"q, k, v must share one [B, H, N, d] shape, got {tuple(q.shape)}, "
                         f"{tuple(k.shape)}, {tuple(v.shape)}")
    if k.dtype != q.dtype or v.dtype != q.dtype:
        raise TypeError("q, k, v must share one dtype")
    if k.device != q.device or v.device != q.device:
        raise ValueError("q, k, v must be on one device")
    code = _dtype_code(q)
    B, H, N, d = q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    if out.shape != q.shape or out.dtype != q.dtype or not out.is_contiguous() or out.device != q.device:
        raise ValueError("out must be a contiguous tensor like q")
    if lse.shape != (B, H, N) or lse.dtype != torch.float32 or not lse.is_contiguous() \
            or lse.device != q.device:
        raise ValueError("lse must be a contiguous float32 [B, H, N] tensor on q's device")
    with torch.cuda.device(q.device):
        stream = torch.cuda.current_stream(q.device).cuda_stream
        st = attn_fwd_ptr(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
                          B, H, N, d, float(scale), int(bool(causal)), code, stream)
    if st != ATTN_OK:
        raise AttnError(st, strerror(st))
    return out, lse


class PackedMask(tuple):
    """(bits, tiles) of a packed mask: bits int64 [Bm, Hm, Nq, ceil(Nk / 64)], bit j % 64
    of word j / 64 = key j visible; tiles int64 [Bm, Hm, ceil(Nq / 256), ceil(Nk / 4096)]
    (or None), the per-256-row-tile summary of which 64-key units any row sees."""

    def __new__(cls, bits, tiles):
        return super().__new__(cls, (bits, tiles))

    bits = property(lambda self: self[0])
    tiles = property(lambda self: self[1])


def pack_mask(mask, tiles: bool = True) -> PackedMask:
    """Packs a boolean mask [Bm, Hm, Nq, Nk] (torch.bool or uint8, contiguous, on a HIP
    device; nonzero = key visible) into the format of attn_fwd_masked, with the tile
    summary that lets the kernel skip empty key units (tiles=False: bits only).  The
    packing runs on the GPU (attn_mask_pack) on torch's current stream."""
    import torch
    if not isinstance(mask, torch.Tensor):
        raise TypeError("mask must be a torch.Tensor")
    if mask.device.type != "cuda":
        raise ValueError(f"mask must be on a HIP device, got {mask.device}")
    if mask.dtype not in (torch.bool, torch.uint8):
        raise TypeError(f"mask must be torch.bool or torch.uint8, got {mask.dtype}")
    if mask.dim() != 4 or not mask.is_contiguous():
        raise ValueError("mask must be a contiguous [Bm, Hm, Nq, Nk] tensor")
    Bm, Hm, Nq, Nk = mask.shape
    W = (Nk + 63) // 64
    bits = torch.empty((Bm, Hm, Nq, W), dtype=torch.int64, device=mask.device)
    tl = None
    if tiles:
        tl = torch.empty((Bm, Hm, (Nq + 255) // 256, (W + 63) // 64), dtype=torch.int64, device=mask.device)
    with torch.cuda.device(mask.device):
        stream = torch.cuda.current_stream(mask.device).cuda_stream
        st = attn_mask_pack_ptr(mask.data_ptr(), bits.data_ptr(), None if tl is None else tl.data_ptr(),
                                Bm * Hm, Nq, Nk, stream)
    if st != ATTN_OK:
        raise AttnError(st, strerror(st), "attn_mask_pack")
    return PackedMask(bits, tl)


def attn_fwd_masked(q, k, v, mask=None, causal: bool = False, scale: float | None = None,
                    mask_bits=None, out=None, lse=None):
    """Attention forward with unequal query and key lengths and an optional mask.

    q: [B, H, Nq, d]; k, v: [B, H, Nk, d]; one HIP device, one dtype, contiguous.
    mask: None, or a boolean mask [Bm, Hm, Nq, Nk] (Bm in {1, B}, Hm in {1, H}; true =
    visible), packed on the GPU first; or mask_bits: an already packed mask (see
    pack_mask; a PackedMask, or a bare bits tensor for no unit skipping).  causal:
    keys j > i + Nk - Nq are hidden as well.  Returns (o, lse):
    o like q, lse float32 [B, H, Nq]; a row that sees no key gets o = 0, lse = -inf.
    """
    import torch
    for name, t in (("q", q), ("k", k), ("v", v)):
        if not isinstance(t, torch.Tensor):
            raise TypeError(f"{name} must be a torch.Tensor")
        if t.device.type != "cuda":
            raise ValueError(f"{name} must be on a HIP device, got {t.device}")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    if q.dim() != 4 or k.dim() != 4 or v.shape != k.shape or q.shape[:2] != k.shape[:2] \
            or q.shape[3] != k.shape[3]:
        raise ValueError(f"q [B, H, Nq, d] and k, v [B, H, Nk, d] expected, got {tuple(q.shape)}, "
                         f"{tuple(k.shape)}, {tuple(v.shape)}")
    if k.dtype != q.dtype or v.dtype != q.dtype:
        raise TypeError("q, k, v must share one dtype")
    if k.device != q.device or v.device != q.device:
        raise ValueError("q, k, v must be on one device")
    code = _dtype_code(q)
    B, H, Nq, d = q.shape
    Nk = k.shape[2]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if mask is not None and mask_bits is not None:
        raise ValueError("pass mask or mask_bits, not both")
    if mask is not None:
        if not isinstance(mask, torch.Tensor) or mask.device != q.device:
            raise ValueError("mask must be a tensor on q's device")
        if mask.dim() != 4 or mask.shape[0] not in (1, B) or mask.shape[1] not in (1, H) \
                or tuple(mask.shape[2:]) != (Nq, Nk):
            raise ValueError(f"mask of shape {tuple(mask.shape)} does not match [{B} or 1, {H} or 1, {Nq}, {Nk}]")
        mask_bits = pack_mask(mask)
    sb = sh = 0
    mptr = tptr = None
    if isinstance(mask_bits, PackedMask):
        mask_bits, tiles = mask_bits
    else:
        tiles = None
    if mask_bits is not None:
        W = (Nk + 63) // 64
        if not isinstance(mask_bits, torch.Tensor) or mask_bits.dtype != torch.int64 \
                or mask_bits.dim() != 4 or not mask_bits.is_contiguous() or mask_bits.device != q.device:
            raise ValueError("mask_bits must be a contiguous int64 [Bm, Hm, Nq, ceil(Nk/64)] tensor on q's device")
        Bm, Hm = mask_bits.shape[:2]
        if Bm not in (1, B) or Hm not in (1, H) or tuple(mask_bits.shape[2:]) != (Nq, W):
            raise ValueError(f"mask of shape {tuple(mask_bits.shape)} does not match "
                             f"[{B} or 1, {H} or 1, {Nq}, {W}]")
        sb = 0 if Bm == 1 else Hm
        sh = 0 if Hm == 1 else 1
        mptr = mask_bits.data_ptr()
        if tiles is not None:
            if not isinstance(tiles, torch.Tensor) or tiles.dtype != torch.int64 or not tiles.is_contiguous() \
                    or tiles.device != q.device \
                    or tuple(tiles.shape) != (Bm, Hm, (Nq + 255) // 256, (W + 63) // 64):
                raise ValueError("mask tiles do not match the mask bits")
            tptr = tiles.data_ptr()
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((B, H, Nq), dtype=torch.float32, device=q.device)
    if out.shape != q.shape or out.dtype != q.dtype or not out.is_contiguous() or out.device != q.device:
        raise ValueError("out must be a contiguous tensor like q")
    if lse.shape != (B, H, Nq) or lse.dtype != torch.float32 or not lse.is_contiguous() \
            or lse.device != q.device:
        raise ValueError("lse must be a contiguous float32 [B, H, Nq] tensor on q's device")
    with torch.cuda.device(q.device):
        stream = torch.cuda.current_stream(q.device).cuda_stream
        st = attn_fwd_masked_ptr(q.data_ptr(), k.data_ptr(), v.data_ptr(), mptr, tptr, sb, sh, out.data_ptr(),
                                 lse.data_ptr(), B, H, Nq, Nk, d, float(scale), int(bool(causal)), code,
                                 stream)
    if st != ATTN_OK:
        raise AttnError(st, strerror(st), "attn_fwd_masked")
    return out, lse


def attn_bwd(q, k, v, o, lse, dout, causal: bool = False, scale: float | None = None,
             dq=None, dk=None, dv=None, delta=None, noalloc: bool = False):
    """Attention backward on the GPU.

    q, k, v, o, dout: torch tensors [B, H, N, d] on one HIP device, one dtype
    (float16 or bfloat16), contiguous; o and lse (float32 [B, H, N]) are the
    forward's outputs for the same q, k, v, causal and scale.  Returns
    (dq, dk, dv), each like q.  ``delta`` is an optional float32 [B, H, N]
    workspace (written with dO_i . O_i).  ``scale`` defaults to 1/sqrt(d) rounded
    to fp32.  The call is enqueued on torch's current stream.
    """
    import torch
    ts = {"q": q, "k": k, "v": v, "o": o, "dout": dout}
    for name, t in ts.items():
        if not isinstance(t, torch.Tensor):
            raise TypeError(f"{name} must be a torch.Tensor")
        if t.device.type != "cuda":
            raise ValueError(f"{name} must be on a HIP device, got {t.device}")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
        if t.dim() != 4 or t.shape != q.shape:
            raise ValueError(f"{name} must have q's [B, H, N, d] shape {tuple(q.shape)}, got {tuple(t.shape)}")
        if t.dtype != q.dtype:
            raise TypeError("q, k, v, o, dout must share one dtype")
        if t.device != q.device:
            raise ValueError("q, k, v, o, dout must be on one device")
    code = _dtype_code(q)
    B, H, N, d = q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(d)

    def _vec(t, name):
        if t is None:
            return torch.empty((B, H, N), dtype=torch.float32, device=q.device)
        if t.shape != (B, H, N) or t.dtype != torch.float32 or not t.is_contiguous() \
                or t.device != q.device:
            raise ValueError(f"{name} must be a contiguous float32 [B, H, N] tensor on q's device")
        return t

    def _like(t, name):
        if t is None:
            return torch.empty_like(q)
        if t.shape != q.shape or t.dtype != q.dtype or not t.is_contiguous() or t.device != q.device:
            raise ValueError(f"{name} must be a contiguous tensor like q")
        return t

    if not isinstance(lse, torch.Tensor):
        raise TypeError("lse must be a torch.Tensor")
    lse = _vec(lse, "lse")
    dq, dk, dv = _like(dq, "dq"), _like(dk, "dk"), _like(dv, "dv")
    if noalloc:
        if delta is not None:
            raise ValueError("the no-allocation backward takes no delta workspace")
    else:
        delta = _vec(delta, "delta")
    with torch.cuda.device(q.device):
        stream = torch.cuda.current_stream(q.device).cuda_stream
        if noalloc:
            st = attn_bwd_noalloc_ptr(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                                      dout.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(),
                                      B, H, N, d, float(scale), int(bool(causal)), code, stream)
        else:
            st = attn_bwd_ptr(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                              dout.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(),
                              delta.data_ptr(), B, H, N, d, float(scale), int(bool(causal)), code, stream)
    if st != ATTN_OK:
        raise AttnError(st, strerror(st), "attn_bwd_noalloc" if noalloc else "attn_bwd")
    return dq, dk, dv


def attn_bwd_noalloc(q, k, v, o, lse, dout, dq, dk, dv, causal: bool = False, scale: float | None = None):
    """attn_bwd through the entry point that allocates nothing (the per-row term D
    lives in the library's fixed device scratch, B*H*N <= 2^22): for callers that
    cannot allocate.  dq, dk, dv are the caller's output tensors (like q).  Calls
    that overlap in time on one GPU race on that scratch."""
    return attn_bwd(q, k, v, o, lse, dout, causal=causal, scale=scale, dq=dq, dk=dk, dv=dv, noalloc=True)
