"""Exact scaled-dot-product attention (forward and backward) for MI355X (gfx950).

The computation runs in the HIP library ``libattn.so`` (C ABI in
include/attn.h); this package holds its ctypes binding, the in-tree build and
the seeded workload generators.
"""
from ._binding import (ATTN_BF16, ATTN_EHIP, ATTN_EINVAL, ATTN_ESCRATCH, ATTN_EUNSUPPORTED, ATTN_F16,
                       ATTN_F32, ATTN_OK, AttnError, abi_version, attn_bwd, attn_bwd_ptr,
                       attn_bwd_noalloc, attn_bwd_noalloc_ptr,
                       attn_fwd, attn_fwd_masked, attn_fwd_masked_ptr, attn_fwd_ptr,
                       attn_mask_pack_ptr, pack_mask, PackedMask, strerror,
                       attn_linear_fwd, attn_linear_fwd_ptr, linear_workspace_bytes)

__all__ = ["attn_fwd", "attn_fwd_ptr", "attn_fwd_masked", "attn_fwd_masked_ptr", "pack_mask", "PackedMask",
           "attn_linear_fwd", "attn_linear_fwd_ptr", "linear_workspace_bytes",
           "attn_mask_pack_ptr", "attn_bwd", "attn_bwd_ptr", "attn_bwd_noalloc", "attn_bwd_noalloc_ptr",
           "abi_version", "strerror",
           "AttnError", "ATTN_F32", "ATTN_F16", "ATTN_BF16", "ATTN_OK", "ATTN_EINVAL",
           "ATTN_EUNSUPPORTED", "ATTN_EHIP", "ATTN_ESCRATCH"]
