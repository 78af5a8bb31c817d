"""Packed block verification for block-diffusion speculative decoding on MI355X (gfx950).

The compute lives in libdsv.so (hand-written HIP kernels behind the C ABI of
include/dsv.h); this package is the thin Python binding over it.  Every entry point
loads the library on first use and raises ImportError when it has not been built
(`python -m block_verification_attention_amd.build`); there is no fallback path.
"""
from . import _lib
from ._lib import DsvError, MAX_W, STATUS_BAD_REQUEST, STATUS_BUDGET, STATUS_NAN, STATUS_POOL, STATUS_PREFILL


from .api import (
    Prefill,
    accept,
    accept_sample,
    accept_sample_workspace_bytes,
    allocate_pack,
    draft_features,
    draft_features_workspace_bytes,
    philox_uniforms,
    accept_workspace_bytes,
    attn_args,
    new_status,
    pack_slots,
    pack_verify_attn,
    verify_attn,
    verify_attn_call,
    verify_attn_noalloc_call,
    verify_attn_workspace_bytes,
)

__all__ = [
    "DsvError", "MAX_W", "STATUS_BAD_REQUEST", "STATUS_BUDGET", "STATUS_NAN", "STATUS_POOL",
    "STATUS_PREFILL", "Prefill", "accept", "accept_sample", "accept_sample_workspace_bytes",
    "accept_workspace_bytes", "allocate_pack", "attn_args",
    "draft_features", "draft_features_workspace_bytes", "philox_uniforms", "new_status",
    "pack_slots", "pack_verify_attn", "verify_attn", "verify_attn_call", "verify_attn_noalloc_call",
    "verify_attn_workspace_bytes",
]


def load_library():
    """Loads libdsv.so now (raises ImportError if it is missing); returns its path."""
    _lib.load()
    return _lib.LIB_PATH
