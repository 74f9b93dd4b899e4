"""MI355X-native (gfx950) bf16 attention forward.

The product is the C-ABI library ``libattn_fwd.so`` (declared in
``include/attn_fwd.h``) built from ``csrc/`` by ``build.py``.  This package
holds the thin ctypes binding with the same entry-point names and the
seeded workload generators.  Importing it does not load the library; the
first call does, and raises if it is not built.
"""
from .binding import (AttnError, attn_bwd_bf16, attn_fwd_bf16, attn_fwd_bf16_gqa, attn_fwd_bf16_hd,  # noqa: F401
                      attn_fwd_bf16_hd_noalloc, attn_fwd_bf16_paged, attn_fwd_bf16_raw, attn_fwd_bf16_varlen,
                      attn_status_string, attn_version,
                      load_library, LIB_PATH, EXPORTS, NOALLOC_SCRATCH_BYTES)

__all__ = ["attn_fwd_bf16", "attn_fwd_bf16_gqa", "attn_fwd_bf16_hd", "attn_fwd_bf16_hd_noalloc", "attn_fwd_bf16_paged",
           "attn_fwd_bf16_varlen", "attn_bwd_bf16", "attn_fwd_bf16_raw", "attn_status_string",
           "attn_version", "load_library", "AttnError", "LIB_PATH", "EXPORTS"]
