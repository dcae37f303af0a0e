"""Shared-latent MLA attention forward for AMD Instinct MI355X (gfx950).

The compute runs in libmla355.so (hand-written HIP kernels behind a C ABI,
declared in include/mla355.h); this package is its Python binding.  Importing
it loads the library and raises if it has not been built
(``python ring_chunk_attention_amd/build.py``).
"""
from .binding import (EXPORTS, LIB_PATH, MAX_GROUP, MlaError, debug_gather, decode_fwd, fwd, fwd_fp8, fwd_group,
                      merge, ring_fwd, ring_order, ring_schedule,
                      ring_workspace_size, sparse_fwd, split_fwd, version, vup)

__all__ = ["EXPORTS", "LIB_PATH", "MAX_GROUP", "MlaError", "debug_gather", "decode_fwd", "fwd", "fwd_fp8",
           "fwd_group", "merge", "ring_fwd", "ring_order", "ring_schedule", "ring_workspace_size", "sparse_fwd",
           "split_fwd", "version", "vup"]
