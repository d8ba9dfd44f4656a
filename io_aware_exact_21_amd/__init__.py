"""Exact FlashAttention forward, backward and split-KV decode for AMD Instinct MI355X (gfx950).

The computation lives in hand-written HIP kernels behind a C ABI (include/fa.h,
libfa.so). This package is the thin Python binding: it checks tensors, passes
pointers and the current HIP stream, and raises on any library error. Importing
it loads libfa.so and fails loudly if the library is not built.
"""
from . import _lib
from .api import (bpt_layer, bpt_workspace_bytes, bwd, bwd_workspace_bytes, decode, decode_chunk_bounds, decode_combine, decode_default_splits,
                  decode_noalloc,
                  decode_paged, decode_paged_default_splits, decode_partials, decode_workspace_bytes, fwd,
                  fwd_fp8)

_lib.load()

__all__ = ["fwd", "fwd_fp8", "bwd", "bpt_layer", "bpt_workspace_bytes", "bwd_workspace_bytes", "decode", "decode_paged", "decode_paged_default_splits",
           "decode_partials", "decode_combine", "decode_noalloc", "decode_default_splits", "decode_workspace_bytes",
           "decode_chunk_bounds"]
