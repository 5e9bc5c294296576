"""Paged-attention decode on AMD Instinct MI355X (gfx950).

The computation lives in libpa.so (HIP kernels behind the C ABI in
include/pa.h); this package is its thin binding plus the seeded synthetic
input generator (workloads).
"""
from ._binding import (PAError, copy_blocks, decode, decode_cascade, decode_cascade_append,
                       decode_cascade_append_fp8, decode_cascade_fp8, decode_cascade_workspace_size, decode_fp8,
                       decode_noalloc, decode_workspace_size, load, multi_query, multi_query_fp8,
                       reshape_and_cache, reshape_and_cache_fp8, status_string, swap_blocks)

__all__ = ["PAError", "copy_blocks", "decode", "decode_cascade", "decode_cascade_append",
           "decode_cascade_append_fp8", "decode_cascade_fp8", "decode_cascade_workspace_size", "decode_fp8",
           "decode_noalloc", "decode_workspace_size", "load", "multi_query", "multi_query_fp8", "reshape_and_cache",
           "reshape_and_cache_fp8", "status_string", "swap_blocks"]
