"""Paged-attention hot path for AMD Instinct MI355X (gfx950).

The work runs in hand-written HIP kernels behind the C ABI of include/pa.h (libpa.so); this package
is the thin Python binding over it. See binding.py for the entry points.
"""
from .binding import (BLOCK_SIZE, PAError, alloc_decode_workspace, copy_blocks, decode,  # noqa: F401
                      decode_fp8, decode_shared_prefix, decode_shared_prefix_workspace_size,
                      decode_workspace_size, default_partition_size, lib, prefill_chunk,
                      reshape_and_cache, reshape_and_cache_fp8)
