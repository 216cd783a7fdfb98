"""CSA2 FP4 (E2M1) compressed-sparse-attention hot path for AMD MI355X.

The kernels are hand-written HIP for gfx950 in ``csrc/``, exported through
the C ABI declared in ``include/csa2.h`` (libcsa2.so).  This package is the
thin Python binding: the functions carry the C names and only marshal torch
tensors (device memory) and the current HIP stream.
"""
from ._binding import (NOALLOC_SCRATCH_BYTES, CSA2_OP_INDEX_FULL, CSA2_OP_INDEX_POOL, CSA2_OP_INDEX_REINDEX, Cache,
                       Csa2Error, Swa, attn_workspace, block_keys_buffer,
                       csa2_attn_workspace_size, csa2_cache_append, csa2_cache_export,
                       csa2_cache_import, csa2_index_full, csa2_index_full_noalloc, csa2_index_pool,
                       csa2_index_reindex, csa2_index_scan, csa2_index_scan_append, csa2_quantize_fp4, csa2_sparse_attn,
                       csa2_swa_merge, csa2_workspace_size, load, version, workspace)

__all__ = [
    "NOALLOC_SCRATCH_BYTES",
    "CSA2_OP_INDEX_FULL", "CSA2_OP_INDEX_POOL", "CSA2_OP_INDEX_REINDEX", "Cache", "Csa2Error",
    "Swa", "attn_workspace", "block_keys_buffer", "csa2_attn_workspace_size", "csa2_cache_append", "csa2_cache_export",
    "csa2_cache_import", "csa2_index_full", "csa2_index_full_noalloc", "csa2_index_pool", "csa2_index_reindex",
    "csa2_index_scan", "csa2_index_scan_append", "csa2_quantize_fp4", "csa2_sparse_attn",
    "csa2_swa_merge", "csa2_workspace_size", "load", "version", "workspace",
]
