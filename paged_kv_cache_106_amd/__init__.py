"""Paged-KV-cache decode attention for AMD Instinct MI355X (gfx950).

The product is libpa.so (HIP kernels + C ABI + host block allocator, declared
in include/pa.h).  This package is its thin Python binding: the names follow
the C ABI, torch tensors supply device memory and the current HIP stream.
Importing fails loudly when libpa.so has not been built; there is no CPU
fallback.
"""
from ._native import (  # noqa: F401
    LIB_PATH,
    PA_BF16,
    PA_F16,
    Allocator,
    PaError,
    PaOOM,
    lib,
    pa_copy_blocks,
    pa_copy_blocks_int8,
    pa_decode,
    pa_decode_int8,
    pa_decode_partitioned,
    pa_decode_partitioned_int8,
    pa_decode_partitioned_noalloc,
    pa_decode_partitioned_noalloc_max_workspace,
    pa_decode_partitioned_workspace_size,
    pa_prefill,
    pa_reshape_and_cache,
    pa_reshape_and_cache_int8,
    pa_update_block_tables,
    pa_write_step,
    pa_write_step_int8,
    partition_work_items,
)

__all__ = [
    "Allocator", "PaError", "PaOOM", "PA_F16", "PA_BF16", "lib", "pa_copy_blocks",
    "pa_copy_blocks_int8", "pa_decode", "pa_decode_int8", "pa_decode_partitioned",
    "pa_decode_partitioned_int8", "pa_decode_partitioned_noalloc",
    "pa_decode_partitioned_noalloc_max_workspace", "pa_decode_partitioned_workspace_size",
    "pa_prefill",
    "pa_reshape_and_cache",
    "pa_reshape_and_cache_int8", "pa_update_block_tables", "pa_write_step",
    "pa_write_step_int8", "partition_work_items",
]
