"""NVFP4-compressed sparse-MLA decode for MI355X (gfx950).

The computation lives in the HIP library ``libmla_nvfp4.so`` (C ABI in ``include/mla_nvfp4.h``);
this package holds its build script, the ctypes binding and the seeded workload generators.
"""

from ._lib import (  # noqa: F401
    MLA_LAYOUT_BLOCK_MAJOR,
    MLA_LAYOUT_LAYER_MAJOR,
    MlaError,
    load_library,
    mla_check_dense_tables,
    mla_check_slots,
    mla_check_sparse_indices,
    mla_copy_kv_blocks,
    mla_debug_checks_enabled,
    mla_decode_workspace_size,
    mla_dense_decode,
    mla_dense_decode_num_splits,
    mla_dense_decode_split_tokens,
    mla_fp8_append,
    mla_fp8_dense_decode,
    mla_fp8_sparse_decode,
    mla_indexer_scores,
    mla_kv_transfer_regions,
    mla_nvfp4_dequantize_rows,
    mla_nvfp4_quantize_append,
    mla_nvfp4_stage_fp8,
    mla_set_debug_checks,
    mla_set_timing_events,
    mla_shared_decode_num_splits,
    mla_shared_decode_workspace_size,
    mla_sparse_decode,
    mla_sparse_decode_append,
    mla_sparse_decode_shared,
    mla_sparse_decode_num_splits,
    mla_staged_sparse_decode,
    mla_staged_workspace_size,
    mla_topk_indices,
    mla_topk_workspace_size,
)
