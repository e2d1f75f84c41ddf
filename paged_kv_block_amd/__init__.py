"""paged_kv_block_amd -- paged / block-sparse attention for AMD Instinct MI355X.

The compute lives in libpkb.so (hand-written gfx950 HIP kernels behind a C ABI,
declared in include/pkb.h).  This package is the thin torch binding: importing
it loads the library and fails loudly if it has not been built.
"""
from . import _lib
from ._lib import PkbError, lib

lib()  # load now: no fallback path exists

from .ops import (  # noqa: E402
    BatchPrefillPagedWrapper,
    BlockSparsePagedWrapper,
    batch_decode_with_paged_kv_cache,
    batch_prefill_with_paged_kv_cache,
    block_sparse_attention_with_paged_kv_cache,
    bsa_attn_blk64_sage_fwd,
    bsa_plan,
    bsa_run,
    bsa_sage_run,
    bsa_sage_validate,
    bsa_validate,
    num_cus,
    paged_decode_q_run,
    paged_decode_q_validate,
    paged_decode_q_workspace_size,
    paged_decode_run,
    paged_decode_run_noalloc,
    paged_decode_validate,
    paged_decode_workspace_size,
    paged_prefill_plan,
    paged_prefill_plan_capacity,
    paged_prefill_run,
    paged_prefill_validate,
    qsa_forward,
    qsa_run,
    qsa_validate,
    split_kv_cache,
)

__all__ = [
    "PkbError", "lib", "BatchPrefillPagedWrapper", "BlockSparsePagedWrapper",
    "batch_decode_with_paged_kv_cache", "batch_prefill_with_paged_kv_cache",
    "block_sparse_attention_with_paged_kv_cache", "bsa_attn_blk64_sage_fwd", "bsa_plan",
    "bsa_run", "bsa_sage_run", "bsa_sage_validate", "bsa_validate", "num_cus",
    "paged_decode_q_run", "paged_decode_q_validate", "paged_decode_q_workspace_size",
    "paged_decode_run", "paged_decode_run_noalloc", "paged_decode_validate", "paged_decode_workspace_size",
    "paged_prefill_plan", "paged_prefill_plan_capacity", "paged_prefill_run",
    "paged_prefill_validate", "qsa_forward", "qsa_run", "qsa_validate", "split_kv_cache",
]
