"""Paged KV-cache decode attention, KV append and block management for MI355X
(gfx950).

The computation lives in hand-written HIP kernels behind the C ABI of
libpagedkv.so (include/pagedkv.h); this package is its Python binding.
"""
from ._lib import (  # noqa: F401
    DTYPE_BF16,
    BlockManager,
    OutOfBlocksError,
    copy_blocks,
    DTYPE_F32,
    LIB_PATH,
    SIGNATURES,
    DecodeAppendCall,
    DecodeCall,
    PagedKVError,
    append,
    append_at,
    decode,
    decode_append,
    decode_noalloc,
    decode_shared,
    DecodeSharedCall,
    shared_workspace_size,
    STAGE_PREPARE,
    STAGE_ATTEND,
    STAGE_MERGE,
    STAGES_ALL,
    NOALLOC_SCRATCH_BYTES,
    load_library,
    plan,
    prefill,
    slot_mapping,
    status_str,
    swap_in,
    swap_out,
    swap_staging_bytes,
    workspace_size,
)
