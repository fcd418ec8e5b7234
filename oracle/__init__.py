"""fp64 CPU oracle for paged decode attention and KV append.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the benchmark's
CPU-baseline leg may import this package.  The product path (the HIP library
and its Python binding) never imports it and shares no code with it.

Every function here is pinned by a CPU test against something other than
itself (worked examples printed on the pages, closed forms, invariants,
library routines, brute force); none is "parity unpinned".
"""
from .paged_attention import (  # noqa: F401
    decode_storage,
    slot_of,
    kv_head_of,
    oracle_slot_mapping,
    oracle_append,
    gather_context,
    softmax_attention,
    oracle_decode,
    oracle_decode_sampled,
)
from .block_manager import OutOfBlocks, RefBlockManager, copy_blocks  # noqa: F401,E402
