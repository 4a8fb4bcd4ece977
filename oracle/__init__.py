"""CPU oracle for the paged KV-cache transfer path.

TEST INFRASTRUCTURE ONLY. Only the test suite, the smoke check and the benchmark's
CPU-baseline leg may import this package. The product path (the HIP library and its
Python binding) never imports, links or calls anything here, and this package imports
nothing from the product.

Every function is the plain definition of one step, written as obvious loops over
requests, blocks and rows with numpy slice copies; nothing is blocked, fused or
reordered beyond what the definition says. All data movement is on raw bytes
(uint8 views), so results are bit-exact by construction; there is no floating-point
arithmetic anywhere in the path.
"""
from .kv_oracle import (  # noqa: F401
    DEVERR_BLOCK_RANGE,
    DEVERR_OFFSETS,
    DEVERR_SLOT_RANGE,
    DEVERR_TABLE_RANGE,
    MODE_DIRECT,
    MODE_PACK,
    MODE_UNPACK,
    buffer_order,
    copy_direct,
    pack,
    pack_kv_first,
    pack_split,
    reshape_and_cache,
    slot_mapping,
    split_block,
    unpack,
    unpack_block,
    unpack_kv_first,
    xfer_list,
)
