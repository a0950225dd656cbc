"""fp64 CPU oracle for paged decode attention.

TEST INFRASTRUCTURE: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import it; the library never does.
"""
from .paged_attention import (  # noqa: F401
    BLOCK_SIZE, widen, slot_of, slot_ids, tile_byte_offset, k_rows, v_rows, attend_range,
    paged_decode, num_partitions, paged_decode_partials, merge_partials, write_kv,
    copy_blocks, gather_blocks, scatter_blocks, draft_limit, paged_verify, paged_verify_partials,
)
from .dense import dense_attention  # noqa: F401
