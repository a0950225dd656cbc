"""Launch-shape choices shared by the benchmark and the full-size parity tests.

The only free launch parameter of ``pa_decode`` is the partition size.  A
partition is the unit of work of one workgroup; splitting a long context gives
the 256 compute units enough workgroups when (sequences x KV heads) alone is
too few, at the price of partial results and a second small kernel
(``pa_reduce``).  The rules below were read off measured sweeps on MI355X
(partition sizes 0 / 256 / 512 / 1024 / 2048 on every workload shape).
"""
from __future__ import annotations

BLOCK_SIZE = 16
MIN_UNITS = 512          # workgroups below which a context is split
LONG_CONTEXT = 3072      # unsplit partitions this long stream well
SPLIT_TOKENS = 1024      # smallest partition used when splitting


def round_up(x: int, m: int) -> int:
    return -(-x // m) * m


def choose_partition_size(num_seqs: int, num_q_heads: int, num_kv_heads: int,
                          max_context_len: int) -> int:
    """0 (single phase) or a partition size in tokens (a multiple of 16)."""
    chunks = -(-(num_q_heads // num_kv_heads) // 16)   # 16 query heads per workgroup
    units = num_seqs * num_kv_heads * chunks
    if max_context_len <= SPLIT_TOKENS:
        return 0
    if units >= MIN_UNITS:
        # enough workgroups: keep long contexts whole, cut mid-length ones in
        # 1024-token pieces so the ragged tails even out
        return 0 if max_context_len >= LONG_CONTEXT else SPLIT_TOKENS
    parts = -(-MIN_UNITS // units)
    size = max(SPLIT_TOKENS, round_up(-(-max_context_len // parts), BLOCK_SIZE))
    return 0 if size >= max_context_len else size


def partition_for(workload, own: bool = True) -> int:
    """Partition size a workload runs with: its own if it names one (and ``own``),
    else the choice above."""
    if own and workload.partition_size:
        return workload.partition_size
    return choose_partition_size(workload.num_seqs, workload.num_q_heads, workload.num_kv_heads,
                                 workload.max_context_len)
