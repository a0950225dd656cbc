"""Launch-shape choices shared by the benchmark and the full-size parity tests.

The only free launch parameter of ``pa_decode`` is the partition size.  A
partition is the unit of work of one workgroup; splitting a long context gives
the 256 compute units enough workgroups when (sequences x KV heads) alone is
too few, at the price of a second small kernel (``pa_reduce``).
"""
from __future__ import annotations

NUM_CUS = 256
BLOCK_SIZE = 16


def round_up(x: int, m: int) -> int:
    return -(-x // m) * m


def choose_partition_size(num_seqs: int, num_kv_heads: int, max_context_len: int,
                          target_workgroups: int = 4 * NUM_CUS, min_partition: int = 256) -> int:
    """0 (single phase) when sequences x KV heads already fill the chip, else the
    largest multiple of 16 (at least ``min_partition``) that reaches about
    ``target_workgroups`` workgroups."""
    units = num_seqs * num_kv_heads
    if units >= target_workgroups or max_context_len <= min_partition:
        return 0
    parts = -(-target_workgroups // units)
    size = round_up(-(-max_context_len // parts), BLOCK_SIZE)
    size = max(size, min_partition)
    return 0 if size >= max_context_len else size


def partition_for(workload) -> int:
    """Partition size a workload runs with: its own if it names one, else the choice above."""
    if workload.partition_size:
        return workload.partition_size
    return choose_partition_size(workload.num_seqs, workload.num_kv_heads, workload.max_context_len)
