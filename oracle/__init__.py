"""CPU float64 oracle for the paged KV-cache decode path (test infrastructure only).

Imported by tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg;
never by the GPU library.  oracle/oracle.py holds the decode step (slot write,
paged attention); oracle/block_manager.py the block pool (allocation, reference
counts, copy-on-write, freeing) and the block copy.
"""
from .oracle import (  # noqa: F401
    BF16, F16, F32, attend, blocks_needed, decode, decode_split, gather_sequence, kv_write,
    lse_merge, newest_token_slots, partition_state, prefill, slot_to_block_offset, to_float64,
)
