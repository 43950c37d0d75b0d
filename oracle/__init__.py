"""fp64 CPU oracle for Ring Attention (test infrastructure only; see ring_oracle.py).

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may import this
package.  The product path never does.
"""
from .ring_oracle import (  # noqa: F401
    LAYOUTS, allowed_mask, allowed_pairs, attend, attention_over_shards, brute_force_row, merge,
    document_of, key_grads, online_blocks, ring_order, shard_attention, shard_dq_rows, shard_grads,
    shard_tokens,
    step_attention, usp_tokens,
)
