"""fp64 CPU oracle for paged-attention decode, prefix/chunked prefill over the
same paged cache, and the MoE routing path. TEST INFRASTRUCTURE ONLY.

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may use
this package. The library (paged_attention_decode_06_amd) never imports it and
it never imports the library: the two share no code.

Every function is pinned by CPU tests (tests/test_oracle.py,
tests/test_oracle_prefill.py, tests/test_oracle_moe.py) to brute force,
library routines (torch scaled_dot_product_attention in fp64, torch topk and
softmax, einsum over a dense routing matrix), closed forms
and invariants. No function here is "parity unpinned".
"""
from .attention import (  # noqa: F401
    BLOCK_SIZE, PARTITION_SIZE, V2_THRESHOLD,
    widen, gather_list, gather_kv, attend_seq, attend_dense,
    choose_path, num_partitions, partition_stats, attend_v2_seq, attend_v2,
    lse_combine,
)
from .prefill import (  # noqa: F401
    query_positions, attend_prefill_seq, attend_prefill, attend_prefill_row,
)
from . import moe  # noqa: F401  (topk_softmax, sort_by_expert, permute_rows, combine)
