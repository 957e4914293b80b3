"""Paged-attention decode for MI355X (gfx950).

The compute path is the HIP library libpa_decode.so (include/pa_decode.h:
decode and prefill attention over the paged cache; include/pa_moe.h: the MoE
routing path; include/pa_probe.h: measurement kernels beside the path);
this package is its thin ctypes binding plus the seeded input generators
(`workloads`). Build the library with `python -m paged_attention_decode_06_amd._build`.
"""
from ._lib import (  # noqa: F401
    BLOCK_SIZE, HipEvents, PARTITION_SIZE, V2_THRESHOLD, MODE_AUTO, MODE_V1, MODE_V2, PA_F32, PA_BF16, PA_F16,
    PaError, PaShape, alloc_partials, load, make_shape, max_partitions, pa_decode, pa_decode_noalloc,
    pa_decode_partitions,
    pa_decode_partitions_debug, pa_decode_partitions_timed, pa_decode_v1, pa_decode_v2, pa_lse_reduce,
    pa_lse_reduce_timed, pa_prefill, status_string, check_sizes,
    pa_probe_empty, pa_probe_paged_read, probe_read_grid,
    pa_moe_topk_softmax, moe_sort_workspace_bytes, pa_moe_sort_by_expert, pa_moe_permute, pa_moe_combine,
)
