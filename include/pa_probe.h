/*
 * pa_probe.h — measurement kernels beside the decode path (not part of it).
 *
 * They give the floors against which the decode kernels are measured on
 * this GPU: what one kernel launch costs when it does nothing, and how fast the
 * bytes the decode must read (K and V of every context token, per KV head, in
 * the block order of the tables) can be read when nothing else is done with
 * them. The decode reads exactly these bytes (the roofline of the
 * "bandwidth-limited" path: project_6 blame of
 * optimizations/prefix_prefill_patch.py, hardware part of the docstring, and
 * project_6 commit cd0d9e1a, "V2 implementation").
 *
 * Memory and ownership as in pa_decode.h: device pointers owned by the
 * caller, nothing allocated or freed, asynchronous on `stream`. `start` and
 * `stop` are optional hipEvent_t handles recorded at the start and the end
 * of the kernel's own dispatch (NULL: none).
 */
#ifndef PA_PROBE_H
#define PA_PROBE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* One workgroup of one wave that returns at once. Returns 0 or PA_EHIP. */
int pa_probe_empty(void* start, void* stop, void* stream);

/* Read-only pass over `num_ids` blocks of both caches at every KV head:
 * unit u < num_ids * num_kv_heads reads k_cache and v_cache at block
 * block_ids[u % num_ids], head u / num_ids: 16 * head_dim * elem_bytes
 * bytes each, the same bytes the decode reads for those blocks. Workgroups
 * of 256 threads take `units_per_wg` consecutive units each. Nothing is
 * computed with the data beyond an xor fold; `sink` (one uint32 per
 * workgroup, device memory) is written only if a fold hits a fixed 32-bit
 * value, which keeps the loads without costing stores.
 * Caches [num_blocks, num_kv_heads, 16, head_dim] as in pa_decode.h;
 * block_ids int32 device array, every entry in [0, num_blocks) (checked on
 * the device: entries outside read block 0). elem_bytes 2 or 4, head_dim 128
 * or 256. Returns 0, PA_EINVAL (null pointer, bad size, sink smaller than
 * the grid, given as sink_words) or PA_EHIP. */
int pa_probe_paged_read(const void* k_cache, const void* v_cache, const int32_t* block_ids, int64_t num_ids,
                        int32_t num_kv_heads, int32_t head_dim, int32_t elem_bytes, int64_t num_blocks,
                        int32_t units_per_wg, uint32_t* sink, int64_t sink_words, void* start, void* stop,
                        void* stream);

/* Workgroups pa_probe_paged_read launches for these sizes (to size `sink`). */
int64_t pa_probe_paged_read_grid(int64_t num_ids, int32_t num_kv_heads, int32_t units_per_wg);

#ifdef __cplusplus
}
#endif
#endif
