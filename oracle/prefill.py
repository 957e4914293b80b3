"""fp64 reference for prefix / chunked-prefill attention over the paged cache
(test infrastructure only).

Source pages:
  [cd0d9e1a]   project_6 commit cd0d9e1a, qwen3_6_scripts: the
               "paged_attn.py rewrite" item 1 (the prefix path gathers the
               whole context's K/V from the cache once, then walks query
               tiles over it) and "patch_enable_triton.py" (prefill as one
               launch of flash attention with the online softmax).
  [prefix-doc] project_6 blame of optimizations/prefix_prefill_patch.py: the
               prefix-prefill kernel tiles query positions (BLOCK_M) against
               key/value tiles (BLOCK_N) of the context, head_dim 128/256, GQA,
               fp16/bf16; chunked prefill splits a prompt into chunks.

Reading (the pages give no formula for this step; this is the plainest one
the rest supports, and the design notes list it):
  * sequence s holds L_s tokens in the paged cache, the last Q_s of which are
    the chunk being prefilled now; their K/V are already in the cache.
  * query token i of the chunk (0 <= i < Q_s) sits at position
    pos = L_s - Q_s + i and attends to every cached token t <= pos (its
    prefix plus the chunk's earlier tokens and itself: causal).
  * a token with pos < 0 (a chunk longer than its sequence) attends to
    nothing and gets a zero output.
  * q and out are packed by token: rows query_start_loc[s] ..
    query_start_loc[s+1]-1 belong to sequence s; each row is [H, D].
  * head h reads KV head h // G, as in decode; the scale multiplies the
    logits before the max.

For a single query token (Q_s = 1) this is exactly decode attention over the
whole context.
"""
from __future__ import annotations

import numpy as np

from .attention import gather_kv, gather_list, widen


def query_positions(L: int, Q: int) -> np.ndarray:
    """Cache positions of the chunk's query tokens: L - Q, ..., L - 1."""
    return np.arange(L - Q, L, dtype=np.int64)


def attend_prefill_seq(q_rows: np.ndarray, k_cache, v_cache, block_ids, L: int, scale: float,
                       dtype: str) -> np.ndarray:
    """One sequence's chunk: q_rows [Q, H, D] (stored dtype) -> out [Q, H, D] float64.

    Per KV head: logits Z = scale * Q_g K^T over the whole context, keys
    after a token's own position masked out, softmax per row, then the
    weighted sum of V. The masked matrix is built in full (no tiling).
    """
    Q, H, D = q_rows.shape
    Hkv = k_cache.shape[1]
    G = H // Hkv
    out = np.zeros((Q, H, D), dtype=np.float64)
    if Q == 0 or L <= 0:
        return out
    pos = query_positions(L, Q)
    live = pos >= 0
    if not live.any():
        return out
    qf = widen(q_rows, dtype)
    t = np.arange(L, dtype=np.int64)
    allowed = t[None, :] <= pos[:, None]                     # [Q, L] causal over the context
    for kv in range(Hkv):
        K = gather_kv(k_cache, block_ids, kv, L, dtype)      # [L, D]
        V = gather_kv(v_cache, block_ids, kv, L, dtype)
        for g in range(G):
            h = kv * G + g
            z = scale * (qf[:, h, :] @ K.T)                  # [Q, L]
            z = np.where(allowed, z, -np.inf)
            zl = z[live]
            m = zl.max(axis=1, keepdims=True)
            w = np.exp(zl - m)
            out[live, h, :] = (w @ V) / w.sum(axis=1, keepdims=True)
    return out


def attend_prefill(q, k_cache, v_cache, block_tables, seq_lens, query_start_loc, scale: float,
                   dtype: str) -> np.ndarray:
    """Whole batch: q [T, H, D] packed by token -> out [T, H, D] float64."""
    lists = gather_list(block_tables, seq_lens)
    qsl = np.asarray(query_start_loc, dtype=np.int64)
    out = np.zeros(q.shape, dtype=np.float64)
    for s in range(len(lists)):
        a, b = int(qsl[s]), int(qsl[s + 1])
        out[a:b] = attend_prefill_seq(q[a:b], k_cache, v_cache, lists[s], int(seq_lens[s]), scale, dtype)
    return out


def attend_prefill_row(q_row: np.ndarray, k_cache, v_cache, block_ids, pos: int, scale: float,
                       dtype: str) -> np.ndarray:
    """One query token at position pos: q_row [H, D] -> [H, D] float64 over keys 0..pos.

    The same definition for a single row (used to check sampled rows of
    workloads too large to compute whole).
    """
    H, D = q_row.shape
    out = np.zeros((H, D), dtype=np.float64)
    if pos < 0:
        return out
    return attend_prefill_seq(q_row[None], k_cache, v_cache, block_ids, pos + 1, scale, dtype)[0]
