"""fp64 reference for paged-attention decode (test infrastructure only).

Citations name the source pages by their identity and the passage:
  [cd0d9e1a]  project_6 commit cd0d9e1a, qwen3_6_scripts (commit messages)
  [prefix-doc] project_6 blame of optimizations/prefix_prefill_patch.py (docstring)

Everything is computed in float64 from exactly widened inputs. Plain loops
over (sequence, KV head); a BLAS matmul is the only library primitive used.

Readings taken where the pages are silent (each one is listed in the design
notes with its reason):
  * K/V pools are [num_blocks, num_kv_heads, 16, head_dim]; a 16-token block
    is reached through block_tables[s][t // 16], slot t % 16.
  * query head h reads KV head h // G, with G = num_heads // num_kv_heads.
  * the scale multiplies the logits before the max is taken.
  * a zero-length context gives a zero output.
  * partition p of a long context covers tokens [512 p, min(512 p + 512, L)),
    so there are ceil(L / 512) partitions (the pages' count at 100K tokens is
    one short of that ceiling; the last partition holds the remainder).
  * the per-partition output is already divided by its own exp-sum (the
    combine step multiplies by the exp-sum again, which only makes sense for
    a normalised partial).
"""
from __future__ import annotations

import numpy as np

BLOCK_SIZE = 16        # tokens per physical KV block
PARTITION_SIZE = 512   # [cd0d9e1a] V2 implementation: context split into 512-token partitions
V2_THRESHOLD = 8192    # [cd0d9e1a] paged_attn.py rewrite, item 2: contexts longer than 8192 take V2


def widen(a: np.ndarray, dtype: str) -> np.ndarray:
    """Exact float64 view of stored values ("f32" / "f16" floats or "bf16" uint16 bit patterns)."""
    if dtype == "f32":
        return np.asarray(a, dtype=np.float32).astype(np.float64)
    if dtype == "f16":
        return np.asarray(a, dtype=np.float16).astype(np.float64)
    if dtype == "bf16":
        bits = np.asarray(a, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
        return bits.view(np.float32).astype(np.float64)
    raise ValueError(f"unsupported dtype {dtype!r}")


def gather_list(block_tables: np.ndarray, seq_lens: np.ndarray, block_size: int = BLOCK_SIZE):
    """Physical block ids each sequence's context occupies, in logical order.

    [cd0d9e1a] paged_attn.py rewrite, item 1: the context's K/V are fetched
    by indexing the cache with the sequence's block ids.
    """
    out = []
    for s, L in enumerate(np.asarray(seq_lens).reshape(-1)):
        n = (int(L) + block_size - 1) // block_size if L > 0 else 0
        out.append(np.asarray(block_tables[s, :n], dtype=np.int64).copy())
    return out


def gather_kv(cache: np.ndarray, block_ids: np.ndarray, kv_head: int, L: int, dtype: str) -> np.ndarray:
    """[L, D] float64 rows t = 0..L-1 of one KV head, token t in block t // 16, slot t % 16."""
    D = cache.shape[-1]
    if L <= 0:
        return np.zeros((0, D), dtype=np.float64)
    rows = cache[block_ids, kv_head]                  # [nblk, 16, D]
    rows = rows.reshape(-1, D)[:L]
    return widen(rows, dtype)


def _softmax_weighted_sum(z: np.ndarray, V: np.ndarray):
    """For logits z [G, L] and values V [L, D]: (max m [G], exp-sum l [G], normalised out [G, D])."""
    m = z.max(axis=1)
    w = np.exp(z - m[:, None])
    l = w.sum(axis=1)
    o = (w @ V) / l[:, None]
    return m, l, o


def attend_seq(q_s: np.ndarray, k_cache, v_cache, block_ids, L: int, scale: float, dtype: str) -> np.ndarray:
    """Decode attention for one sequence: q_s [H, D] (stored dtype) -> out [H, D] float64.

    [cd0d9e1a] V2 implementation, phase 1 names the per-head computation: a
    dot product of the query with every context key, a softmax over the
    context, and the softmax-weighted sum of the values. Done here over the
    whole context at once, which is what the single-pass V1 computes.
    """
    H, D = q_s.shape
    Hkv = k_cache.shape[1]
    G = H // Hkv
    out = np.zeros((H, D), dtype=np.float64)
    if L <= 0:
        return out
    qf = widen(q_s, dtype)
    for kv in range(Hkv):
        K = gather_kv(k_cache, block_ids, kv, L, dtype)
        V = gather_kv(v_cache, block_ids, kv, L, dtype)
        z = scale * (qf[kv * G:(kv + 1) * G] @ K.T)      # [G, L]
        _, _, o = _softmax_weighted_sum(z, V)
        out[kv * G:(kv + 1) * G] = o
    return out


def attend_dense(q, k_cache, v_cache, block_tables, seq_lens, scale: float, dtype: str) -> np.ndarray:
    """Plain definition for a whole batch: out [S, H, D] float64."""
    lists = gather_list(block_tables, seq_lens)
    S, H, D = q.shape
    out = np.zeros((S, H, D), dtype=np.float64)
    for s in range(S):
        out[s] = attend_seq(q[s], k_cache, v_cache, lists[s], int(seq_lens[s]), scale, dtype)
    return out


def choose_path(L: int, threshold: int = V2_THRESHOLD) -> str:
    """Per-sequence path: "v2" when the context is longer than the threshold, else "v1".

    [cd0d9e1a] paged_attn.py rewrite, item 2 (the heuristic restored there).
    """
    return "v2" if int(L) > threshold else "v1"


def num_partitions(L: int, partition_size: int = PARTITION_SIZE) -> int:
    """ceil(L / partition_size): every token falls in exactly one partition."""
    L = int(L)
    return 0 if L <= 0 else (L + partition_size - 1) // partition_size


def partition_stats(q_s, k_cache, v_cache, block_ids, L: int, scale: float, dtype: str,
                    partition_size: int = PARTITION_SIZE):
    """Phase-1 partials for one sequence.

    [cd0d9e1a] V2 implementation, phase 1: for each (head, partition) the
    logits, softmax and weighted V sum over that partition's tokens, kept as
    three partials: max logit m_p, exp-sum l_p = sum exp(z - m_p), and the
    output o_p (normalised by l_p). Returns (m [H, P], l [H, P], o [H, P, D]).
    """
    H, D = q_s.shape
    Hkv = k_cache.shape[1]
    G = H // Hkv
    P = num_partitions(L, partition_size)
    m = np.zeros((H, P)); l = np.zeros((H, P)); o = np.zeros((H, P, D))
    qf = widen(q_s, dtype)
    for kv in range(Hkv):
        K = gather_kv(k_cache, block_ids, kv, L, dtype)
        V = gather_kv(v_cache, block_ids, kv, L, dtype)
        for p in range(P):
            lo, hi = p * partition_size, min((p + 1) * partition_size, L)
            z = scale * (qf[kv * G:(kv + 1) * G] @ K[lo:hi].T)
            mp, lp, op = _softmax_weighted_sum(z, V[lo:hi])
            m[kv * G:(kv + 1) * G, p] = mp
            l[kv * G:(kv + 1) * G, p] = lp
            o[kv * G:(kv + 1) * G, p] = op
    return m, l, o


def lse_combine(m: np.ndarray, l: np.ndarray, o: np.ndarray) -> np.ndarray:
    """Phase 2 for one (sequence, head): m [P], l [P], o [P, D] -> out [D].

    [cd0d9e1a] V2 implementation, phase 2: take the largest partition max,
    weight each partition by exp(its max minus that global max) times its
    exp-sum, and average the partition outputs with those weights divided by
    their total.
    """
    if m.size == 0:
        return np.zeros(o.shape[-1])
    M = m.max()
    c = np.exp(m - M) * l
    return (c[:, None] * o).sum(axis=0) / c.sum()


def attend_v2_seq(q_s, k_cache, v_cache, block_ids, L: int, scale: float, dtype: str,
                  partition_size: int = PARTITION_SIZE):
    """Two-phase (partitioned) form for one sequence: (out [H, D], (m, l, o))."""
    m, l, o = partition_stats(q_s, k_cache, v_cache, block_ids, L, scale, dtype, partition_size)
    H, D = q_s.shape
    out = np.zeros((H, D))
    for h in range(H):
        out[h] = lse_combine(m[h], l[h], o[h])
    return out, (m, l, o)


def attend_v2(q, k_cache, v_cache, block_tables, seq_lens, scale: float, dtype: str,
              partition_size: int = PARTITION_SIZE) -> np.ndarray:
    """Two-phase form for a whole batch: out [S, H, D] float64."""
    lists = gather_list(block_tables, seq_lens)
    S, H, D = q.shape
    out = np.zeros((S, H, D))
    for s in range(S):
        out[s], _ = attend_v2_seq(q[s], k_cache, v_cache, lists[s], int(seq_lens[s]), scale, dtype,
                                  partition_size)
    return out
