"""fp64 / exact-integer reference for the MoE routing path (test infrastructure only).

Source pages:
  [cd0d9e1a]  project_6 commit cd0d9e1a, qwen3_6_scripts: the MoE prefill
              rewrite (256 experts, top_k = 8): flatten the T x K
              token-expert assignments, sort them by expert id so every
              expert's tokens are contiguous, run each expert on its
              contiguous rows, and add the weighted expert outputs back to
              their tokens in one scatter (index_add_).
  [490ff98a]  project_6 commit 490ff98a, Dockerfile: the router's
              topk_softmax kernel (softmax over the experts, then the top k).

Readings (the pages name the steps, not their exact conventions; each is
listed in the design notes):
  * topk_softmax: probabilities p = softmax(logits) over all E experts in
    float64; the k experts with the largest logits are chosen (softmax keeps
    the order, so this is the top k of p), in descending order, a tie going
    to the lower expert id. The selection compares the stored fp32 logits
    exactly, so it is the same decision in any precision. Weights are the
    chosen p, or p / sum of the chosen p with renormalize.
  * sort by expert: the T*K pairs, pair index a = t*K + j, are ordered by
    expert id, stably (ascending a within an expert); expert_offsets[e] is
    where expert e's range starts (E + 1 entries, the last = T*K).
  * permute: row i of the sorted input is the hidden row of the token of
    sorted pair i.
  * combine (the scatter-back): out[t] = sum over j of w[t, j] * y[pos(t, j)],
    y the expert outputs in sorted order, pos(t, j) the sorted position of
    pair t*K + j; the sum over j runs in order j = 0..K-1.
  The expert GEMMs and their activation sit between permute and combine and
  need trained weights: they are not part of this path.
"""
from __future__ import annotations

import numpy as np


def topk_softmax(logits: np.ndarray, k: int, renormalize: bool = False):
    """logits float32 [T, E] -> (weights float64 [T, k], ids int32 [T, k])."""
    lg = np.asarray(logits, dtype=np.float32)
    T, E = lg.shape
    z = lg.astype(np.float64)
    p = np.exp(z - z.max(axis=1, keepdims=True))
    p /= p.sum(axis=1, keepdims=True)
    # descending by logit, ties to the lower id: a stable sort on (-logit)
    order = np.argsort(-z, axis=1, kind="stable")[:, :k]
    w = np.take_along_axis(p, order, axis=1)
    if renormalize:
        w = w / w.sum(axis=1, keepdims=True)
    return w, order.astype(np.int32)


def sort_by_expert(topk_ids: np.ndarray, num_experts: int):
    """ids int32 [T, K] -> (sorted_pairs int32 [T*K], pair_pos int32 [T*K], expert_offsets int32 [E+1]).

    sorted_pairs[i] = the pair index a = t*K + j at sorted position i;
    pair_pos[a] = its sorted position."""
    flat = np.asarray(topk_ids, dtype=np.int64).reshape(-1)
    sorted_pairs = np.argsort(flat, kind="stable")
    pair_pos = np.empty_like(sorted_pairs)
    pair_pos[sorted_pairs] = np.arange(flat.size)
    counts = np.bincount(flat, minlength=num_experts)
    offsets = np.zeros(num_experts + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(counts)
    return sorted_pairs.astype(np.int32), pair_pos.astype(np.int32), offsets.astype(np.int32)


def permute_rows(x: np.ndarray, sorted_pairs: np.ndarray, k: int) -> np.ndarray:
    """x [T, Hd] -> x_sorted [T*K, Hd]: row i = x[sorted_pairs[i] // k] (a copy, any dtype)."""
    return np.asarray(x)[np.asarray(sorted_pairs, dtype=np.int64) // k]


def combine(y_sorted: np.ndarray, weights: np.ndarray, pair_pos: np.ndarray) -> np.ndarray:
    """y_sorted float64 [T*K, Hd], weights [T, K] -> out float64 [T, Hd]."""
    w = np.asarray(weights, dtype=np.float64)
    T, K = w.shape
    pos = np.asarray(pair_pos, dtype=np.int64).reshape(T, K)
    out = np.zeros((T, y_sorted.shape[1]), dtype=np.float64)
    for j in range(K):
        out += w[:, j:j + 1] * y_sorted[pos[:, j]]
    return out
