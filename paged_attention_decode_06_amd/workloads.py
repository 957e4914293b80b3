"""Seeded synthetic inputs for paged-attention decode.

This module only *draws* inputs: sequence lengths, block tables, queries and
the paged K/V pools. It holds none of the attention arithmetic, so both the
fp64 oracle (via the tests) and the HIP path can be fed from it without
sharing any of the method's code.

Workload shapes follow the pages' serving context: head_dim 128 (and 256),
grouped-query attention, bf16/fp16 caches (project_6 blame view of
optimizations/prefix_prefill_patch.py, "Qwen3.6-35B-A3B attention" part of
the docstring); contexts up to 100K tokens (same docstring, yaml analysis;
project_6 commit cd0d9e1a, V2 implementation); up to 256 concurrent
sequences (project_6 commit 490ff98a, computility-run.yaml change).

Recipe (every config):
  * one NumPy PCG64 stream per (config seed, purpose, chunk): purpose ids are
    0 = lengths and tables, 1 = q, 2 = K, 3 = V, 4 = the K outlier mask;
    chunks hold 2**24 elements, so generation is reproducible and threaded.
  * values are N(0, 1) drawn in fp32, then rounded to the cache dtype
    (round-to-nearest-even for bf16); q and out share the cache dtype.
  * the K/V pools are [num_blocks, num_kv_heads, 16, head_dim], row-major;
    the pool holds exactly sum(ceil(L/16)) blocks (64 for the tiny config),
    handed out to the sequences in the order of one random permutation.
  * table entries past ceil(L/16) are 0 (or the poison block, see `poison`).
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np

BLOCK_SIZE = 16
CHUNK = 1 << 24

_PURPOSE_TABLE, _PURPOSE_Q, _PURPOSE_K, _PURPOSE_V, _PURPOSE_KMASK = 0, 1, 2, 3, 4


@dataclass(frozen=True)
class DecodeConfig:
    """One decode workload. `lengths` names the seq_len distribution."""
    name: str
    num_seqs: int
    num_heads: int
    num_kv_heads: int
    head_dim: int
    dtype: str                 # "f32", "bf16" or "f16"
    lengths: tuple             # ("fixed", L) | ("uniform", lo, hi) | ("loguniform", lo, hi)
    pool_blocks: int | None = None   # fixed pool size (tiny config); None = exactly what is used
    k_outlier_frac: float = 0.0      # fraction of K scalars multiplied by k_outlier_mult
    k_outlier_mult: float = 1.0
    scale: float | None = None       # None = 1/sqrt(head_dim)

    @property
    def softmax_scale(self) -> float:
        return self.scale if self.scale is not None else 1.0 / math.sqrt(self.head_dim)


# The five decode workloads (seed = 1000 + number).
DECODE_WORKLOADS = {
    1: DecodeConfig("tiny-L37-fp32", 1, 2, 1, 128, "f32", ("fixed", 37), pool_blocks=64),
    2: DecodeConfig("batch8-U1-8192-bf16", 8, 16, 2, 128, "bf16", ("uniform", 1, 8192)),
    3: DecodeConfig("ctx100K-bf16", 1, 16, 2, 128, "bf16", ("fixed", 100000)),
    4: DecodeConfig("batch64-logU512-65536-bf16", 64, 16, 2, 128, "bf16", ("loguniform", 512, 65536)),
    5: DecodeConfig("batch256-U1024-32768-d256-bf16", 256, 16, 2, 256, "bf16", ("uniform", 1024, 32768),
                    k_outlier_frac=0.01, k_outlier_mult=20.0),
    # fp16-cache variant of the 100K-token decode (the model's other 16-bit type)
    6: DecodeConfig("ctx100K-f16", 1, 16, 2, 128, "f16", ("fixed", 100000)),
}


@dataclass
class DecodeInputs:
    """Host-side inputs. bf16 arrays are stored as uint16 bit patterns, f16 as float16."""
    cfg: DecodeConfig
    seed: int
    seq_lens: np.ndarray        # int32 [S]
    block_tables: np.ndarray    # int32 [S, max_blocks_per_seq]
    q: np.ndarray               # [S, H, D]  float32 or uint16(bf16 bits)
    k_cache: np.ndarray         # [NB, Hkv, 16, D]
    v_cache: np.ndarray         # [NB, Hkv, 16, D]
    scale: float
    extra: dict = field(default_factory=dict)

    @property
    def num_blocks(self) -> int:
        return int(self.k_cache.shape[0])

    @property
    def max_blocks_per_seq(self) -> int:
        return int(self.block_tables.shape[1])


def _rng(seed: int, purpose: int, chunk: int = 0) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed, spawn_key=(purpose, chunk))))


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16 (nearest, ties to even); NaN stays a quiet NaN."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    rounded = ((u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)).astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        rounded[nan] = np.uint16(0x7FC0)
    return rounded


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to fp32 (input plumbing only)."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _workers() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _fill_normal(out_flat: np.ndarray, seed: int, purpose: int, dtype: str,
                 outlier_frac: float = 0.0, outlier_mult: float = 1.0) -> None:
    """Fill `out_flat` (float32 or uint16 bf16 bits) with seeded N(0,1) draws, chunk by chunk."""
    n = out_flat.size
    nchunks = (n + CHUNK - 1) // CHUNK

    def work(c: int) -> None:
        lo, hi = c * CHUNK, min(n, (c + 1) * CHUNK)
        vals = _rng(seed, purpose, c).standard_normal(hi - lo, dtype=np.float32)
        if outlier_frac > 0.0:
            mask = _rng(seed, _PURPOSE_KMASK, c).random(hi - lo, dtype=np.float32) < outlier_frac
            vals[mask] *= np.float32(outlier_mult)
        if dtype == "f32":
            out_flat[lo:hi] = vals
        elif dtype == "f16":
            out_flat[lo:hi] = vals.astype(np.float16)   # round to nearest even
        else:
            out_flat[lo:hi] = f32_to_bf16_bits(vals)

    if nchunks == 1:
        work(0)
    else:
        with ThreadPoolExecutor(_workers()) as ex:
            list(ex.map(work, range(nchunks)))


def draw_seq_lens(cfg: DecodeConfig, rng: np.random.Generator) -> np.ndarray:
    kind = cfg.lengths[0]
    S = cfg.num_seqs
    if kind == "fixed":
        lens = np.full(S, cfg.lengths[1], dtype=np.int64)
    elif kind == "uniform":
        lo, hi = cfg.lengths[1], cfg.lengths[2]
        lens = rng.integers(lo, hi + 1, size=S)
    elif kind == "loguniform":
        lo, hi = cfg.lengths[1], cfg.lengths[2]
        lens = np.rint(np.exp(rng.uniform(math.log(lo), math.log(hi), size=S))).astype(np.int64)
        lens = np.clip(lens, lo, hi)
    else:
        raise ValueError(f"unknown length distribution {kind!r}")
    return lens.astype(np.int32)


def build_tables(seq_lens: np.ndarray, rng: np.random.Generator, pool_blocks: int | None,
                 max_blocks_per_seq: int | None = None):
    """Shuffled block tables; returns (tables int32 [S, MB], num_blocks)."""
    need = [(int(L) + BLOCK_SIZE - 1) // BLOCK_SIZE for L in seq_lens]
    total = sum(need)
    mb = max(1, max(need) if need else 1)
    if max_blocks_per_seq is not None:
        if max_blocks_per_seq < mb:
            raise ValueError("max_blocks_per_seq too small for the drawn lengths")
        mb = max_blocks_per_seq
    if pool_blocks is None:
        nb = max(total, 1)
        ids = rng.permutation(nb)
    else:
        if pool_blocks < total:
            raise ValueError("pool too small")
        nb = pool_blocks
        ids = rng.choice(pool_blocks, total, replace=False)
    tables = np.zeros((len(seq_lens), mb), dtype=np.int32)
    pos = 0
    for s, n in enumerate(need):
        tables[s, :n] = ids[pos:pos + n]
        pos += n
    return tables, nb


def make_inputs(cfg: DecodeConfig | int, seed: int | None = None, *, seq_lens=None,
                max_blocks_per_seq: int | None = None, pool_blocks: int | None = None,
                poison: bool = False) -> DecodeInputs:
    """Draw one workload.

    cfg            a DecodeConfig or a config number (1..5)
    seed           defaults to 1000 + config number (or 1000 for ad-hoc configs)
    seq_lens       override the drawn lengths (edge-case tests)
    poison         add one extra pool block full of NaN that every padding table
                   entry points at, and set every slot the context does not cover
                   (tail slots of last blocks, unreferenced blocks) to NaN/Inf
    """
    number = None
    if isinstance(cfg, int):
        number = cfg
        cfg = DECODE_WORKLOADS[cfg]
    if seed is None:
        seed = 1000 + (number if number is not None else 0)
    trng = _rng(seed, _PURPOSE_TABLE)
    if seq_lens is None:
        lens = draw_seq_lens(cfg, trng)
    else:
        lens = np.asarray(seq_lens, dtype=np.int32).reshape(-1)
        cfg = DecodeConfig(cfg.name + "-custom", int(lens.size), cfg.num_heads, cfg.num_kv_heads,
                           cfg.head_dim, cfg.dtype, ("custom",), cfg.pool_blocks,
                           cfg.k_outlier_frac, cfg.k_outlier_mult, cfg.scale)
    pb = pool_blocks if pool_blocks is not None else cfg.pool_blocks
    tables, nb = build_tables(lens, trng, pb, max_blocks_per_seq)
    S, H, Hkv, D = cfg.num_seqs, cfg.num_heads, cfg.num_kv_heads, cfg.head_dim
    store = {"f32": np.float32, "f16": np.float16, "bf16": np.uint16}[cfg.dtype]
    nb_alloc = nb + (1 if poison else 0)

    q = np.empty((S, H, D), dtype=store)
    _fill_normal(q.reshape(-1), seed, _PURPOSE_Q, cfg.dtype)
    k = np.empty((nb_alloc, Hkv, BLOCK_SIZE, D), dtype=store)
    v = np.empty((nb_alloc, Hkv, BLOCK_SIZE, D), dtype=store)
    _fill_normal(k[:nb].reshape(-1), seed, _PURPOSE_K, cfg.dtype, cfg.k_outlier_frac, cfg.k_outlier_mult)
    _fill_normal(v[:nb].reshape(-1), seed, _PURPOSE_V, cfg.dtype)

    extra = {}
    if poison:
        _poison(lens, tables, k, v, nb, cfg.dtype)
        extra["poison_block"] = nb
    return DecodeInputs(cfg, seed, lens, tables, q, k, v, cfg.softmax_scale, extra)


def _poison(lens, tables, k, v, poison_block, dtype) -> None:
    """Fill every slot no context reaches with NaN (V) and +Inf/NaN (K)."""
    if dtype == "f32":
        nan, inf = np.float32(np.nan), np.float32(np.inf)
    elif dtype == "f16":
        nan, inf = np.float16(np.nan), np.float16(np.inf)
    else:
        nan, inf = np.uint16(0x7FC0), np.uint16(0x7F80)
    used = np.zeros(k.shape[0], dtype=bool)
    for s, L in enumerate(lens):
        nblk = (int(L) + BLOCK_SIZE - 1) // BLOCK_SIZE
        used[tables[s, :nblk]] = True
        tables[s, nblk:] = poison_block
        if nblk and L % BLOCK_SIZE:
            last = tables[s, nblk - 1]
            k[last, :, L % BLOCK_SIZE:, :] = inf
            v[last, :, L % BLOCK_SIZE:, :] = nan
    unused = ~used
    k[unused] = nan
    v[unused] = nan


# ---------------------------------------------------------------- prefix / chunked prefill
@dataclass(frozen=True)
class PrefillConfig:
    """One prefix/chunked-prefill workload over the paged cache.

    Sequence s holds C_s cached prefix tokens followed by Q_s chunk tokens
    (seq_len L_s = C_s + Q_s, all of it in the cache); the chunk's Q_s query
    tokens are packed by token into q [sum Q_s, H, D]. `context` and `chunk`
    name the distributions of C_s and Q_s like DecodeConfig.lengths."""
    name: str
    num_seqs: int
    num_heads: int
    num_kv_heads: int
    head_dim: int
    dtype: str
    context: tuple
    chunk: tuple
    scale: float | None = None

    @property
    def softmax_scale(self) -> float:
        return self.scale if self.scale is not None else 1.0 / math.sqrt(self.head_dim)


# Prefill workloads (seed = 2000 + number): the last 2048-token chunk of a
# 100K-token prompt with its prefix cached; a batch of fresh 1024-token
# prompts (16K batched tokens); a mixed batch of cached prefixes and chunks;
# the same mix at head_dim 256. Chunked prefill with 8K-32K batched tokens and
# 100K contexts is the serving setting the pages describe (prefix_prefill_patch.py
# docstring, yaml analysis; commit 490ff98a, computility-run.yaml change).
PREFILL_WORKLOADS = {
    1: PrefillConfig("chunk2048-ctx100K-bf16", 1, 16, 2, 128, "bf16", ("fixed", 100000 - 2048), ("fixed", 2048)),
    2: PrefillConfig("batch16-prompt1024-bf16", 16, 16, 2, 128, "bf16", ("fixed", 0), ("fixed", 1024)),
    3: PrefillConfig("batch8-ctxU0-32768-chunkU1-2048-bf16", 8, 16, 2, 128, "bf16",
                     ("uniform", 0, 32768), ("uniform", 1, 2048)),
    4: PrefillConfig("batch4-ctxU0-8192-chunk512-d256-bf16", 4, 16, 2, 256, "bf16",
                     ("uniform", 0, 8192), ("fixed", 512)),
}


@dataclass
class PrefillInputs:
    cfg: PrefillConfig
    seed: int
    seq_lens: np.ndarray         # int32 [S]: C_s + Q_s tokens in the cache
    query_lens: np.ndarray       # int32 [S]: Q_s
    query_start_loc: np.ndarray  # int32 [S + 1]: exclusive prefix sum of query_lens
    block_tables: np.ndarray     # int32 [S, max_blocks_per_seq]
    q: np.ndarray                # [sum Q_s, H, D]
    k_cache: np.ndarray
    v_cache: np.ndarray
    scale: float
    extra: dict = field(default_factory=dict)

    @property
    def num_blocks(self) -> int:
        return int(self.k_cache.shape[0])

    @property
    def max_blocks_per_seq(self) -> int:
        return int(self.block_tables.shape[1])

    @property
    def num_query_tokens(self) -> int:
        return int(self.query_start_loc[-1])

    @property
    def max_query_len(self) -> int:
        return int(self.query_lens.max(initial=0))


def _draw(dist: tuple, n: int, rng: np.random.Generator) -> np.ndarray:
    kind = dist[0]
    if kind == "fixed":
        return np.full(n, dist[1], dtype=np.int64)
    if kind == "uniform":
        return rng.integers(dist[1], dist[2] + 1, size=n)
    raise ValueError(f"unknown length distribution {kind!r}")


def make_prefill_inputs(cfg: PrefillConfig | int, seed: int | None = None, *, context_lens=None,
                        query_lens=None, max_blocks_per_seq: int | None = None,
                        poison: bool = False) -> PrefillInputs:
    """Draw one prefill workload (same pool, table and value recipe as decode;
    the prefix lengths are drawn first, then the chunk lengths)."""
    number = None
    if isinstance(cfg, int):
        number = cfg
        cfg = PREFILL_WORKLOADS[cfg]
    if seed is None:
        seed = 2000 + (number if number is not None else 0)
    trng = _rng(seed, _PURPOSE_TABLE)
    if context_lens is None or query_lens is None:
        ctx = _draw(cfg.context, cfg.num_seqs, trng)
        ql = _draw(cfg.chunk, cfg.num_seqs, trng)
    if context_lens is not None:
        ctx = np.asarray(context_lens, dtype=np.int64).reshape(-1)
    if query_lens is not None:
        ql = np.asarray(query_lens, dtype=np.int64).reshape(-1)
    if ctx.size != ql.size:
        raise ValueError("context_lens and query_lens differ in length")
    if ctx.size != cfg.num_seqs:
        cfg = PrefillConfig(cfg.name + "-custom", int(ctx.size), cfg.num_heads, cfg.num_kv_heads,
                            cfg.head_dim, cfg.dtype, ("custom",), ("custom",), cfg.scale)
    lens = (ctx + ql).astype(np.int32)
    ql = ql.astype(np.int32)
    tables, nb = build_tables(lens, trng, None, max_blocks_per_seq)
    S, H, Hkv, D = cfg.num_seqs, cfg.num_heads, cfg.num_kv_heads, cfg.head_dim
    store = {"f32": np.float32, "f16": np.float16, "bf16": np.uint16}[cfg.dtype]
    nb_alloc = nb + (1 if poison else 0)
    qsl = np.zeros(S + 1, dtype=np.int32)
    qsl[1:] = np.cumsum(ql)
    q = np.empty((int(qsl[-1]), H, D), dtype=store)
    _fill_normal(q.reshape(-1), seed, _PURPOSE_Q, cfg.dtype)
    k = np.empty((nb_alloc, Hkv, BLOCK_SIZE, D), dtype=store)
    v = np.empty((nb_alloc, Hkv, BLOCK_SIZE, D), dtype=store)
    _fill_normal(k[:nb].reshape(-1), seed, _PURPOSE_K, cfg.dtype)
    _fill_normal(v[:nb].reshape(-1), seed, _PURPOSE_V, cfg.dtype)
    extra = {}
    if poison:
        _poison(lens, tables, k, v, nb, cfg.dtype)
        extra["poison_block"] = nb
    return PrefillInputs(cfg, seed, lens, ql, qsl, tables, q, k, v, cfg.softmax_scale, extra)


def prefill_flops(seq_lens, query_lens, num_heads: int, head_dim: int) -> int:
    """Multiply-adds x 2 the chunk tokens' attention must do: every query row
    (token, head) against every key it may see (pos + 1 of them), for Q.K^T and
    for P.V: 4 * D flops per (row, key)."""
    tot = 0
    for L, Q in zip(np.asarray(seq_lens, dtype=np.int64), np.asarray(query_lens, dtype=np.int64)):
        Q = int(min(Q, L))
        first = int(L) - Q + 1                      # keys seen by the chunk's first token
        tot += (first + int(L)) * Q // 2 if Q else 0  # sum of first .. L
    return 4 * head_dim * num_heads * tot


def prefill_to_device(x: PrefillInputs, device="cuda"):
    d = to_device(x, device)
    import torch
    d["query_start_loc"] = torch.from_numpy(x.query_start_loc).to(device)
    return d


# ---------------------------------------------------------------- MoE routing
@dataclass(frozen=True)
class MoeConfig:
    """One MoE routing workload: T tokens, E experts, top k, hidden size."""
    name: str
    num_tokens: int
    num_experts: int
    top_k: int
    hidden: int
    dtype: str = "bf16"          # hidden rows and expert outputs
    renormalize: bool = True


# 256 experts with top 8 (the pages' MoE rewrite); 16384 tokens is the
# prefill batch the same passage sizes; 256 tokens a decode step at 256
# concurrent sequences. Hidden size 2048 is a stand-in (the pages give none).
MOE_WORKLOADS = {
    1: MoeConfig("prefill-T16384-E256-k8-H2048-bf16", 16384, 256, 8, 2048),
    2: MoeConfig("decode-T256-E256-k8-H2048-bf16", 256, 256, 8, 2048),
}


@dataclass
class MoeInputs:
    cfg: MoeConfig
    seed: int
    logits: np.ndarray      # float32 [T, E] router logits
    x: np.ndarray           # [T, Hd] hidden rows (uint16 bf16 bits / float16 / float32)
    y_sorted: np.ndarray    # [T*K, Hd] stand-in expert outputs, in sorted-pair order


def make_moe_inputs(cfg: MoeConfig | int, seed: int | None = None, *, num_tokens: int | None = None) -> MoeInputs:
    """Router logits N(0, 1) in fp32, hidden rows and stand-in expert outputs
    N(0, 1) rounded to the dtype (purposes 1, 2, 3 of the seed)."""
    number = None
    if isinstance(cfg, int):
        number = cfg
        cfg = MOE_WORKLOADS[cfg]
    if num_tokens is not None:
        cfg = MoeConfig(cfg.name + "-custom", int(num_tokens), cfg.num_experts, cfg.top_k, cfg.hidden,
                        cfg.dtype, cfg.renormalize)
    if seed is None:
        seed = 3000 + (number if number is not None else 0)
    T, E, K, Hd = cfg.num_tokens, cfg.num_experts, cfg.top_k, cfg.hidden
    store = {"f32": np.float32, "f16": np.float16, "bf16": np.uint16}[cfg.dtype]
    logits = np.empty((T, E), dtype=np.float32)
    _fill_normal(logits.reshape(-1), seed, 1, "f32")
    x = np.empty((T, Hd), dtype=store)
    _fill_normal(x.reshape(-1), seed, 2, cfg.dtype)
    y = np.empty((T * K, Hd), dtype=store)
    _fill_normal(y.reshape(-1), seed, 3, cfg.dtype)
    return MoeInputs(cfg, seed, logits, x, y)


def moe_bytes(cfg: MoeConfig) -> dict:
    """Algorithmic bytes of each routing step (elem = bytes per hidden value)."""
    T, E, K, Hd = cfg.num_tokens, cfg.num_experts, cfg.top_k, cfg.hidden
    e = {"f32": 4, "f16": 2, "bf16": 2}[cfg.dtype]
    N = T * K
    return {
        "topk_softmax": T * E * 4 + N * 8,               # logits in; weights + ids out
        "sort_by_expert": N * 4 + N * 8 + (E + 1) * 4,   # ids in; sorted pairs, positions, offsets out
        "permute": N * 4 + T * Hd * e + N * Hd * e,      # pair list; each token row read once, N rows written
        "combine": N * (4 + 4) + N * Hd * e + T * Hd * e,  # positions, weights; expert rows in; out rows
    }


def algorithmic_bytes(seq_lens, num_heads: int, num_kv_heads: int, head_dim: int, elem_bytes: int) -> int:
    """Bytes the decode step must move at minimum.

    K and V: 2 * head_dim * elem_bytes per context token per KV head (the
    pages' per-token KV arithmetic, yaml analysis of the prefix_prefill_patch.py
    docstring); plus q and out (S*H*D each), the table entries used and the
    seq_lens. V2 partials are implementation overhead and are not counted.
    """
    lens = np.asarray(seq_lens, dtype=np.int64)
    S = lens.size
    kv = int(lens.sum()) * num_kv_heads * 2 * head_dim * elem_bytes
    qo = 2 * S * num_heads * head_dim * elem_bytes
    table = 4 * int(((lens + BLOCK_SIZE - 1) // BLOCK_SIZE).sum())
    return kv + qo + table + 4 * S


def to_device(x: DecodeInputs, device="cuda"):
    """Copy a workload to torch tensors on `device` (bf16 bit patterns become torch.bfloat16)."""
    import torch

    def conv(a):
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).to(device).view(torch.bfloat16)
        return torch.from_numpy(np.ascontiguousarray(a)).to(device)

    return {
        "q": conv(x.q),
        "k_cache": conv(x.k_cache),
        "v_cache": conv(x.v_cache),
        "block_tables": torch.from_numpy(x.block_tables).to(device),
        "seq_lens": torch.from_numpy(x.seq_lens).to(device),
    }


def from_device(t) -> np.ndarray:
    """Host float64 copy of a float32 or bfloat16 tensor."""
    import torch
    if t.dtype == torch.bfloat16:
        return bf16_bits_to_f32(t.view(torch.int16).cpu().numpy().view(np.uint16)).astype(np.float64)
    return t.float().cpu().numpy().astype(np.float64)
