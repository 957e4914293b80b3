"""GPU parity of the prefix/chunked-prefill kernel (through the C ABI) against
the fp64 oracle (oracle.prefill).

Tolerances (max |error| over every compared element): 2e-2 for bf16 caches,
1e-2 for fp16, with fp32 accumulation inside the kernel.
"""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
import paged_attention_decode_06_amd as pa
from paged_attention_decode_06_amd import workloads as W

pytestmark = pytest.mark.gpu

TOL = {"bf16": 2e-2, "f16": 1e-2}


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    pa.load()
    return torch.device("cuda:0")


def say(*a):
    print(*a, flush=True)


def run(x, dev, d=None, max_query_len=None):
    d = d or W.prefill_to_device(x, dev)
    out = torch.full_like(d["q"], float("nan"))
    mq = x.max_query_len if max_query_len is None else max_query_len
    pa.pa_prefill(out, d["q"], d["k_cache"], d["v_cache"], d["block_tables"], d["seq_lens"],
                  d["query_start_loc"], x.scale, mq)
    torch.cuda.synchronize(dev)
    return out


def max_err(got, ref):
    e = np.abs(got - ref)
    return float("inf") if np.isnan(e).any() else float(e.max(initial=0.0))


def check_all(x, out, label=""):
    ref = oracle.attend_prefill(x.q, x.k_cache, x.v_cache, x.block_tables, x.seq_lens, x.query_start_loc,
                                x.scale, x.cfg.dtype)
    got = W.from_device(out)
    err = max_err(got, ref)
    say(f"  {label}: max|err| = {err:.3e} over {got.shape[0]} tokens (tol {TOL[x.cfg.dtype]})")
    assert err <= TOL[x.cfg.dtype], label
    return got


def check_rows(x, out, rows, label=""):
    """Sampled chunk tokens of a workload too large for the whole oracle."""
    got = W.from_device(out)
    lists = oracle.gather_list(x.block_tables, x.seq_lens)
    qsl = x.query_start_loc
    worst = 0.0
    for r in rows:
        s = int(np.searchsorted(qsl, r, side="right") - 1)
        i = r - int(qsl[s])
        pos = int(x.seq_lens[s]) - int(x.query_lens[s]) + i
        ref = oracle.attend_prefill_row(x.q[r], x.k_cache, x.v_cache, lists[s], pos, x.scale, x.cfg.dtype)
        worst = max(worst, max_err(got[r], ref))
    say(f"  {label}: max|err| = {worst:.3e} over {len(rows)} sampled tokens")
    assert worst <= TOL[x.cfg.dtype], label
    assert np.isfinite(got).all()


def sample_rows(x, n, rng):
    """First and last token of every sequence's chunk, plus random others."""
    qsl = x.query_start_loc
    pick = set()
    for s in range(x.cfg.num_seqs):
        if qsl[s + 1] > qsl[s]:
            pick.update([int(qsl[s]), int(qsl[s + 1]) - 1])
    T = x.num_query_tokens
    pick.update(int(r) for r in rng.choice(T, size=min(n, T), replace=False))
    return sorted(pick)


# ---------------------------------------------------------------- the prefill workloads
@pytest.mark.parametrize("num", [1, 2, 3, 4])
def test_prefill_workload_parity(dev, num):
    x = W.make_prefill_inputs(num)
    say(f"prefill workload {num} {x.cfg.name}: tokens={x.num_query_tokens} L={x.seq_lens.tolist()[:8]}")
    out = run(x, dev)
    if num in (2, 4):
        # every chunk token: the whole-batch oracle fits in memory and seconds
        ref = oracle.attend_prefill(x.q, x.k_cache, x.v_cache, x.block_tables, x.seq_lens, x.query_start_loc,
                                    x.scale, x.cfg.dtype)
        got = W.from_device(out)
        worst = max_err(got, ref)
        say(f"  {x.cfg.name}: max|err| = {worst:.3e} over all {x.num_query_tokens} tokens")
        assert worst <= TOL[x.cfg.dtype]
        assert np.isfinite(got).all()
        return
    # workloads 1 and 3: a chunk of 2048 over 100K tokens, and eight chunks over
    # up to 32K: the whole-batch fp64 score matrices would not fit, so sampled
    # rows (the first and last of every chunk and random others)
    n = {1: 10, 3: 24}[num]
    check_rows(x, out, sample_rows(x, n, np.random.default_rng(num)), x.cfg.name)


# ---------------------------------------------------------------- shapes and edges
SMALL = [
    ([0, 37, 600], [50, 1, 130]),     # no prefix, a single token, prefix + chunk
    ([1000], [200]),                  # chunk of 200 over a 1000-token prefix
    ([5, 0], [16, 129]),              # chunk lengths around the 16-token query tile
    ([15, 16, 17], [1, 17, 33]),      # block edges
]


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("D", [128, 256])
@pytest.mark.parametrize("case", range(len(SMALL)))
def test_prefill_small_cases(dev, case, D, dtype):
    ctx, ql = SMALL[case]
    cfg = W.PrefillConfig(f"small-{dtype}-d{D}", len(ctx), 16, 2, D, dtype, ("custom",), ("custom",))
    x = W.make_prefill_inputs(cfg, seed=40 + case, context_lens=ctx, query_lens=ql)
    say(f"prefill small case {case}: ctx={ctx} chunk={ql} D={D} {dtype}")
    check_all(x, run(x, dev), f"case {case}")


@pytest.mark.parametrize("H,Hkv", [(8, 8), (16, 8), (32, 2), (12, 4), (10, 2), (4, 1)])
def test_prefill_group_sizes(dev, H, Hkv):
    cfg = W.PrefillConfig("groups", 2, H, Hkv, 128, "bf16", ("custom",), ("custom",))
    x = W.make_prefill_inputs(cfg, seed=50, context_lens=[300, 0], query_lens=[77, 150])
    say(f"prefill group size G={H // Hkv}")
    check_all(x, run(x, dev), f"G={H // Hkv}")


def test_prefill_poisoned_pool(dev):
    cfg = W.PrefillConfig("poison", 3, 16, 2, 128, "bf16", ("custom",), ("custom",))
    x = W.make_prefill_inputs(cfg, seed=51, context_lens=[20, 0, 513], query_lens=[9, 31, 40],
                              max_blocks_per_seq=80, poison=True)
    say("prefill with NaN/Inf outside every context")
    got = check_all(x, run(x, dev), "poison")
    assert np.isfinite(got).all()


def test_prefill_chunk_longer_than_context_gives_zeros(dev):
    cfg = W.PrefillConfig("neg", 1, 16, 2, 128, "bf16", ("custom",), ("custom",))
    x = W.make_prefill_inputs(cfg, seed=52, context_lens=[0], query_lens=[40])
    # claim 45 query tokens for a 40-token sequence: the first 5 sit at negative positions
    extra = W.make_prefill_inputs(cfg, seed=53, context_lens=[0], query_lens=[5]).q
    x.q = np.concatenate([extra, x.q])
    x.query_lens = np.array([45], dtype=np.int32)
    x.query_start_loc = np.array([0, 45], dtype=np.int32)
    say("prefill chunk longer than its sequence")
    got = check_all(x, run(x, dev), "negative positions")
    assert (got[:5] == 0).all()


def test_single_token_chunks_match_decode(dev):
    cfg = W.PrefillConfig("q1", 4, 16, 2, 128, "bf16", ("custom",), ("custom",))
    x = W.make_prefill_inputs(cfg, seed=54, context_lens=[0, 36, 5000, 9000], query_lens=[1, 1, 1, 1])
    d = W.prefill_to_device(x, dev)
    say("single-token chunks vs pa_decode")
    pre = W.from_device(run(x, dev, d))
    out = torch.empty_like(d["q"])
    sh = pa.make_shape(d["q"], d["k_cache"], d["block_tables"])
    es, ml, to = pa.alloc_partials(sh, dev)
    pa.pa_decode(out, d["q"], d["k_cache"], d["v_cache"], d["block_tables"], d["seq_lens"], x.scale, es, ml, to)
    torch.cuda.synchronize(dev)
    assert max_err(pre, W.from_device(out)) <= 2 * TOL["bf16"]
    check_all(x, torch.from_numpy(pre).to(dev), "q=1")


def test_prefill_empty_inputs(dev):
    cfg = W.PrefillConfig("empty", 2, 16, 2, 128, "bf16", ("custom",), ("custom",))
    x = W.make_prefill_inputs(cfg, seed=55, context_lens=[10, 20], query_lens=[0, 0])
    d = W.prefill_to_device(x, dev)
    out = torch.empty((0, 16, 128), dtype=torch.bfloat16, device=dev)
    say("prefill with no query tokens")
    pa.pa_prefill(out, out, d["k_cache"], d["v_cache"], d["block_tables"], d["seq_lens"],
                  d["query_start_loc"], x.scale, 0)
    torch.cuda.synchronize(dev)


def test_prefill_block_permutation_bitwise_and_deterministic(dev):
    x = W.make_prefill_inputs(W.PREFILL_WORKLOADS[2], seed=56, context_lens=[700, 40], query_lens=[300, 90])
    say("prefill block permutation / determinism")
    a = W.from_device(run(x, dev))
    b = W.from_device(run(x, dev))
    assert np.array_equal(a, b)
    perm = np.random.default_rng(0).permutation(x.num_blocks)
    k2 = np.empty_like(x.k_cache); v2 = np.empty_like(x.v_cache)
    k2[perm] = x.k_cache; v2[perm] = x.v_cache
    x.k_cache, x.v_cache = k2, v2
    x.block_tables = perm[x.block_tables].astype(np.int32)
    c = W.from_device(run(x, dev))
    assert np.array_equal(a, c)


def test_prefill_rejects_f32(dev):
    cfg = W.PrefillConfig("f32", 1, 2, 1, 128, "f32", ("custom",), ("custom",))
    x = W.make_prefill_inputs(cfg, seed=57, context_lens=[3], query_lens=[2])
    with pytest.raises(pa.PaError):
        run(x, dev)


# Table widths for the many-workgroup tests: the natural one (at most 8192
# tokens: the 4-wave short-table shape) and 600 blocks (9600 tokens: the
# 8-wave shape).
WIDE = [None, 600]


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("mb", WIDE)
def test_prefill_large_grid_every_token(dev, mb, dtype):
    """More than 512 workgroups (the many-workgroup launch shapes), every token
    compared, with bf16 and with fp16 caches."""
    rng = np.random.default_rng(58)
    S = 40
    ctx = rng.integers(0, 300, size=S)
    ql = rng.integers(100, 129, size=S)
    cfg = dataclasses.replace(W.PREFILL_WORKLOADS[2], dtype=dtype)
    x = W.make_prefill_inputs(cfg, seed=58, context_lens=ctx, query_lens=ql, max_blocks_per_seq=mb)
    say(f"prefill large grid, {dtype}: {S} seqs, {x.num_query_tokens} tokens, table width {x.max_blocks_per_seq}")
    check_all(x, run(x, dev), f"large grid {dtype}")


@pytest.mark.parametrize("mb", WIDE)
def test_prefill_large_grid_odd_group(dev, mb):
    """The many-workgroup shapes with G = 3 (42 tokens x 3 heads = 126 of 128
    rows, or 85 x 3 = 255 of 256), every token."""
    rng = np.random.default_rng(59)
    S = 40
    cfg = W.PrefillConfig("g3", S, 12, 4, 128, "bf16", ("custom",), ("custom",))
    x = W.make_prefill_inputs(cfg, seed=59, context_lens=rng.integers(0, 200, size=S),
                              query_lens=rng.integers(150, 201, size=S), max_blocks_per_seq=mb)
    say(f"prefill large grid, G=3: {x.num_query_tokens} tokens")
    check_all(x, run(x, dev), "large grid G=3")


@pytest.mark.parametrize("mult", [-1.0, 0.0, 4.0])
@pytest.mark.parametrize("D", [128, 256])
def test_prefill_scale_sign_and_zero(dev, D, mult):
    """A negative scale (folded into q as a sign flip), a zero scale (every
    visible key weighs the same) and a large one, on both launch forms."""
    cfg = W.PrefillConfig(f"scale-d{D}", 2, 16, 2, D, "bf16", ("custom",), ("custom",))
    x = W.make_prefill_inputs(cfg, seed=61, context_lens=[400, 33], query_lens=[90, 70])
    x = dataclasses.replace(x, scale=x.scale * mult)
    say(f"prefill scale x{mult} D={D}")
    check_all(x, run(x, dev), f"scale x{mult} D={D}")


@pytest.mark.parametrize("mb", WIDE)
def test_prefill_large_grid_negative_scale(dev, mb):
    """The many-workgroup shapes with a negative scale, every token."""
    rng = np.random.default_rng(62)
    S = 40
    x = W.make_prefill_inputs(W.PREFILL_WORKLOADS[2], seed=62, context_lens=rng.integers(0, 300, size=S),
                              query_lens=rng.integers(100, 129, size=S), max_blocks_per_seq=mb)
    x = dataclasses.replace(x, scale=-x.scale)
    say(f"prefill large grid, negative scale: {x.num_query_tokens} tokens")
    check_all(x, run(x, dev), "large grid, scale < 0")


@pytest.mark.parametrize("mb", WIDE)
@pytest.mark.parametrize("S", [80, 300])
def test_prefill_many_sequences(dev, mb, S):
    """80 sequences (ranked launch order, two sequences per lane of the rank
    search) and 300 (more than 256: the order by query-tile rounds), every token."""
    rng = np.random.default_rng(63)
    x = W.make_prefill_inputs(W.PREFILL_WORKLOADS[2], seed=63, context_lens=rng.integers(0, 400, size=S),
                              query_lens=rng.integers(1, 60, size=S), max_blocks_per_seq=mb)
    say(f"prefill {S} sequences: {x.num_query_tokens} tokens")
    check_all(x, run(x, dev), f"{S} sequences")


@pytest.mark.parametrize("S", [5, 70, 260])
def test_prefill_tokens_past_max_query_len_not_computed(dev, S):
    """max_query_len = 64 below the longest chunk: chunk tokens 0..63 of every
    sequence are right, the later ones keep what the output held (64 is a whole
    number of query tiles in every launch shape at G = 8). Both launch orders
    (by cost up to 256 sequences, by rounds above)."""
    rng = np.random.default_rng(64 + S)
    ql = rng.integers(1, 200, size=S)
    ql[0] = 199
    x = W.make_prefill_inputs(W.PREFILL_WORKLOADS[2], seed=64 + S, context_lens=rng.integers(0, 600, size=S),
                              query_lens=ql)
    out = W.from_device(run(x, dev, max_query_len=64))
    ref = oracle.attend_prefill(x.q, x.k_cache, x.v_cache, x.block_tables, x.seq_lens, x.query_start_loc,
                                x.scale, x.cfg.dtype)
    qsl = x.query_start_loc
    inside = np.zeros(x.num_query_tokens, dtype=bool)
    for s in range(S):
        inside[qsl[s]:min(qsl[s + 1], qsl[s] + 64)] = True
    err = max_err(out[inside], ref[inside])
    say(f"  max_query_len 64, {S} seqs: max|err| = {err:.3e} over {int(inside.sum())} tokens, "
        f"{int((~inside).sum())} past it")
    assert err <= TOL[x.cfg.dtype]
    assert np.isnan(out[~inside]).all()


@pytest.mark.parametrize("mb", WIDE)
@pytest.mark.parametrize("S", [64, 256])
def test_prefill_ranked_order_slot_edges(dev, mb, S):
    """64 sequences (one per lane of the rank search) and 256 (four per lane,
    the most that take the launch order ranked by cost), every token."""
    rng = np.random.default_rng(66)
    x = W.make_prefill_inputs(W.PREFILL_WORKLOADS[2], seed=66, context_lens=rng.integers(0, 500, size=S),
                              query_lens=rng.integers(1, 100, size=S), max_blocks_per_seq=mb)
    say(f"prefill {S} sequences (ranked order): {x.num_query_tokens} tokens")
    check_all(x, run(x, dev), f"{S} sequences")


def test_prefill_mixed_batch_with_chunks_longer_than_their_sequence(dev):
    """A mixed batch (ranked order, not the equal-sequence shortcut) in which two
    chunks claim more tokens than their sequence holds: whole query tiles with
    no visible key (zeros) rank below every other item and still run."""
    cfg = W.PrefillConfig("neg-mixed", 6, 16, 2, 128, "bf16", ("custom",), ("custom",))
    x = W.make_prefill_inputs(cfg, seed=67, context_lens=[0, 300, 0, 50, 1000, 0],
                              query_lens=[40, 20, 30, 70, 5, 64])
    claim = {0: 100, 2: 40}  # extra query tokens at negative positions, before the chunk's own
    rows, qsl, ql = [], [0], []
    for s in range(cfg.num_seqs):
        extra = claim.get(s, 0)
        if extra:
            rows.append(W.make_prefill_inputs(cfg, seed=68 + s, context_lens=[0] * 6, query_lens=[extra] * 6)
                        .q[:extra])
        rows.append(x.q[x.query_start_loc[s]:x.query_start_loc[s + 1]])
        ql.append(int(x.query_lens[s]) + extra)
        qsl.append(qsl[-1] + ql[-1])
    x.q = np.concatenate(rows)
    x.query_lens = np.array(ql, dtype=np.int32)
    x.query_start_loc = np.array(qsl, dtype=np.int32)
    say(f"prefill mixed batch, chunks longer than their sequence: {x.num_query_tokens} tokens")
    got = check_all(x, run(x, dev), "negative positions, mixed batch")
    assert (got[0:100] == 0).all() and (got[qsl[2]:qsl[2] + 40] == 0).all()


@pytest.mark.parametrize("S", [16, 64, 100])
def test_prefill_fresh_prompts_of_different_lengths(dev, S):
    """No prefix, chunks of different lengths (every sequence's prefix is the
    same: up to 64 sequences the ranked search, above it the round order), and
    the same with equal chunks (the equal-sequence shortcut), every token."""
    rng = np.random.default_rng(70 + S)
    for label, ql in (("mixed chunks", rng.integers(1, 200, size=S)), ("equal chunks", np.full(S, 77))):
        x = W.make_prefill_inputs(W.PREFILL_WORKLOADS[2], seed=70 + S, context_lens=[0] * S, query_lens=ql)
        say(f"prefill {S} fresh prompts, {label}: {x.num_query_tokens} tokens")
        check_all(x, run(x, dev), f"{S} fresh prompts, {label}")
        # the same prefix for every sequence, not zero
        x = W.make_prefill_inputs(W.PREFILL_WORKLOADS[2], seed=71 + S, context_lens=[300] * S, query_lens=ql)
        check_all(x, run(x, dev), f"{S} prompts behind equal prefixes, {label}")
