"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle.

Tolerances (max |error| over every compared element): 1e-3 for fp32 caches,
2e-2 for bf16 caches with fp32 accumulation. Integer results (the gather
trace, the error word) must match exactly.
"""
import numpy as np
import pytest
import torch

import oracle
import paged_attention_decode_06_amd as pa
from paged_attention_decode_06_amd import workloads as W

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-3, "bf16": 2e-2, "f16": 1e-2}
MODES = ("auto", "v1", "v2")
# Table widths: the natural one, and 4096 blocks, which gives 128 partitions
# per sequence and so exercises the one-partition-per-wave launch layout.
WIDTHS = (None, 4096)


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    pa.load()
    return torch.device("cuda:0")


def say(*a):
    print(*a, flush=True)


def run(x, dev, mode="auto", d=None, ps=0):
    """Run one decode (ps: partition size, 0 = the 512 default); returns
    (out, (exp_sums, max_logits, tmp_out)) as device tensors."""
    d = d or W.to_device(x, dev)
    out = torch.full_like(d["q"], float("nan"))
    sh = pa.make_shape(d["q"], d["k_cache"], d["block_tables"], ps)
    es, ml, to = pa.alloc_partials(sh, dev)
    for t in (es, ml, to):
        t.fill_(float("nan"))
    args = (out, d["q"], d["k_cache"], d["v_cache"], d["block_tables"], d["seq_lens"], x.scale)
    if mode == "auto":
        pa.pa_decode(*args, es, ml, to, partition_size=ps)
    elif mode == "v1":
        pa.pa_decode_v1(*args)
    elif mode == "v2":
        pa.pa_decode_v2(*args, es, ml, to, partition_size=ps)
    else:
        raise ValueError(mode)
    torch.cuda.synchronize(dev)
    return out, (es, ml, to)


def ref_rows(x, seqs=None):
    """Oracle rows of the given sequences (all by default), one sequence per
    task on a thread pool sized to the host's cores (the oracle's matrix
    products release the interpreter lock), each task's BLAS single-threaded."""
    import os
    from concurrent.futures import ThreadPoolExecutor
    seqs = list(range(x.cfg.num_seqs) if seqs is None else seqs)
    lists = oracle.gather_list(x.block_tables, x.seq_lens)
    one = lambda s: oracle.attend_seq(x.q[s], x.k_cache, x.v_cache, lists[s], int(x.seq_lens[s]), x.scale,
                                      x.cfg.dtype)
    from threadpoolctl import threadpool_limits
    workers = max(1, min(16, len(os.sched_getaffinity(0)), len(seqs)))
    # one BLAS thread per task: a pool over multithreaded BLAS oversubscribes
    # the cores (measured 40x slower on the batch-256 workload)
    with threadpool_limits(1), ThreadPoolExecutor(workers) as ex:
        return dict(zip(seqs, ex.map(one, seqs)))


def max_err(got, ref):
    e = np.abs(got - ref)
    return float("inf") if np.isnan(e).any() else float(e.max(initial=0.0))


def assert_close(x, out, seqs=None, label=""):
    got = W.from_device(out)
    refs = ref_rows(x, seqs)
    worst = max(max_err(got[s], r) for s, r in refs.items())
    say(f"  {label} {x.cfg.name}: max|err| = {worst:.3e} over {len(refs)} seqs (tol {TOL[x.cfg.dtype]})")
    assert worst <= TOL[x.cfg.dtype], f"{label}: {worst}"
    return got


# ---------------------------------------------------------------- the five workloads
@pytest.mark.parametrize("num", [1, 2, 3, 4, 5])
def test_config_parity(dev, num):
    say(f"config {num}: generating")
    x = W.make_inputs(num)
    say(f"config {num} {x.cfg.name}: S={x.cfg.num_seqs} sum(L)={int(x.seq_lens.sum())} NB={x.num_blocks}; pa_decode")
    out, _ = run(x, dev, "auto")
    got = assert_close(x, out, None, "auto")   # every output row of every workload
    assert np.isfinite(got).all()


def test_long_context_f16(dev):
    """The 100K-token shape with an fp16 cache (fp16 variant of the path)."""
    cfg = W.DecodeConfig("ctx100K-f16", 1, 16, 2, 128, "f16", ("fixed", 100000))
    x = W.make_inputs(cfg, seed=1103)
    say("100K-token context, fp16 cache")
    out, _ = run(x, dev, "auto")
    assert np.isfinite(assert_close(x, out, label="auto")).all()


# ---------------------------------------------------------------- paths agree
MIXED = [1, 37, 512, 513, 5000, 8192, 8193, 20000]


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("width", WIDTHS)
@pytest.mark.parametrize("D", [128, 256])
@pytest.mark.parametrize("mode", MODES)
def test_modes_vs_oracle(dev, D, mode, width, dtype):
    cfg = W.DecodeConfig(f"mixed-{dtype}-d{D}", len(MIXED), 16, 2, D, dtype, ("custom",))
    x = W.make_inputs(cfg, seed=11, seq_lens=MIXED, max_blocks_per_seq=width)
    say(f"mode {mode} D={D} lens={MIXED} table width={x.max_blocks_per_seq}")
    out, _ = run(x, dev, mode)
    assert_close(x, out, label=mode)


def test_v1_and_v2_agree(dev):
    cfg = W.DecodeConfig("v1v2", len(MIXED), 16, 2, 128, "bf16", ("custom",))
    x = W.make_inputs(cfg, seed=12, seq_lens=MIXED)
    d = W.to_device(x, dev)
    say("v1 vs v2 on", MIXED)
    o1 = W.from_device(run(x, dev, "v1", d)[0])
    o2 = W.from_device(run(x, dev, "v2", d)[0])
    oa = W.from_device(run(x, dev, "auto", d)[0])
    assert max_err(o1, o2) <= 2e-2
    long_ = np.asarray(MIXED) > 8192
    # AUTO runs the single pass for short contexts; forced V1 may use another
    # launch shape (waves split the tokens differently), so equal up to rounding.
    assert max_err(oa[~long_], o1[~long_]) <= 2e-2
    # the two phases for long contexts use the same launch shape: bitwise equal
    assert np.array_equal(oa[long_], o2[long_])


@pytest.mark.parametrize("dtype,D,H,Hkv", [("bf16", 128, 32, 2), ("bf16", 256, 4, 4), ("f32", 256, 3, 1),
                                           ("f32", 128, 16, 2), ("bf16", 128, 5, 1), ("f16", 128, 16, 2),
                                           ("f16", 256, 8, 1),
                                           # group size 16 at head_dim 256: the merge rows need more than
                                           # the default 64 KB of LDS (fp32 and the 16-bit single pass)
                                           ("f32", 256, 16, 1), ("bf16", 256, 16, 1), ("bf16", 128, 16, 1)])
@pytest.mark.parametrize("mode", MODES)
def test_group_sizes(dev, dtype, D, H, Hkv, mode):
    lens = [3, 600, 9000]
    cfg = W.DecodeConfig(f"g{H // Hkv}-{dtype}-d{D}", len(lens), H, Hkv, D, dtype, ("custom",))
    x = W.make_inputs(cfg, seed=13, seq_lens=lens)
    say(f"group size {H // Hkv} {dtype} D={D} mode={mode}")
    out, _ = run(x, dev, mode)
    assert_close(x, out, label=mode)


# ---------------------------------------------------------------- edge cases
EDGE = [1, 15, 16, 17, 37, 511, 512, 513, 8191, 8192, 8193, 16384]


@pytest.mark.parametrize("dtype,D", [("bf16", 128), ("bf16", 256), ("f32", 128), ("f16", 128), ("f16", 256)])
@pytest.mark.parametrize("mode", MODES)
def test_edge_lengths(dev, dtype, D, mode):
    cfg = W.DecodeConfig(f"edge-{dtype}-d{D}", len(EDGE), 16, 2, D, dtype, ("custom",))
    x = W.make_inputs(cfg, seed=14, seq_lens=EDGE)
    say(f"edge lengths {dtype} D={D} mode={mode}")
    out, _ = run(x, dev, mode)
    assert_close(x, out, label=mode)


@pytest.mark.parametrize("mode", MODES)
def test_zero_length_contexts_write_zeros(dev, mode):
    lens = [0, 5, 0, 9000]
    cfg = W.DecodeConfig("zero", len(lens), 16, 2, 128, "bf16", ("custom",))
    x = W.make_inputs(cfg, seed=15, seq_lens=lens)
    say(f"zero-length contexts mode={mode}")
    out, _ = run(x, dev, mode)
    got = W.from_device(out)
    assert np.array_equal(got[0], np.zeros_like(got[0])) and np.array_equal(got[2], np.zeros_like(got[2]))
    assert_close(x, out, seqs=[1, 3], label=mode)


@pytest.mark.parametrize("mode", MODES)
def test_compact_work_list_over_several_chunks(dev, mode):
    """130 sequences: the kernel's work-list scan walks three 64-sequence
    chunks (the last one partial). Zero, short, threshold-edge and long
    contexts are mixed; every output row is checked, and on the partitioned
    path every partial of every sequence with partitions."""
    rng = np.random.default_rng(1130)
    lens = rng.integers(1, 3000, size=130)
    lens[::7] = 0
    lens[5::11] = rng.integers(8193, 20000, size=lens[5::11].size)
    lens[3], lens[4], lens[127] = 8192, 8193, 20000
    cfg = W.DecodeConfig("compact130", lens.size, 16, 2, 128, "bf16", ("custom",))
    x = W.make_inputs(cfg, seed=1130, seq_lens=lens.tolist())
    say(f"compact work list: 130 seqs, mode={mode}")
    out, (es, ml, to) = run(x, dev, mode)
    got = assert_close(x, out, label=f"compact {mode}")
    for s_ in np.where(lens == 0)[0]:
        assert np.array_equal(got[s_], np.zeros_like(got[s_]))
    if mode == "v1":
        return
    lists = oracle.gather_list(x.block_tables, x.seq_lens)
    es, ml, to = es.cpu().numpy(), ml.cpu().numpy(), to.cpu().numpy()
    for s_, L in enumerate(lens.tolist()):
        P = 0 if (mode == "auto" and L <= 8192) else oracle.num_partitions(L, 512)
        if P:
            m, l, o = oracle.partition_stats(x.q[s_], x.k_cache, x.v_cache, lists[s_], L, x.scale, "bf16", 512)
            assert np.abs(ml[s_, :, :P] - m).max() <= 1e-3
            assert (np.abs(es[s_, :, :P] - l) / l).max() <= 1e-2
            assert max_err(to[s_, :, :P], o) <= 2e-2
        assert np.isnan(ml[s_, :, P:]).all() and np.isnan(to[s_, :, P:]).all()   # untouched


@pytest.mark.parametrize("S", [600, 1024])
def test_compact_work_list_large_batches(dev, S):
    """600 and 1024 sequences: the length pass over 10 and 16 chunks of 64
    (its unrolled body and its remainder), mostly short contexts with a long
    partitioned one now and then, in a table 16K tokens wide; every row is
    checked."""
    rng = np.random.default_rng(S)
    lens = rng.integers(0, 301, size=S)
    long_ = rng.random(S) < 0.03
    lens[long_] = rng.integers(8193, 12001, size=int(long_.sum()))
    lens[-1] = 12000
    cfg = W.DecodeConfig(f"compact{S}", S, 16, 2, 128, "bf16", ("custom",))
    x = W.make_inputs(cfg, seed=S, seq_lens=lens.tolist(), max_blocks_per_seq=1024)
    say(f"compact work list: {S} seqs, {int(long_.sum()) + 1} partitioned")
    out, _ = run(x, dev, "auto")
    assert_close(x, out, label=f"compact {S}")


def _random_case(i):
    """Shape and lengths of seeded random case i (sizes the oracle finishes
    in well under a second)."""
    rng = np.random.default_rng(5000 + i)
    dtype = ("bf16", "f16", "f32")[rng.integers(3)]
    D = int(rng.choice([128, 256]))
    Hkv = int(rng.choice([1, 2, 4]))
    G = int(rng.choice([1, 2, 4, 8]))
    S = int(rng.choice([1, 2, 3, 17, 64, 65, 200]))
    short = rng.integers(0, 700, size=S)
    longs = rng.integers(8000, 9400, size=S)      # both sides of the threshold
    lens = np.where(rng.random(S) < 0.3, longs, short)
    width = int(rng.choice([0, 700, 2048]))       # 0: the narrowest table
    width = None if width == 0 else max(width, int(-(-lens.max() // 16)))
    mode = ("auto", "v1", "v2")[rng.integers(3)]
    return dtype, D, Hkv, G, S, lens, width, mode


@pytest.mark.parametrize("i", range(24))
def test_random_shapes_vs_oracle(dev, i):
    """Seeded random shapes: dtype, head_dim, KV heads, group size, batch
    size (one sequence, several 64-sequence chunks), lengths on both sides of
    the single-pass threshold, table width and mode; every row against the
    oracle."""
    dtype, D, Hkv, G, S, lens, width, mode = _random_case(i)
    cfg = W.DecodeConfig(f"rand{i}", S, Hkv * G, Hkv, D, dtype, ("custom",))
    x = W.make_inputs(cfg, seed=5000 + i, seq_lens=lens.tolist(), max_blocks_per_seq=width)
    say(f"random case {i}: {dtype} D={D} Hkv={Hkv} G={G} S={S} width={x.max_blocks_per_seq} mode={mode}")
    out, _ = run(x, dev, mode)
    assert_close(x, out, label=f"random {i} {mode}")


def test_batch_above_the_work_list_limit(dev):
    """1100 sequences (above the batch size the compact work list serves):
    the grid keeps its direct order; mostly short contexts with a long
    partitioned one every 100 sequences, every row checked."""
    rng = np.random.default_rng(1100)
    lens = rng.integers(0, 65, size=1100)
    lens[50::100] = rng.integers(9000, 12001, size=lens[50::100].size)
    cfg = W.DecodeConfig("direct1100", lens.size, 16, 2, 128, "bf16", ("custom",))
    x = W.make_inputs(cfg, seed=1100, seq_lens=lens.tolist())
    say("direct order: 1100 seqs")
    out, _ = run(x, dev, "auto")
    assert_close(x, out, label="direct 1100")


def test_graph_replay_matches_eager(dev):
    """pa_decode captured in a HIP graph (as a serving loop would capture a
    decode step): each replay, with q changed in place and eager work in
    between, matches an eager call on the same inputs bit for bit, and the
    last one matches the oracle."""
    lens = [37, 9000, 513, 0, 20000, 8192]
    x = W.make_inputs(W.DECODE_WORKLOADS[2], seed=91, seq_lens=lens)
    d = W.to_device(x, dev)
    q, kc, vc, bt, sl = d["q"], d["k_cache"], d["v_cache"], d["block_tables"], d["seq_lens"]
    sh = pa.make_shape(q, kc, bt)
    es, ml, to = pa.alloc_partials(sh, dev)
    out = torch.empty_like(q)
    side = torch.cuda.Stream(dev)
    side.wait_stream(torch.cuda.current_stream(dev))
    with torch.cuda.stream(side):
        pa.pa_decode(out, q, kc, vc, bt, sl, x.scale, es, ml, to)
    torch.cuda.current_stream(dev).wait_stream(side)
    torch.cuda.synchronize(dev)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        pa.pa_decode(out, q, kc, vc, bt, sl, x.scale, es, ml, to)
    torch.cuda.synchronize(dev)
    say("graph replay vs eager")
    gen = torch.Generator(device="cpu").manual_seed(92)
    ref_out = torch.empty_like(q)
    es2, ml2, to2 = pa.alloc_partials(sh, dev)
    for rep in range(3):
        q.copy_(torch.randn(q.shape, generator=gen).to(q.dtype))
        out.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize(dev)
        pa.pa_decode(ref_out, q, kc, vc, bt, sl, x.scale, es2, ml2, to2)
        torch.cuda.synchronize(dev)
        assert torch.equal(out, ref_out), f"replay {rep}"
    x.q[...] = q.cpu().view(torch.int16).numpy().view(np.uint16)   # bf16 bits, as the workload stores q
    assert_close(x, out, label="graph replay")


def test_empty_batch(dev):
    cfg = W.DecodeConfig("empty", 0, 16, 2, 128, "bf16", ("custom",))
    x = W.make_inputs(cfg, seed=1, seq_lens=np.zeros(0, np.int32))
    say("empty batch")
    out, _ = run(x, dev, "auto")
    assert out.numel() == 0


@pytest.mark.parametrize("dtype", ["bf16", "f32", "f16"])
@pytest.mark.parametrize("width", [600, 4096])
@pytest.mark.parametrize("mode", MODES)
def test_poison_outside_contexts_never_reaches_output(dev, dtype, mode, width):
    lens = [37, 1, 8200, 700]
    cfg = W.DecodeConfig(f"poison-{dtype}", len(lens), 16, 2, 128, dtype, ("custom",))
    x = W.make_inputs(cfg, seed=16, seq_lens=lens, max_blocks_per_seq=width, poison=True)
    say(f"poisoned pool {dtype} mode={mode}")
    out, _ = run(x, dev, mode)
    got = assert_close(x, out, label=mode)
    assert np.isfinite(got).all()


# ---------------------------------------------------------------- invariants
def test_block_permutation_is_bitwise_invariant(dev):
    x = W.make_inputs(W.DECODE_WORKLOADS[2], seed=17, seq_lens=[37, 4000, 9000, 20000])
    say("block permutation")
    base = W.from_device(run(x, dev, "auto")[0])
    rng = np.random.default_rng(0)
    perm = rng.permutation(x.num_blocks)
    k2 = np.empty_like(x.k_cache); v2 = np.empty_like(x.v_cache)
    k2[perm] = x.k_cache; v2[perm] = x.v_cache
    x2 = W.DecodeInputs(x.cfg, x.seed, x.seq_lens, perm[x.block_tables].astype(np.int32), x.q, k2, v2, x.scale)
    again = W.from_device(run(x2, dev, "auto")[0])
    assert np.array_equal(base, again)


def test_runs_are_bitwise_deterministic(dev):
    x = W.make_inputs(W.DECODE_WORKLOADS[2], seed=18, seq_lens=[100, 8192, 30000])
    d = W.to_device(x, dev)
    say("determinism")
    a = W.from_device(run(x, dev, "auto", d)[0])
    b = W.from_device(run(x, dev, "auto", d)[0])
    assert np.array_equal(a, b)


@pytest.mark.parametrize("dtype", ["bf16", "f32", "f16"])
def test_single_token_returns_v_exactly(dev, dtype):
    cfg = W.DecodeConfig("one", 3, 16, 2, 128, dtype, ("custom",))
    x = W.make_inputs(cfg, seed=19, seq_lens=[1, 1, 1])
    say(f"single token {dtype}")
    got = W.from_device(run(x, dev, "auto")[0])
    for s in range(3):
        blk = x.block_tables[s, 0]
        for h in range(16):
            v0 = oracle.widen(x.v_cache[blk, h // 8, 0], dtype)
            assert np.array_equal(got[s, h], v0)


@pytest.mark.parametrize("mode", MODES)
def test_constant_v_gives_the_constant(dev, mode):
    x = W.make_inputs(W.DECODE_WORKLOADS[2], seed=20, seq_lens=[37, 8192, 9000, 20000])
    x.v_cache[:] = W.f32_to_bf16_bits(np.full(1, 1.625, np.float32))[0]
    say(f"constant V mode={mode}")
    got = W.from_device(run(x, dev, mode)[0])
    assert np.array_equal(got, np.full_like(got, 1.625))


def test_zero_query_gives_mean_of_v(dev):
    x = W.make_inputs(W.DECODE_WORKLOADS[2], seed=21, seq_lens=[37, 3000, 9000])
    x.q[:] = 0
    say("zero query")
    out, _ = run(x, dev, "auto")
    got = W.from_device(out)
    lists = oracle.gather_list(x.block_tables, x.seq_lens)
    for s in range(3):
        for kv in range(2):
            mean = oracle.gather_kv(x.v_cache, lists[s], kv, int(x.seq_lens[s]), "bf16").mean(axis=0)
            assert max_err(got[s, kv * 8:(kv + 1) * 8], mean[None]) <= 2e-2


# ---------------------------------------------------------------- gather trace, partials, dispatch
@pytest.mark.parametrize("width", [1300, 4096])
@pytest.mark.parametrize("mode", MODES)
def test_gather_trace_matches_oracle_exactly(dev, mode, width):
    lens = [37, 1, 8192, 8193, 20000, 513, 40000, 9000]
    x = W.make_inputs(W.DECODE_WORKLOADS[2], seed=22, seq_lens=lens, max_blocks_per_seq=max(width, 2500), poison=True)
    d = W.to_device(x, dev)
    sh = pa.make_shape(d["q"], d["k_cache"], d["block_tables"])
    es, ml, to = pa.alloc_partials(sh, dev)
    out = torch.empty_like(d["q"])
    trace = torch.full(tuple(x.block_tables.shape), -1, dtype=torch.int32, device=dev)
    err = torch.zeros(1, dtype=torch.int32, device=dev)
    mcode = {"auto": pa.MODE_AUTO, "v1": pa.MODE_V1, "v2": pa.MODE_V2}[mode]
    say(f"gather trace mode={mode}")
    pa.pa_decode_partitions_debug(out, d["q"], d["k_cache"], d["v_cache"], d["block_tables"], d["seq_lens"],
                                  x.scale, es, ml, to, mcode, trace, err)
    torch.cuda.synchronize(dev)
    tr = trace.cpu().numpy()
    for s, ids in enumerate(oracle.gather_list(x.block_tables, x.seq_lens)):
        assert np.array_equal(tr[s, :ids.size], ids)
        assert (tr[s, ids.size:] == -1).all()
    assert int(err.item()) == 0


@pytest.mark.parametrize("ps", [512, 256])
@pytest.mark.parametrize("width", WIDTHS)
def test_partials_match_oracle_partition_stats(dev, width, ps):
    lens = [1100, 513, 9000, 1, 257]
    x = W.make_inputs(W.DECODE_WORKLOADS[2], seed=23, seq_lens=lens, max_blocks_per_seq=width)
    d = W.to_device(x, dev)
    sh = pa.make_shape(d["q"], d["k_cache"], d["block_tables"], ps)
    es, ml, to = pa.alloc_partials(sh, dev)
    for t in (es, ml, to):
        t.fill_(float("nan"))
    out = torch.empty_like(d["q"])
    say(f"V2 partials vs oracle, partition size {ps}")
    pa.pa_decode_partitions(out, d["q"], d["k_cache"], d["v_cache"], d["block_tables"], d["seq_lens"], x.scale,
                            es, ml, to, pa.MODE_V2, partition_size=ps)
    torch.cuda.synchronize(dev)
    assert es.shape[2] == -(-x.max_blocks_per_seq * 16 // ps)
    es, ml, to = es.cpu().numpy(), ml.cpu().numpy(), to.cpu().numpy()
    lists = oracle.gather_list(x.block_tables, x.seq_lens)
    for s, L in enumerate(lens):
        m, l, o = oracle.partition_stats(x.q[s], x.k_cache, x.v_cache, lists[s], L, x.scale, "bf16", ps)
        P = oracle.num_partitions(L, ps)
        assert np.abs(ml[s, :, :P] - m).max() <= 1e-3
        assert (np.abs(es[s, :, :P] - l) / l).max() <= 1e-2
        assert max_err(to[s, :, :P], o) <= 2e-2
        assert np.isnan(ml[s, :, P:]).all() and np.isnan(to[s, :, P:]).all()   # untouched


# (S, H, D): the reduce picks its slice width from S * H rows; these reach the
# 32-, 64-, 128- and 256-wide slices.
REDUCE_SHAPES = [(3, 4, 128), (64, 16, 128), (128, 16, 128), (128, 16, 256)]


@pytest.mark.parametrize("S,H,D,ps", [(*sh, 512) for sh in REDUCE_SHAPES] + [(64, 16, 128, 256), (3, 4, 256, 256)])
@pytest.mark.parametrize("dtype", ["bf16", "f32", "f16"])
def test_reduce_fed_with_oracle_partials(dev, dtype, S, H, D, ps):
    rng = np.random.default_rng(24)
    MB = 100                               # Pmax = ceil(100*16/ps): 4 at 512, 7 at 256
    lens = rng.integers(1, 1601, size=S).astype(np.int32)
    lens[0] = 1600
    P = -(-MB * 16 // ps)
    m = rng.normal(0, 5, (S, H, P)); l = rng.uniform(1, 50, (S, H, P)); o = rng.normal(0, 1, (S, H, P, D))
    want = np.zeros((S, H, D))
    for s in range(S):
        n = oracle.num_partitions(int(lens[s]), ps)
        for h in range(H):
            want[s, h] = oracle.lse_combine(m[s, h, :n], l[s, h, :n], o[s, h, :n])
    tdt = {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}[dtype]
    code = {"bf16": pa.PA_BF16, "f16": pa.PA_F16, "f32": pa.PA_F32}[dtype]
    out = torch.full((S, H, D), float("nan"), dtype=tdt, device=dev)
    to_t = lambda a: torch.from_numpy(a.astype(np.float32)).to(dev)
    sh = pa.PaShape(S, H, 1, D, 16, MB, 10, code, 0 if ps == 512 else ps)
    assert pa.max_partitions(sh) == P
    say(f"reduce from oracle partials {dtype} S={S} H={H} D={D} partition size {ps}")
    pa.pa_lse_reduce(out, to_t(l), to_t(m), to_t(o), torch.from_numpy(lens).to(dev), sh, pa.MODE_V2)
    torch.cuda.synchronize(dev)
    assert max_err(W.from_device(out), want) <= {"bf16": 2e-2, "f16": 5e-3, "f32": 1e-5}[dtype]


@pytest.mark.parametrize("width", WIDTHS)
def test_auto_writes_partials_only_for_long_contexts(dev, width):
    lens = [37, 8192, 8193, 20000, 600]
    x = W.make_inputs(W.DECODE_WORKLOADS[2], seed=25, seq_lens=lens, max_blocks_per_seq=width)
    d = W.to_device(x, dev)
    sh = pa.make_shape(d["q"], d["k_cache"], d["block_tables"])
    es, ml, to = pa.alloc_partials(sh, dev)
    for t in (es, ml, to):
        t.fill_(float("nan"))
    out = torch.full_like(d["q"], float("nan"))
    say("AUTO dispatch")
    pa.pa_decode_partitions(out, d["q"], d["k_cache"], d["v_cache"], d["block_tables"], d["seq_lens"], x.scale,
                            es, ml, to, pa.MODE_AUTO)
    torch.cuda.synchronize(dev)
    ml_h = ml.cpu().numpy(); got = W.from_device(out)
    for s, L in enumerate(lens):
        if oracle.choose_path(L) == "v2":
            assert np.isfinite(ml_h[s, :, :oracle.num_partitions(L)]).all()
            assert np.isnan(got[s]).all()            # phase 2 not run yet
        else:
            assert np.isnan(ml_h[s]).all()
            assert np.isfinite(got[s]).all()


def test_data_errors_are_flagged_not_faulted(dev):
    x = W.make_inputs(W.DECODE_WORKLOADS[2], seed=26, seq_lens=[40, 40])
    x.block_tables[1, 1] = x.num_blocks + 5          # out of the pool
    x.seq_lens[0] = 40 + 16 * x.max_blocks_per_seq    # longer than the table
    d = W.to_device(x, dev)
    sh = pa.make_shape(d["q"], d["k_cache"], d["block_tables"])
    es, ml, to = pa.alloc_partials(sh, dev)
    out = torch.empty_like(d["q"])
    err = torch.zeros(1, dtype=torch.int32, device=dev)
    say("data errors")
    pa.pa_decode_partitions_debug(out, d["q"], d["k_cache"], d["v_cache"], d["block_tables"], d["seq_lens"],
                                  x.scale, es, ml, to, pa.MODE_AUTO, None, err)
    torch.cuda.synchronize(dev)
    assert int(err.item()) == 3


@pytest.mark.parametrize("mode", MODES)
def test_timed_entry_points_match_untimed(dev, mode):
    """The *_timed forms run the same kernels: bitwise equal outputs, and both
    event pairs complete (also where the reduce has nothing to launch)."""
    x = W.make_inputs(W.DECODE_WORKLOADS[2], seed=19, seq_lens=[5, 3000, 8192, 8193, 40000])
    d = W.to_device(x, dev)
    say(f"timed entry points, mode {mode}")
    m = {"auto": pa.MODE_AUTO, "v1": pa.MODE_V1, "v2": pa.MODE_V2}[mode]
    args = (d["q"], d["k_cache"], d["v_cache"], d["block_tables"], d["seq_lens"], x.scale)
    sh = pa.make_shape(d["q"], d["k_cache"], d["block_tables"])
    outs = []
    hev = pa.HipEvents()
    try:
        for timed in (False, True):
            out = torch.full_like(d["q"], float("nan"))
            es, ml, to = pa.alloc_partials(sh, dev)
            if timed:
                ev = [hev.new() for _ in range(4)]
                pa.pa_decode_partitions_timed(out, *args, es, ml, to, m, ev[0], ev[1])
                pa.pa_lse_reduce_timed(out, es, ml, to, d["seq_lens"], sh, m, ev[2], ev[3])
            else:
                pa.pa_decode_partitions(out, *args, es, ml, to, m)
                pa.pa_lse_reduce(out, es, ml, to, d["seq_lens"], sh, m)
            torch.cuda.synchronize(dev)
            outs.append(W.from_device(out))
        k1, k2 = hev.ms(ev[0], ev[1]), hev.ms(ev[2], ev[3])
        say(f"  partition {k1 * 1e3:.1f} us, reduce {k2 * 1e3:.1f} us")
        assert k1 > 0 and k2 >= 0
        if mode == "v1":
            assert k2 < 0.05  # nothing launched: the two marks are back to back
    finally:
        hev.close()
    assert np.array_equal(outs[0], outs[1])
    assert_close(x, torch.from_numpy(outs[1]).to(dev))


def test_timed_entry_points_on_an_empty_batch(dev):
    x = W.make_inputs(W.DECODE_WORKLOADS[2], seed=20, seq_lens=[7])
    d = W.to_device(x, dev)
    q0 = d["q"][:0]
    out = torch.empty_like(q0)
    sh = pa.make_shape(q0, d["k_cache"], d["block_tables"][:0])
    es, ml, to = pa.alloc_partials(sh, dev)
    hev = pa.HipEvents()
    try:
        ev = [hev.new() for _ in range(4)]
        pa.pa_decode_partitions_timed(out, q0, d["k_cache"], d["v_cache"], d["block_tables"][:0],
                                      d["seq_lens"][:0], x.scale, es, ml, to, pa.MODE_AUTO, ev[0], ev[1])
        pa.pa_lse_reduce_timed(out, es, ml, to, d["seq_lens"][:0], sh, pa.MODE_AUTO, ev[2], ev[3])
        torch.cuda.synchronize(dev)
        assert hev.ms(ev[0], ev[1]) >= 0 and hev.ms(ev[2], ev[3]) >= 0
    finally:
        hev.close()


# ---------------------------------------------------------------- opt-in 256-token partitions
@pytest.mark.parametrize("num", [3, 5])
def test_config_parity_partition_256(dev, num):
    x = W.make_inputs(num)
    say(f"config {num} {x.cfg.name} with 256-token partitions")
    out, _ = run(x, dev, "auto", ps=256)
    assert np.isfinite(assert_close(x, out, None, "auto/256")).all()


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("width", WIDTHS)
@pytest.mark.parametrize("D", [128, 256])
@pytest.mark.parametrize("mode", ["auto", "v2"])
def test_modes_vs_oracle_partition_256(dev, D, mode, width, dtype):
    lens = [1, 37, 255, 256, 257, 512, 513, 8192, 8193, 20000]
    cfg = W.DecodeConfig(f"ps256-{dtype}-d{D}", len(lens), 16, 2, D, dtype, ("custom",))
    x = W.make_inputs(cfg, seed=31, seq_lens=lens, max_blocks_per_seq=width)
    say(f"partition 256, mode {mode} D={D} {dtype} table width={x.max_blocks_per_seq}")
    out, _ = run(x, dev, mode, ps=256)
    assert_close(x, out, label=f"{mode}/256")


@pytest.mark.parametrize("mode", ["auto", "v2"])
def test_gather_trace_partition_256(dev, mode):
    lens = [300, 4000, 9000]
    x = W.make_inputs(W.DECODE_WORKLOADS[2], seed=32, seq_lens=lens, max_blocks_per_seq=1300)
    d = W.to_device(x, dev)
    sh = pa.make_shape(d["q"], d["k_cache"], d["block_tables"], 256)
    es, ml, to = pa.alloc_partials(sh, dev)
    out = torch.empty_like(d["q"])
    trace = torch.full(tuple(x.block_tables.shape), -7, dtype=torch.int32, device=dev)
    err = torch.zeros(1, dtype=torch.int32, device=dev)
    m = {"auto": pa.MODE_AUTO, "v2": pa.MODE_V2}[mode]
    say(f"gather trace, partition 256, mode {mode}")
    pa.pa_decode_partitions_debug(out, d["q"], d["k_cache"], d["v_cache"], d["block_tables"], d["seq_lens"],
                                  x.scale, es, ml, to, m, trace, err, partition_size=256)
    torch.cuda.synchronize(dev)
    got = trace.cpu().numpy()
    for s, ids in enumerate(oracle.gather_list(x.block_tables, x.seq_lens)):
        assert np.array_equal(got[s, :len(ids)], ids)
        assert (got[s, len(ids):] == -7).all()
    assert int(err.item()) == 0


def test_partition_256_and_512_agree(dev):
    x = W.make_inputs(W.DECODE_WORKLOADS[2], seed=33, seq_lens=[9000, 30000, 100])
    d = W.to_device(x, dev)
    say("256 vs 512 partitions")
    a = W.from_device(run(x, dev, "v2", d)[0])
    b = W.from_device(run(x, dev, "v2", d, ps=256)[0])
    assert max_err(a, b) <= 2 * TOL["bf16"]
    assert_close(x, torch.from_numpy(b).to(dev), label="v2/256")
