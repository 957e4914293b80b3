"""Benchmark: paged-attention decode on one MI355X.

A step is one pa_decode call (per-sequence V1/V2 dispatch, partition kernel,
log-sum-exp reduce kernel) over one batch of synthetic inputs already resident
in HBM. Before every timed step a 1 GiB scrub *read* evicts the L2s and the
256 MB Infinity Cache, so a workload that would fit there is still read from
HBM; the scrub sits outside the timed window (events bracket the decode call
only). A read scrub leaves no dirty lines behind: a 1 GiB write scrub was
measured to slow the timed 100K-token step by ~18 us through write-backs that
compete with the decode's reads. The default workload is the 100K-token decode
(1 sequence, 16 query / 2 KV heads, head_dim 128, bf16, 196 partitions of 512
tokens).

Timing events: the step's two events are timing-only events
(hipEventDisableSystemFence, which the HIP runtime documents for timing): a
default event also writes back and invalidates the caches at system scope when
it is recorded, which on this GPU adds ~2 us to every marked interval (two
default events with nothing between them read ~4.3 us, timing-only ones
~3.2 us). The default-event figure is reported beside it.

Prints ONE JSON line (per workload with --all):
  value        algorithmic bytes / median event-timed step time, GB/s
  ms_per_step  median cold-cache step time (both kernels and the gap between)
  roofline     the partition kernel's algorithmic bytes / its mean duration,
               against 8 TB/s. The duration comes from HIP events that the
               library records at the start and the end of that kernel's own
               dispatch (pa_decode_partitions_timed), on the launch stream,
               over the same kind of scrubbed steps; it reads about 1 us above
               the profiler's per-dispatch average (the attached events' cost).
  cpu_baseline the fp64 oracle timed on this host's cores (bounded sample)

--floors measures, on the same workload and buffers, what the decode is up
against on this GPU: an empty launch, event pairs with nothing between them,
and a read-only pass over exactly the decode's K/V bytes in its block order
(include/pa_probe.h) at several workgroup sizes, beside the decode kernels;
--cold-only runs just the warmup and the timed scrubbed steps (for a
profiler run whose per-dispatch averages then cover cold calls only);
--copy-calibration MiB runs a plain device-to-device copy of that size, the
reference for scaling the FETCH_SIZE / WRITE_SIZE counters;
--partition-size 256 measures the opt-in 256-token partitions (not the
headline: 512 is the method's size).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "paged-attn decode achieved HBM GB/s (% of peak) + µs/step at 100K ctx"
PEAK_GBS = 8000.0
SCRUB_BYTES = 1 << 30
CSRC = os.path.join(ROOT, "paged_attention_decode_06_amd", "csrc")
# Sources of the decode kernels (the counter summary is tied to these bytes)
KERNEL_SRCS = [os.path.join(CSRC, "pa_decode.hip"), os.path.join(CSRC, "pa_common.h")]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_counters.txt")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


_CODE_TOKENS = re.compile(r'("(?:\\.|[^"\\\n])*")|//[^\n]*|/\*.*?\*/', re.S)


def code_only(text: str) -> str:
    """C/C++ source with comments removed and whitespace runs collapsed, so
    that editing a comment does not change a kernel's source hash (string
    literals, such as inline assembly, are kept as written)."""
    text = _CODE_TOKENS.sub(lambda m: m.group(1) or " ", text)
    return " ".join(text.split())


def kernel_source_hash(paths=None) -> str:
    """Hash of the code (comments excluded) of the given kernel sources."""
    h = hashlib.sha256()
    for p in (paths or KERNEL_SRCS):
        h.update(code_only(open(p).read()).encode())
        h.update(b"\0")
    return h.hexdigest()[:16]


def workload_label(x, ps: int = 512) -> dict:
    c = x.cfg
    lens = x.seq_lens
    n_v2 = int((lens > 8192).sum())
    return {
        "workload": c.name,
        "num_seqs": c.num_seqs, "num_heads": c.num_heads, "num_kv_heads": c.num_kv_heads,
        "head_dim": c.head_dim, "block_size": 16, "cache_dtype": c.dtype,
        "seq_lens": "x".join(map(str, lens.tolist())) if lens.size <= 4 else
                    f"{c.lengths[0]}{list(c.lengths[1:])}: sum={int(lens.sum())} min={int(lens.min())} max={int(lens.max())}",
        "seqs_on_v2": n_v2, "partition_size": ps, "v2_threshold": 8192,
        "seed": x.seed,
    }


def partition_kernel_bytes(x, elem) -> int:
    """Algorithmic bytes the partition kernel must move: K and V of every
    context token per KV head (2 * D * elem), q, the table entries and
    seq_lens, and the out rows of single-pass sequences."""
    from paged_attention_decode_06_amd import workloads as W
    c = x.cfg
    total = W.algorithmic_bytes(x.seq_lens, c.num_heads, c.num_kv_heads, c.head_dim, elem)
    v2_rows = int((x.seq_lens > 8192).sum()) * c.num_heads * c.head_dim * elem
    return total - v2_rows        # out of V2 rows is written by the reduce kernel


def read_traffic_file(path: str = TRAFFIC_FILE) -> dict:
    """`key: value` lines of the committed counter summary (text)."""
    rec = {}
    try:
        for line in open(path):
            line = line.split("#", 1)[0].strip()
            if ":" in line:
                k, v = line.split(":", 1)
                rec[k.strip()] = v.strip()
    except OSError:
        pass
    return rec


def traffic_for(num: int):
    """Calibrated HBM bytes (FETCH + WRITE) per partition-kernel launch from the
    committed counter runs, when they were taken on the current kernel source;
    otherwise None."""
    rec = read_traffic_file()
    if rec.get("kernel_source_sha256_16") != kernel_source_hash():
        return None
    v = rec.get(f"workload_{num}_partition_traffic_bytes")
    return None if v is None else int(float(v))


def moe_traffic_for(num: int, stage: str):
    """Calibrated HBM bytes per launch of a MoE stage's kernel from the
    committed counter runs, when they were taken on the current MoE kernel
    source; otherwise None."""
    rec = read_traffic_file()
    if rec.get("moe_kernel_source_sha256_16") != kernel_source_hash([os.path.join(CSRC, "pa_moe.hip")]):
        return None
    v = rec.get(f"moe_{num}_{stage}_traffic_bytes")
    return None if v is None else int(float(v))


def host_cores() -> int:
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        return os.cpu_count() or 1


def cpu_baseline(x, gpu_out, budget_s: float):
    """Time the fp64 oracle on the host's cores over a bounded sample of the
    workload: whole sequences, one per task on a thread pool sized to the
    cores this process may run on (each task's matrix products single-threaded,
    so the pool is what spreads the work), in a fixed random order until the
    time budget is spent (the workload is repeated when it is shorter)."""
    from concurrent.futures import ThreadPoolExecutor

    import oracle
    from paged_attention_decode_06_amd import workloads as W
    try:
        from threadpoolctl import threadpool_limits
    except Exception:  # pragma: no cover
        threadpool_limits = None
    c = x.cfg
    cores = host_cores()
    lists = oracle.gather_list(x.block_tables, x.seq_lens)
    order = [int(s) for s in np.random.default_rng(0).permutation(c.num_seqs)]
    got = W.from_device(gpu_out)
    elem = 4 if c.dtype == "f32" else 2

    def one(s):
        return s, oracle.attend_seq(x.q[s], x.k_cache, x.v_cache, lists[s], int(x.seq_lens[s]), x.scale, c.dtype)

    sample_bytes, tokens, visits, worst = 0, 0, 0, 0.0
    checked = set()
    limits = threadpool_limits(1) if threadpool_limits else None
    try:
        with ThreadPoolExecutor(cores) as ex:
            t0 = time.perf_counter()
            i = 0
            while time.perf_counter() - t0 < budget_s and visits < 100000:
                batch = [order[(i + j) % len(order)] for j in range(cores)]
                i += cores
                for s, ref in ex.map(one, batch):
                    if s not in checked:
                        worst = max(worst, float(np.abs(got[s] - ref).max()))
                        checked.add(s)
                    L = int(x.seq_lens[s])
                    sample_bytes += W.algorithmic_bytes([L], c.num_heads, c.num_kv_heads, c.head_dim, elem)
                    tokens += L
                    visits += 1
            elapsed = time.perf_counter() - t0
    finally:
        if limits is not None:
            limits.restore_original_limits()
    return {
        "value": round(sample_bytes / elapsed / 1e9, 4), "unit": "GB/s", "cores": int(cores), "kind": "oracle",
        "sample": f"fp64 NumPy oracle over {visits} sequence visits ({len(checked)} distinct of {c.num_seqs}, "
                  f"{tokens} context tokens) in {elapsed:.1f} s on a pool of {cores} threads, one sequence "
                  "per task, single-threaded BLAS per task",
        "seconds": round(elapsed, 3),
        "max_abs_err_vs_gpu": worst,
    }


def bench_one(num: int, steps: int, warmup: int, scrub: bool, cpu_budget: float, dev, cold_only=False,
              ps: int = 512):
    import torch

    import paged_attention_decode_06_amd as pa
    from paged_attention_decode_06_amd import workloads as W

    t0 = time.time()
    x = W.make_inputs(num)
    log(f"[bench] config {num} {x.cfg.name}: inputs drawn in {time.time() - t0:.1f}s; "
        f"sum(L)={int(x.seq_lens.sum())}")
    d = W.to_device(x, dev)
    q, kc, vc, bt, sl = d["q"], d["k_cache"], d["v_cache"], d["block_tables"], d["seq_lens"]
    out = torch.empty_like(q)
    sh = pa.make_shape(q, kc, bt, ps)
    es, ml, to = pa.alloc_partials(sh, dev)
    elem = 4 if x.cfg.dtype == "f32" else 2
    step_bytes = W.algorithmic_bytes(x.seq_lens, x.cfg.num_heads, x.cfg.num_kv_heads, x.cfg.head_dim, elem)
    pk_bytes = partition_kernel_bytes(x, elem)
    scrub_buf = torch.empty(SCRUB_BYTES // 4, dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)

    def step():
        pa.pa_decode(out, q, kc, vc, bt, sl, x.scale, es, ml, to, stream=stream, partition_size=ps)

    sink = torch.empty((), dtype=torch.float32, device=dev)

    def do_scrub(i):
        if scrub:
            torch.sum(scrub_buf, dim=None, out=sink)

    for i in range(warmup):
        do_scrub(i)
        step()
    torch.cuda.synchronize(dev)

    # --- timed region: K steps, each bracketed by timing-only events (scrub outside the events)
    hev = pa.HipEvents(pa.HipEvents.DISABLE_SYSTEM_FENCE)
    marks = [(hev.new(), hev.new()) for _ in range(steps)]
    torch.cuda.synchronize(dev)
    wall0 = time.perf_counter()
    for i in range(steps):
        do_scrub(i)
        hev.record(marks[i][0], stream)
        step()
        hev.record(marks[i][1], stream)
    torch.cuda.synchronize(dev)
    wall = time.perf_counter() - wall0
    ms = np.array([hev.ms(a, b) for a, b in marks])
    if cold_only:
        hev.close()
        return {"config": workload_label(x, ps), "us_per_step": round(float(np.median(ms)) * 1e3, 2)}

    # --- the same steps between default events (each adds a system-scope cache flush)
    evd = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for i in range(steps):
        do_scrub(i)
        evd[i][0].record(stream)
        step()
        evd[i][1].record(stream)
    torch.cuda.synchronize(dev)
    ms_default = np.array([a.elapsed_time(b) for a, b in evd])

    # --- per-kernel durations: the same scrubbed steps, each kernel launched
    #     with events attached to its own dispatch
    kmarks = [[hev.new() for _ in range(4)] for _ in range(steps)]
    for i in range(steps):
        do_scrub(i)
        a, b, c, d_ = kmarks[i]
        pa.pa_decode_partitions_timed(out, q, kc, vc, bt, sl, x.scale, es, ml, to, pa.MODE_AUTO, a, b,
                                      stream=stream, partition_size=ps)
        pa.pa_lse_reduce_timed(out, es, ml, to, sl, sh, pa.MODE_AUTO, c, d_, stream=stream)
    torch.cuda.synchronize(dev)
    k1 = np.array([hev.ms(m[0], m[1]) for m in kmarks])
    k2 = np.array([hev.ms(m[2], m[3]) for m in kmarks])
    hev.close()
    k1_ms, k2_ms = float(k1.mean()), float(k2.mean())

    def partitions():
        pa.pa_decode_partitions(out, q, kc, vc, bt, sl, x.scale, es, ml, to, pa.MODE_AUTO, stream=stream,
                                partition_size=ps)

    def reduce():
        pa.pa_lse_reduce(out, es, ml, to, sl, sh, pa.MODE_AUTO, stream=stream)

    def pipelined(*work):
        e = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
        e[0].record(stream)
        for i in range(steps):
            do_scrub(i)
            for w in work:
                w()
        e[1].record(stream)
        for i in range(steps):
            do_scrub(i)
        e[2].record(stream)
        torch.cuda.synchronize(dev)
        return (e[0].elapsed_time(e[1]) - e[1].elapsed_time(e[2])) / steps

    pipelined_ms = pipelined(partitions, reduce)

    # --- warm (cache-resident) figure, labelled as such
    hw = pa.HipEvents(pa.HipEvents.DISABLE_SYSTEM_FENCE)
    evw = [(hw.new(), hw.new()) for _ in range(steps)]
    for i in range(steps):
        hw.record(evw[i][0], stream)
        step()
        hw.record(evw[i][1], stream)
    torch.cuda.synchronize(dev)
    warm = np.array([hw.ms(a, b) for a, b in evw])
    hw.close()

    ms_step = float(np.median(ms))
    gbs = step_bytes / (ms_step * 1e-3) / 1e9
    achieved = pk_bytes / (k1_ms * 1e-3) / 1e9
    res = {
        "metric": METRIC,
        "value": round(gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": x.cfg.dtype,
        "data": "synthetic",
        "config": workload_label(x, ps),
        "us_per_step": round(ms_step * 1e3, 2),
        "pct_of_peak": round(100 * gbs / PEAK_GBS, 2),
        "us_per_step_p10_p50_p90": [round(float(np.percentile(ms, p)) * 1e3, 2) for p in (10, 50, 90)],
        "us_per_step_mean": round(float(ms.mean()) * 1e3, 2),
        "step_timing": "median of per-step intervals between timing-only events (hipEventDisableSystemFence) "
                       "recorded before and after pa_decode on the launch stream, each step after a 1 GiB "
                       "read scrub",
        "us_per_step_default_events_p50": round(float(np.median(ms_default)) * 1e3, 2),
        "cache_scrub_bytes_per_step": SCRUB_BYTES if scrub else 0,
        "warm_cache_us_per_step": round(float(np.median(warm)) * 1e3, 2),
        "pipelined_us_per_step": round(pipelined_ms * 1e3, 2),
        "algorithmic_bytes_per_step": int(step_bytes),
        "seq_steps_per_s": round(x.cfg.num_seqs / (ms_step * 1e-3), 1),
        "context_tokens_per_s": round(float(x.seq_lens.sum()) / (ms_step * 1e-3), 1),
        "wall_s_timed_region_incl_scrub": round(wall, 4),
        "kernels_us_mean": {"pa_partition": round(k1_ms * 1e3, 2), "pa_lse_reduce": round(k2_ms * 1e3, 2),
                            "pa_partition_p10_p50_p90": [round(float(np.percentile(k1, q_)) * 1e3, 2)
                                                         for q_ in (10, 50, 90)],
                            "method": "HIP events recorded at the start/end of each kernel's own dispatch "
                                      "(pa_*_timed), on the launch stream, scrubbed steps"},
        "roofline": {
            "bound": "hbm",
            "achieved": round(achieved, 2),
            "peak": PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / PEAK_GBS, 4),
            "traffic": traffic_for(num) if ps == 512 else None,
            "kernel": "pa_partition",
            "algorithmic_bytes_per_launch": int(pk_bytes),
        },
        "kernel_source_sha256_16": kernel_source_hash(),
    }
    if cpu_budget > 0:
        log(f"[bench] config {num}: timing the fp64 oracle (~{cpu_budget:.0f}s budget)")
        res["cpu_baseline"] = cpu_baseline(x, out, cpu_budget)
    else:
        res["cpu_baseline"] = None
    del scrub_buf
    return res


def bench_floors(num: int, steps: int, dev) -> dict:
    """Floors of the decode step on this GPU, on the workload's own buffers:
    an empty launch, event pairs around nothing, and a read-only pass over
    exactly the decode's K/V bytes in its block order, beside the decode's
    partition kernel, its reduce kernel and the whole step. Every figure is
    the median over `steps` repetitions, each after a 1 GiB read scrub."""
    import torch

    import oracle
    import paged_attention_decode_06_amd as pa
    from paged_attention_decode_06_amd import workloads as W

    x = W.make_inputs(num)
    d = W.to_device(x, dev)
    q, kc, vc, bt, sl = d["q"], d["k_cache"], d["v_cache"], d["block_tables"], d["seq_lens"]
    out = torch.empty_like(q)
    sh = pa.make_shape(q, kc, bt)
    es, ml, to = pa.alloc_partials(sh, dev)
    elem = 4 if x.cfg.dtype == "f32" else 2
    kv_bytes = 2 * int(x.seq_lens.astype(np.int64).sum()) * x.cfg.num_kv_heads * x.cfg.head_dim * elem
    # the decode's block order: every sequence's gather list, concatenated (each at every KV head)
    ids_host = np.concatenate([np.asarray(b, dtype=np.int32) for b in oracle.gather_list(x.block_tables, x.seq_lens)])
    ids = torch.from_numpy(ids_host).to(dev)
    scrub_buf = torch.empty(SCRUB_BYTES // 4, dtype=torch.float32, device=dev)
    sink1 = torch.empty((), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)
    hev = pa.HipEvents(pa.HipEvents.DISABLE_SYSTEM_FENCE)

    def median_us(fn, attached: bool, scrub=True):
        ts = []
        for i in range(steps + 3):
            if scrub:
                torch.sum(scrub_buf, dim=None, out=sink1)
            a, b = hev.new(), hev.new()
            if attached:
                fn(a, b)
            else:
                hev.record(a, stream)
                fn(None, None)
                hev.record(b, stream)
            torch.cuda.synchronize(dev)
            if i >= 3:
                ts.append(hev.ms(a, b) * 1e3)
        return round(float(np.median(ts)), 2)

    res = {"metric": "decode-step floors on this GPU (us, medians)", "config": workload_label(x),
           "kv_bytes": kv_bytes, "steps": steps}
    res["two_timing_only_events_nothing_between"] = median_us(lambda a, b: None, False)
    res["empty_kernel_between_events"] = median_us(lambda a, b: pa.pa_probe_empty(stream=stream), False)
    res["empty_kernel_attached_events"] = median_us(lambda a, b: pa.pa_probe_empty(a, b, stream=stream), True)
    reads = {}
    for per in (2, 4, 8, 16, 32):
        grid = pa.probe_read_grid(ids.numel(), x.cfg.num_kv_heads, per)
        sink = torch.empty((grid,), dtype=torch.int32, device=dev)
        t = median_us(lambda a, b: pa.pa_probe_paged_read(kc, vc, ids, per, sink, a, b, stream=stream), True)
        reads[f"blocks_per_workgroup_{per}"] = {"workgroups": grid, "us_attached": t,
                                                "GB_s": round(kv_bytes / (t * 1e-6) / 1e9, 1)}
    res["paged_read_probe"] = reads
    best = min(v["us_attached"] for v in reads.values())
    res["paged_read_floor_us_attached"] = best
    part = lambda a, b: pa.pa_decode_partitions_timed(out, q, kc, vc, bt, sl, x.scale, es, ml, to, pa.MODE_AUTO,
                                                      a, b, stream=stream)
    res["partition_kernel_attached"] = median_us(part, True)
    red = lambda a, b: pa.pa_lse_reduce_timed(out, es, ml, to, sl, sh, pa.MODE_AUTO, a, b, stream=stream)
    res["reduce_kernel_attached"] = median_us(red, True)
    res["step_between_events"] = median_us(
        lambda a, b: pa.pa_decode(out, q, kc, vc, bt, sl, x.scale, es, ml, to, stream=stream), False)
    res["partition_kernel_between_events"] = median_us(
        lambda a, b: pa.pa_decode_partitions(out, q, kc, vc, bt, sl, x.scale, es, ml, to, pa.MODE_AUTO,
                                             stream=stream), False)
    best_per = min((2, 4, 8, 16, 32), key=lambda p_: reads[f"blocks_per_workgroup_{p_}"]["us_attached"])
    best_sink = torch.empty((pa.probe_read_grid(ids.numel(), x.cfg.num_kv_heads, best_per),), dtype=torch.int32,
                            device=dev)
    res["paged_read_best_between_events"] = median_us(
        lambda a, b: pa.pa_probe_paged_read(kc, vc, ids, best_per, best_sink, stream=stream), False)
    hev.close()
    del scrub_buf
    return res


PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16/fp16 MFMA


def prefill_cpu_baseline(x, out, budget_s: float) -> dict:
    """The fp64 oracle on sampled chunk tokens of the same workload (TFLOP/s of the same flop count)."""
    import oracle
    from paged_attention_decode_06_amd import workloads as W
    got = W.from_device(out)
    lists = oracle.gather_list(x.block_tables, x.seq_lens)
    rng = np.random.default_rng(0)
    order = rng.permutation(x.num_query_tokens)
    qsl = x.query_start_loc
    flops = 0
    worst = 0.0
    done = 0
    t0 = time.perf_counter()
    for r in order:
        s = int(np.searchsorted(qsl, r, side="right") - 1)
        pos = int(x.seq_lens[s]) - int(x.query_lens[s]) + int(r - qsl[s])
        ref = oracle.attend_prefill_row(x.q[r], x.k_cache, x.v_cache, lists[s], pos, x.scale, x.cfg.dtype)
        worst = max(worst, float(np.abs(got[r] - ref).max()))
        flops += 4 * x.cfg.head_dim * x.cfg.num_heads * max(pos + 1, 0)
        done += 1
        if time.perf_counter() - t0 >= budget_s:
            break
    el = time.perf_counter() - t0
    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:
        cores = os.cpu_count() or 1
    return {"value": round(flops / el / 1e12, 6), "unit": "TFLOP/s", "cores": int(cores), "kind": "oracle",
            "sample": f"fp64 NumPy oracle, one chunk token at a time (all heads), {done} of "
                      f"{x.num_query_tokens} tokens in {el:.1f} s", "seconds": round(el, 3),
            "max_abs_err_vs_gpu": worst}


def bench_prefill(num: int, steps: int, warmup: int, scrub: bool, cpu_budget: float, dev) -> dict:
    """Prefix/chunked prefill over the paged cache: one pa_prefill launch per step."""
    import torch

    import paged_attention_decode_06_amd as pa
    from paged_attention_decode_06_amd import workloads as W

    x = W.make_prefill_inputs(num)
    d = W.prefill_to_device(x, dev)
    out = torch.empty_like(d["q"])
    flops = W.prefill_flops(x.seq_lens, x.query_lens, x.cfg.num_heads, x.cfg.head_dim)
    scrub_buf = torch.empty(SCRUB_BYTES // 4, dtype=torch.float32, device=dev)
    sink = torch.empty((), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)

    def step():
        pa.pa_prefill(out, d["q"], d["k_cache"], d["v_cache"], d["block_tables"], d["seq_lens"],
                      d["query_start_loc"], x.scale, x.max_query_len, stream=stream)

    for _ in range(warmup):
        if scrub:
            torch.sum(scrub_buf, dim=None, out=sink)
        step()
    torch.cuda.synchronize(dev)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for i in range(steps):
        if scrub:
            torch.sum(scrub_buf, dim=None, out=sink)
        ev[i][0].record(stream)
        step()
        ev[i][1].record(stream)
    torch.cuda.synchronize(dev)
    ms = np.array([a.elapsed_time(b) for a, b in ev])
    t = float(ms.mean())
    tf = flops / (t * 1e-3) / 1e12
    c = x.cfg
    res = {
        "metric": "prefix-prefill attention TFLOP/s over the paged cache",
        "value": round(tf, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": steps, "warmup": warmup,
        "ms_per_step": round(t, 5), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": c.dtype, "data": "synthetic",
        "config": {"workload": c.name, "num_seqs": c.num_seqs, "num_heads": c.num_heads,
                   "num_kv_heads": c.num_kv_heads, "head_dim": c.head_dim, "block_size": 16,
                   "query_tokens": x.num_query_tokens, "max_query_len": x.max_query_len,
                   "seq_lens": x.seq_lens.tolist()[:16], "seed": x.seed},
        "us_per_step_p10_p50_p90": [round(float(np.percentile(ms, q_)) * 1e3, 2) for q_ in (10, 50, 90)],
        "flops_per_step": int(flops),
        "tokens_per_s": round(x.num_query_tokens / (t * 1e-3), 1),
        "roofline": {"bound": "mfma", "achieved": round(tf, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(tf / PEAK_BF16_TFLOPS, 4), "traffic": None, "kernel": "pa_prefill",
                     "flops_per_launch": int(flops)},
        "kernel_source_sha256_16": kernel_source_hash([os.path.join(CSRC, "pa_prefill.hip"),
                                                       os.path.join(CSRC, "pa_common.h")]),
    }
    res["cpu_baseline"] = prefill_cpu_baseline(x, out, cpu_budget) if cpu_budget > 0 else None
    del scrub_buf
    return res


def moe_cpu_baseline(x, budget_s: float) -> dict:
    """The oracle's routing steps on the host, over as many tokens as fit the budget."""
    import oracle.moe as om
    from paged_attention_decode_06_amd import workloads as W
    c = x.cfg
    T = c.num_tokens
    y = W.bf16_bits_to_f32(x.y_sorted).astype(np.float64) if c.dtype == "bf16" else x.y_sorted.astype(np.float64)
    t0 = time.perf_counter()
    n = 0
    nbytes = 0
    per = W.moe_bytes(c)
    while True:
        w, ids = om.topk_softmax(x.logits, c.top_k, c.renormalize)
        sp, pp, off = om.sort_by_expert(ids, c.num_experts)
        om.permute_rows(x.x, sp, c.top_k)
        om.combine(y, w, pp)
        n += 1
        nbytes += sum(per.values())
        if time.perf_counter() - t0 >= budget_s:
            break
    el = time.perf_counter() - t0
    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:
        cores = os.cpu_count() or 1
    return {"value": round(nbytes / el / 1e9, 4), "unit": "GB/s", "cores": int(cores), "kind": "oracle",
            "sample": f"NumPy oracle, {n} full routing passes over {T} tokens in {el:.1f} s",
            "seconds": round(el, 3)}


def bench_moe(num: int, steps: int, warmup: int, scrub: bool, cpu_budget: float, dev) -> dict:
    """MoE routing: topk softmax, sort by expert (3 launches), permute, combine per step."""
    import torch

    import paged_attention_decode_06_amd as pa
    from paged_attention_decode_06_amd import workloads as W

    x = W.make_moe_inputs(num)
    c = x.cfg
    T, E, K, Hd = c.num_tokens, c.num_experts, c.top_k, c.hidden
    bf = lambda a: torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)
    logits = torch.from_numpy(x.logits).to(dev)
    xh, ys = bf(x.x), bf(x.y_sorted)
    w = torch.empty((T, K), dtype=torch.float32, device=dev)
    ids = torch.empty((T, K), dtype=torch.int32, device=dev)
    sp = torch.empty((T * K,), dtype=torch.int32, device=dev)
    pp = torch.empty_like(sp)
    off = torch.empty((E + 1,), dtype=torch.int32, device=dev)
    ws = torch.empty((pa.moe_sort_workspace_bytes(T, E, K) // 4,), dtype=torch.int32, device=dev)
    xs = torch.empty((T * K, Hd), dtype=torch.bfloat16, device=dev)
    out = torch.empty((T, Hd), dtype=torch.bfloat16, device=dev)
    stream = torch.cuda.current_stream(dev)
    scrub_buf = torch.empty(SCRUB_BYTES // 4, dtype=torch.float32, device=dev)
    sink = torch.empty((), dtype=torch.float32, device=dev)
    stages = [
        ("topk_softmax", lambda: pa.pa_moe_topk_softmax(w, ids, logits, c.renormalize, stream=stream)),
        ("sort_by_expert", lambda: pa.pa_moe_sort_by_expert(sp, pp, off, ids, E, ws, stream=stream)),
        ("permute", lambda: pa.pa_moe_permute(xs, xh, pp, K, stream=stream)),
        ("combine", lambda: pa.pa_moe_combine(out, ys, w, pp, stream=stream)),
    ]
    for _ in range(warmup):
        for _, f in stages:
            f()
    torch.cuda.synchronize(dev)
    # whole step, events around the four stages
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for i in range(steps):
        if scrub:
            torch.sum(scrub_buf, dim=None, out=sink)
        ev[i][0].record(stream)
        for _, f in stages:
            f()
        ev[i][1].record(stream)
    torch.cuda.synchronize(dev)
    ms = np.array([a.elapsed_time(b) for a, b in ev])
    # per stage, events around each (markers add a few us per stage)
    per = {name: [] for name, _ in stages}
    for i in range(steps):
        if scrub:
            torch.sum(scrub_buf, dim=None, out=sink)
        marks = []
        for name, f in stages:
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream); f(); b.record(stream)
            marks.append((name, a, b))
        torch.cuda.synchronize(dev)
        for name, a, b in marks:
            per[name].append(a.elapsed_time(b))
    per_us = {k: round(float(np.mean(v)) * 1e3, 2) for k, v in per.items()}
    nbytes = W.moe_bytes(c)
    t = float(ms.mean())
    total = sum(nbytes.values())
    gbs = total / (t * 1e-3) / 1e9
    dom = max(per_us, key=per_us.get)      # the dominant stage carries the roofline
    pk = nbytes[dom] / (per_us[dom] * 1e-6) / 1e9
    res = {
        "metric": "MoE routing path (topk softmax, sort by expert, permute, combine) achieved HBM GB/s",
        "value": round(gbs, 2), "unit": "GB/s", "n_gpus": 1, "steps": steps, "warmup": warmup,
        "ms_per_step": round(t, 5), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": c.dtype, "data": "synthetic",
        "config": {"workload": c.name, "num_tokens": T, "num_experts": E, "top_k": K, "hidden": Hd,
                   "renormalize": c.renormalize, "seed": x.seed,
                   "note": "expert GEMMs not included; y_sorted is a seeded stand-in for their outputs"},
        "us_per_step_p10_p50_p90": [round(float(np.percentile(ms, q_)) * 1e3, 2) for q_ in (10, 50, 90)],
        "stage_us_mean": per_us,
        "algorithmic_bytes": nbytes,
        "tokens_per_s": round(T / (t * 1e-3), 1),
        "kernel_source_sha256_16": kernel_source_hash([os.path.join(CSRC, "pa_moe.hip")]),
        "roofline": {"bound": "hbm", "achieved": round(pk, 2), "peak": PEAK_GBS, "unit": "GB/s",
                     "frac": round(pk / PEAK_GBS, 4), "traffic": moe_traffic_for(num, dom), "kernel": "pa_moe_" + dom,
                     "algorithmic_bytes_per_launch": int(nbytes[dom])},
    }
    res["cpu_baseline"] = moe_cpu_baseline(x, cpu_budget) if cpu_budget > 0 else None
    del scrub_buf
    return res


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", type=int, default=3,
                    help="workload number 1..6 (default 3: 100K context, bf16; 6: the same with fp16)")
    ap.add_argument("--all", action="store_true", help="every workload, one JSON line each")
    ap.add_argument("--no-scrub", action="store_true", help="skip the cache scrub (warm-cache timing)")
    ap.add_argument("--cpu-budget", type=float, default=12.0, help="seconds of oracle timing (0 = skip)")
    ap.add_argument("--cold-only", action="store_true", help="only warmup + timed scrubbed steps (profiler runs)")
    ap.add_argument("--partition-size", type=int, default=512, choices=(256, 512),
                    help="V2 partition size (512, the default; 256 is the opt-in alternative)")
    ap.add_argument("--prefill", type=int, default=0, metavar="N",
                    help="measure prefix/chunked-prefill workload N (1..4; 0 = decode); --all-prefill for all")
    ap.add_argument("--all-prefill", action="store_true", help="every prefill workload, one JSON line each")
    ap.add_argument("--moe", type=int, default=0, metavar="N",
                    help="measure MoE routing workload N (1: 16384 tokens, 2: 256 tokens); --all-moe for both")
    ap.add_argument("--all-moe", action="store_true", help="every MoE routing workload, one JSON line each")
    ap.add_argument("--floors", action="store_true",
                    help="measure the step's floors on this GPU (empty launch, event pairs, read-only pass)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="run a plain device copy of MIB MiB (counter calibration) and exit")
    args = ap.parse_args(argv)

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the decode path runs on a single MI355X and has no "
              "multi-GPU mode (across GPUs it would shard by sequence, or by KV head, each GPU running "
              "the same kernels on its share). Run with --gpus 1.",
              file=sys.stderr)
        return 2

    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1
    dev = torch.device("cuda:0")
    if args.copy_calibration:
        n = args.copy_calibration << 20
        src = torch.ones(n // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize(dev)
        print(json.dumps({"copy_calibration_bytes": n, "copies": 3}), flush=True)
        return 0
    import paged_attention_decode_06_amd as pa
    pa.load()
    if args.moe or args.all_moe:
        for n in ([1, 2] if args.all_moe else [args.moe]):
            res = bench_moe(n, args.steps, args.warmup, not args.no_scrub, args.cpu_budget, dev)
            print(json.dumps(res), flush=True)
        return 0
    if args.prefill or args.all_prefill:
        for n in ([1, 2, 3, 4] if args.all_prefill else [args.prefill]):
            res = bench_prefill(n, args.steps, args.warmup, not args.no_scrub, args.cpu_budget, dev)
            print(json.dumps(res), flush=True)
        return 0
    if args.floors:
        for n in ([1, 2, 3, 4, 5] if args.all else [args.config]):
            print(json.dumps(bench_floors(n, args.steps, dev)), flush=True)
        return 0
    nums = [1, 2, 3, 4, 5] if args.all else [args.config]
    for n in nums:
        res = bench_one(n, args.steps, args.warmup, not args.no_scrub, args.cpu_budget, dev, args.cold_only,
                        args.partition_size)
        print(json.dumps(res), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
