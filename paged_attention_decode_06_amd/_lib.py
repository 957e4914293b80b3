"""ctypes binding of libpa_decode.so (argument marshalling only).

Every compute step runs in the HIP library; this module only turns torch
tensors into pointers, sizes and the current HIP stream. It never falls back
to another implementation: a missing library is an error.
"""
from __future__ import annotations

import ctypes
import os
import re

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libpa_decode.so")
HEADER = os.path.join(os.path.dirname(HERE), "include", "pa_decode.h")
HEADERS = [HEADER, os.path.join(os.path.dirname(HERE), "include", "pa_moe.h"),
           os.path.join(os.path.dirname(HERE), "include", "pa_probe.h")]

PA_F32, PA_BF16, PA_F16 = 0, 1, 2
MODE_AUTO, MODE_V1, MODE_V2 = 0, 1, 2
PA_OK, PA_EINVAL, PA_EUNSUPPORTED, PA_EALIGN, PA_EHIP, PA_ESCRATCH = 0, -1, -2, -3, -4, -5
NOALLOC_SCRATCH_BYTES = 64 << 20
BLOCK_SIZE, PARTITION_SIZE, V2_THRESHOLD = 16, 512, 8192


class PaShape(ctypes.Structure):
    _fields_ = [
        ("num_seqs", ctypes.c_int32),
        ("num_heads", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("block_size", ctypes.c_int32),
        ("max_blocks_per_seq", ctypes.c_int32),
        ("num_blocks", ctypes.c_int64),
        ("dtype", ctypes.c_int32),
        ("partition_size", ctypes.c_int32),
    ]


class PaError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: status {status} ({status_string(status)})")


_lib = None

_P = ctypes.c_void_p
_SIGS = {
    "pa_decode_v1": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, ctypes.POINTER(PaShape), ctypes.c_float, _P]),
    "pa_decode_v2": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, ctypes.POINTER(PaShape), ctypes.c_float, _P, _P, _P, _P]),
    "pa_decode": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, ctypes.POINTER(PaShape), ctypes.c_float, _P, _P, _P, _P]),
    "pa_decode_noalloc": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, ctypes.POINTER(PaShape), ctypes.c_float, _P]),
    "pa_decode_partitions": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, ctypes.POINTER(PaShape), ctypes.c_float,
                                            _P, _P, _P, ctypes.c_int, _P]),
    "pa_lse_reduce": (ctypes.c_int, [_P, _P, _P, _P, _P, ctypes.POINTER(PaShape), ctypes.c_int, _P]),
    "pa_decode_partitions_debug": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, ctypes.POINTER(PaShape), ctypes.c_float,
                                                  _P, _P, _P, ctypes.c_int, _P, _P, _P]),
    "pa_decode_partitions_timed": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, ctypes.POINTER(PaShape), ctypes.c_float,
                                                  _P, _P, _P, ctypes.c_int, _P, _P, _P]),
    "pa_lse_reduce_timed": (ctypes.c_int, [_P, _P, _P, _P, _P, ctypes.POINTER(PaShape), ctypes.c_int, _P, _P, _P]),
    "pa_prefill": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, _P, ctypes.POINTER(PaShape), ctypes.c_int32,
                                  ctypes.c_int32, ctypes.c_float, _P]),
    "pa_max_partitions": (ctypes.c_int64, [ctypes.POINTER(PaShape)]),
    "pa_moe_topk_softmax": (ctypes.c_int, [_P, _P, _P, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                           ctypes.c_int, _P]),
    "pa_moe_sort_workspace_bytes": (ctypes.c_int64, [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32]),
    "pa_moe_sort_by_expert": (ctypes.c_int, [_P, _P, _P, _P, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, _P,
                                             ctypes.c_int64, _P]),
    "pa_moe_permute": (ctypes.c_int, [_P, _P, _P, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                      _P]),
    "pa_moe_combine": (ctypes.c_int, [_P, _P, _P, _P, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                      ctypes.c_int32, _P]),
    "pa_partials_elems": (ctypes.c_int64, [ctypes.POINTER(PaShape), ctypes.c_int]),
    "pa_probe_empty": (ctypes.c_int, [_P, _P, _P]),
    "pa_probe_paged_read": (ctypes.c_int, [_P, _P, _P, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                           ctypes.c_int64, ctypes.c_int32, _P, ctypes.c_int64, _P, _P, _P]),
    "pa_probe_paged_read_grid": (ctypes.c_int64, [ctypes.c_int64, ctypes.c_int32, ctypes.c_int32]),
    "pa_check_args": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, ctypes.POINTER(PaShape), _P, _P, _P, ctypes.c_int]),
    "pa_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "pa_version": (ctypes.c_int, []),
}


def header_functions(paths=None) -> list[str]:
    """Names of the functions the library's headers (include/*.h) declare."""
    names = set()
    for path in (paths or HEADERS):
        text = open(path).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        names.update(re.findall(r"\b(pa_[a-z0-9_]+)\s*\(", text))
    return sorted(names)


def _hip_runtimes() -> list[str]:
    """Paths of the HIP runtime libraries mapped into this process (Linux)."""
    try:
        with open("/proc/self/maps") as f:
            paths = {line.split()[-1] for line in f if "libamdhip64" in line}
    except OSError:
        return []
    return sorted({os.path.realpath(x) for x in paths})


def load(path: str | None = None) -> ctypes.CDLL:
    """Load the HIP library (once). Raises if it has not been built."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or os.environ.get("PA_DECODE_LIB", LIB_PATH)
    if not os.path.exists(p):
        raise RuntimeError(f"{p} is missing: build it first with "
                           "`python -c 'import __graft_entry__ as g; g.build()'` "
                           "or `python -m paged_attention_decode_06_amd._build`")
    # torch ships its own HIP runtime. Loaded first, it is the one the library
    # binds to; loaded after the library, the process would map two runtimes,
    # and torch's streams and allocations would be handed to the other one
    # (every launch then fails).
    import torch  # noqa: F401
    lib = ctypes.CDLL(p)
    runtimes = _hip_runtimes()
    if len(runtimes) > 1:
        raise RuntimeError("more than one HIP runtime is mapped in this process "
                           f"({', '.join(runtimes)}): import torch before loading {p}")
    for name, (res, args) in _SIGS.items():
        fn = getattr(lib, name)
        fn.restype, fn.argtypes = res, args
    if path is None:
        _lib = lib
    return lib


def status_string(status: int) -> str:
    return load().pa_status_string(int(status)).decode()


def _dtype_code(dt) -> int:
    import torch
    if dt == torch.float32:
        return PA_F32
    if dt == torch.bfloat16:
        return PA_BF16
    if dt == torch.float16:
        return PA_F16
    raise PaError(PA_EUNSUPPORTED, f"dtype {dt}")


def make_shape(q, k_cache, block_tables, partition_size: int = 0) -> PaShape:
    """pa_shape from q [S, H, D], k_cache [NB, Hkv, 16, D], block_tables [S, MB].

    partition_size 0 means the default (512 tokens); 256 opts into the smaller
    partitions."""
    S, H, D = q.shape
    NB, Hkv, BS, D2 = k_cache.shape
    if D2 != D:
        raise PaError(PA_EINVAL, f"head_dim of q ({D}) and cache ({D2}) differ")
    if block_tables.dim() != 2 or block_tables.shape[0] != S:
        raise PaError(PA_EINVAL, "block_tables must be [num_seqs, max_blocks_per_seq]")
    return PaShape(S, H, Hkv, D, BS, block_tables.shape[1], NB, _dtype_code(q.dtype), int(partition_size))


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream, device):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return ctypes.c_void_p(int(getattr(stream, "cuda_stream", stream)))


def _check_tensors(out, q, k_cache, v_cache, block_tables, seq_lens, partials=()):
    import torch
    ts = [t for t in (out, q, k_cache, v_cache, block_tables, seq_lens, *partials) if t is not None]
    for t in ts:
        if not t.is_cuda:
            raise PaError(PA_EINVAL, "all tensors must be on the GPU")
        if not t.is_contiguous():
            raise PaError(PA_EINVAL, "all tensors must be contiguous")
    if q is not None:
        for t in (out, k_cache, v_cache):
            if t.dtype != q.dtype:
                raise PaError(PA_EINVAL, "q, caches and out must share one dtype")
        if tuple(out.shape) != tuple(q.shape):
            raise PaError(PA_EINVAL, "out must have q's shape")
        if tuple(v_cache.shape) != tuple(k_cache.shape):
            raise PaError(PA_EINVAL, "k_cache and v_cache shapes differ")
    for t in (block_tables, seq_lens):
        if t is not None and t.dtype != torch.int32:
            raise PaError(PA_EINVAL, "block_tables and seq_lens must be int32")
    for t in partials:
        if t is not None and t.dtype != torch.float32:
            raise PaError(PA_EINVAL, "partial buffers must be float32")


def check_sizes(shape: PaShape, out=None, seq_lens=None, partials=None, q=None, k_cache=None) -> None:
    """Element counts of the decode buffers against `shape`, before any launch.

    seq_lens must hold num_seqs entries, out (and q) num_seqs * num_heads *
    head_dim, the caches [num_blocks, num_kv_heads, 16, head_dim], and the
    partial buffers (exp_sums, max_logits, tmp_out) num_seqs * num_heads *
    Pmax (* head_dim) with Pmax the partition count of this very shape (its
    partition size included). Raises PaError(PA_EINVAL) on a mismatch, which
    would otherwise let a kernel write past the end of a buffer."""
    S, H, D = int(shape.num_seqs), int(shape.num_heads), int(shape.head_dim)
    if seq_lens is not None and seq_lens.numel() != S:
        raise PaError(PA_EINVAL, f"seq_lens holds {seq_lens.numel()} entries for {S} sequences")
    for name, t in (("out", out), ("q", q)):
        if t is not None and t.numel() != S * H * D:
            raise PaError(PA_EINVAL, f"{name} holds {t.numel()} elements, the shape needs {S * H * D}")
    if k_cache is not None and tuple(k_cache.shape) != (int(shape.num_blocks), int(shape.num_kv_heads),
                                                        int(shape.block_size), D):
        raise PaError(PA_EINVAL, f"cache shape {tuple(k_cache.shape)} does not match the shape")
    if partials is not None:
        P = (int(shape.max_blocks_per_seq) * int(shape.block_size) + _psize(shape) - 1) // _psize(shape)
        es, ml, to = partials
        for name, t, n in (("exp_sums", es, S * H * P), ("max_logits", ml, S * H * P),
                           ("tmp_out", to, S * H * P * D)):
            if t is not None and t.numel() != n:
                raise PaError(PA_EINVAL, f"{name} holds {t.numel()} elements, the shape needs {n} "
                                         f"({P} partitions of {_psize(shape)} tokens)")


def _psize(shape: PaShape) -> int:
    return int(shape.partition_size) if int(shape.partition_size) else PARTITION_SIZE


def _call(name, rc):
    if rc != PA_OK:
        raise PaError(rc, name)


def max_partitions(shape: PaShape) -> int:
    r = load().pa_max_partitions(ctypes.byref(shape))
    _call("pa_max_partitions", r if r < 0 else 0)
    return int(r)


def alloc_partials(shape: PaShape, device):
    """(exp_sums, max_logits, tmp_out) float32 buffers sized for `shape`."""
    import torch
    P = max_partitions(shape)
    S, H, D = shape.num_seqs, shape.num_heads, shape.head_dim
    return (torch.empty((S, H, P), dtype=torch.float32, device=device),
            torch.empty((S, H, P), dtype=torch.float32, device=device),
            torch.empty((S, H, P, D), dtype=torch.float32, device=device))


def pa_decode_v1(out, q, k_cache, v_cache, block_tables, seq_lens, scale, stream=None):
    _check_tensors(out, q, k_cache, v_cache, block_tables, seq_lens)
    sh = make_shape(q, k_cache, block_tables)
    check_sizes(sh, out=out, seq_lens=seq_lens, q=q, k_cache=k_cache)
    _call("pa_decode_v1", load().pa_decode_v1(_ptr(out), _ptr(q), _ptr(k_cache), _ptr(v_cache),
                                              _ptr(block_tables), _ptr(seq_lens), ctypes.byref(sh),
                                              float(scale), _stream(stream, q.device)))


def _full(name, out, q, k_cache, v_cache, block_tables, seq_lens, scale, exp_sums, max_logits, tmp_out, stream,
          partition_size):
    _check_tensors(out, q, k_cache, v_cache, block_tables, seq_lens, (exp_sums, max_logits, tmp_out))
    sh = make_shape(q, k_cache, block_tables, partition_size)
    check_sizes(sh, out=out, seq_lens=seq_lens, partials=(exp_sums, max_logits, tmp_out), q=q, k_cache=k_cache)
    fn = getattr(load(), name)
    _call(name, fn(_ptr(out), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_tables), _ptr(seq_lens),
                   ctypes.byref(sh), float(scale), _ptr(exp_sums), _ptr(max_logits), _ptr(tmp_out),
                   _stream(stream, q.device)))


def pa_decode_v2(out, q, k_cache, v_cache, block_tables, seq_lens, scale, exp_sums, max_logits, tmp_out,
                 stream=None, partition_size=0):
    _full("pa_decode_v2", out, q, k_cache, v_cache, block_tables, seq_lens, scale, exp_sums, max_logits,
          tmp_out, stream, partition_size)


def pa_decode(out, q, k_cache, v_cache, block_tables, seq_lens, scale, exp_sums, max_logits, tmp_out,
              stream=None, partition_size=0):
    _full("pa_decode", out, q, k_cache, v_cache, block_tables, seq_lens, scale, exp_sums, max_logits,
          tmp_out, stream, partition_size)


def pa_decode_noalloc(out, q, k_cache, v_cache, block_tables, seq_lens, scale, stream=None):
    """pa_decode with the partials in the library's own device scratch: no
    buffer is allocated, here or in the library (PaError PA_ESCRATCH when a
    shape's partials exceed it). Calls that overlap on one GPU race."""
    _check_tensors(out, q, k_cache, v_cache, block_tables, seq_lens)
    sh = make_shape(q, k_cache, block_tables)
    check_sizes(sh, out=out, seq_lens=seq_lens, q=q, k_cache=k_cache)
    _call("pa_decode_noalloc", load().pa_decode_noalloc(_ptr(out), _ptr(q), _ptr(k_cache), _ptr(v_cache),
                                                        _ptr(block_tables), _ptr(seq_lens), ctypes.byref(sh),
                                                        float(scale), _stream(stream, q.device)))


def pa_decode_partitions(out, q, k_cache, v_cache, block_tables, seq_lens, scale, exp_sums, max_logits,
                         tmp_out, mode, stream=None, partition_size=0):
    _check_tensors(out, q, k_cache, v_cache, block_tables, seq_lens, (exp_sums, max_logits, tmp_out))
    sh = make_shape(q, k_cache, block_tables, partition_size)
    check_sizes(sh, out=out, seq_lens=seq_lens, partials=(exp_sums, max_logits, tmp_out), q=q, k_cache=k_cache)
    _call("pa_decode_partitions", load().pa_decode_partitions(
        _ptr(out), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_tables), _ptr(seq_lens),
        ctypes.byref(sh), float(scale), _ptr(exp_sums), _ptr(max_logits), _ptr(tmp_out), int(mode),
        _stream(stream, q.device)))


def pa_decode_partitions_debug(out, q, k_cache, v_cache, block_tables, seq_lens, scale, exp_sums, max_logits,
                               tmp_out, mode, gather_trace=None, err_flag=None, stream=None, partition_size=0):
    _check_tensors(out, q, k_cache, v_cache, block_tables, seq_lens, (exp_sums, max_logits, tmp_out))
    sh = make_shape(q, k_cache, block_tables, partition_size)
    check_sizes(sh, out=out, seq_lens=seq_lens, partials=(exp_sums, max_logits, tmp_out), q=q, k_cache=k_cache)
    _call("pa_decode_partitions_debug", load().pa_decode_partitions_debug(
        _ptr(out), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_tables), _ptr(seq_lens),
        ctypes.byref(sh), float(scale), _ptr(exp_sums), _ptr(max_logits), _ptr(tmp_out), int(mode),
        _ptr(gather_trace), _ptr(err_flag), _stream(stream, q.device)))


def pa_lse_reduce(out, exp_sums, max_logits, tmp_out, seq_lens, shape: PaShape, mode=MODE_V2, stream=None):
    _check_tensors(out, None, None, None, None, seq_lens, (exp_sums, max_logits, tmp_out))
    check_sizes(shape, out=out, seq_lens=seq_lens, partials=(exp_sums, max_logits, tmp_out))
    _call("pa_lse_reduce", load().pa_lse_reduce(_ptr(out), _ptr(exp_sums), _ptr(max_logits), _ptr(tmp_out),
                                                _ptr(seq_lens), ctypes.byref(shape), int(mode),
                                                _stream(stream, out.device)))


def pa_decode_partitions_timed(out, q, k_cache, v_cache, block_tables, seq_lens, scale, exp_sums, max_logits,
                               tmp_out, mode, start_event, stop_event, stream=None, partition_size=0):
    """Phase 1 with raw hipEvent_t handles (ints) recorded around the kernel itself."""
    _check_tensors(out, q, k_cache, v_cache, block_tables, seq_lens, (exp_sums, max_logits, tmp_out))
    sh = make_shape(q, k_cache, block_tables, partition_size)
    check_sizes(sh, out=out, seq_lens=seq_lens, partials=(exp_sums, max_logits, tmp_out), q=q, k_cache=k_cache)
    _call("pa_decode_partitions_timed", load().pa_decode_partitions_timed(
        _ptr(out), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_tables), _ptr(seq_lens),
        ctypes.byref(sh), float(scale), _ptr(exp_sums), _ptr(max_logits), _ptr(tmp_out), int(mode),
        ctypes.c_void_p(start_event), ctypes.c_void_p(stop_event), _stream(stream, q.device)))


def pa_lse_reduce_timed(out, exp_sums, max_logits, tmp_out, seq_lens, shape: PaShape, mode, start_event,
                        stop_event, stream=None):
    """Phase 2 with raw hipEvent_t handles (ints) recorded around the kernel itself."""
    _check_tensors(out, None, None, None, None, seq_lens, (exp_sums, max_logits, tmp_out))
    check_sizes(shape, out=out, seq_lens=seq_lens, partials=(exp_sums, max_logits, tmp_out))
    _call("pa_lse_reduce_timed", load().pa_lse_reduce_timed(
        _ptr(out), _ptr(exp_sums), _ptr(max_logits), _ptr(tmp_out), _ptr(seq_lens), ctypes.byref(shape),
        int(mode), ctypes.c_void_p(start_event), ctypes.c_void_p(stop_event), _stream(stream, out.device)))


def pa_prefill(out, q, k_cache, v_cache, block_tables, seq_lens, query_start_loc, scale, max_query_len,
               stream=None):
    """Prefix/chunked prefill over the paged cache: q, out [T, H, D] packed by token."""
    _check_tensors(out, q, k_cache, v_cache, block_tables, seq_lens)
    import torch
    if not query_start_loc.is_cuda or query_start_loc.dtype != torch.int32 or not query_start_loc.is_contiguous():
        raise PaError(PA_EINVAL, "query_start_loc must be a contiguous int32 GPU tensor")
    if query_start_loc.numel() != block_tables.shape[0] + 1:
        raise PaError(PA_EINVAL, "query_start_loc must hold num_seqs + 1 entries")
    T, H, D = q.shape
    NB, Hkv, BS, D2 = k_cache.shape
    if D2 != D:
        raise PaError(PA_EINVAL, f"head_dim of q ({D}) and cache ({D2}) differ")
    sh = PaShape(block_tables.shape[0], H, Hkv, D, BS, block_tables.shape[1], NB, _dtype_code(q.dtype), 0)
    _call("pa_prefill", load().pa_prefill(
        _ptr(out), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_tables), _ptr(seq_lens),
        _ptr(query_start_loc), ctypes.byref(sh), int(T), int(max_query_len), float(scale),
        _stream(stream, q.device)))


# ---------------------------------------------------------------- MoE routing
def _gpu_contig(*ts):
    for t in ts:
        if not t.is_cuda or not t.is_contiguous():
            raise PaError(PA_EINVAL, "MoE tensors must be contiguous GPU tensors")


def pa_moe_topk_softmax(topk_weights, topk_ids, logits, renormalize=True, stream=None):
    """logits float32 [T, E] -> topk_weights float32 [T, K], topk_ids int32 [T, K]."""
    import torch
    _gpu_contig(topk_weights, topk_ids, logits)
    if logits.dtype != torch.float32 or topk_weights.dtype != torch.float32 or topk_ids.dtype != torch.int32:
        raise PaError(PA_EINVAL, "logits/weights float32, ids int32")
    T, E = logits.shape
    K = topk_ids.shape[1]
    if tuple(topk_weights.shape) != (T, K) or topk_ids.shape[0] != T:
        raise PaError(PA_EINVAL, "weights and ids must be [T, K]")
    _call("pa_moe_topk_softmax", load().pa_moe_topk_softmax(
        _ptr(topk_weights), _ptr(topk_ids), _ptr(logits), T, E, K, int(bool(renormalize)),
        _stream(stream, logits.device)))


def moe_sort_workspace_bytes(T: int, E: int, K: int) -> int:
    r = int(load().pa_moe_sort_workspace_bytes(T, E, K))
    _call("pa_moe_sort_workspace_bytes", r if r < 0 else 0)
    return r


def pa_moe_sort_by_expert(sorted_pairs, pair_pos, expert_offsets, topk_ids, num_experts, workspace, stream=None):
    """topk_ids int32 [T, K] -> sorted_pairs, pair_pos int32 [T*K], expert_offsets int32 [E+1]."""
    import torch
    _gpu_contig(sorted_pairs, pair_pos, expert_offsets, topk_ids, workspace)
    for t in (sorted_pairs, pair_pos, expert_offsets, topk_ids):
        if t.dtype != torch.int32:
            raise PaError(PA_EINVAL, "sort arrays must be int32")
    T, K = topk_ids.shape
    if sorted_pairs.numel() != T * K or pair_pos.numel() != T * K or expert_offsets.numel() != num_experts + 1:
        raise PaError(PA_EINVAL, "sorted_pairs/pair_pos need T*K entries, expert_offsets E+1")
    nbytes = workspace.numel() * workspace.element_size()
    _call("pa_moe_sort_by_expert", load().pa_moe_sort_by_expert(
        _ptr(sorted_pairs), _ptr(pair_pos), _ptr(expert_offsets), _ptr(topk_ids), T, int(num_experts), K,
        _ptr(workspace), int(nbytes), _stream(stream, topk_ids.device)))


def pa_moe_permute(x_sorted, x, pair_pos, top_k, stream=None):
    """x [T, hidden] -> x_sorted [T*K, hidden]: row pair_pos[t*K + j] = x[t]."""
    _gpu_contig(x_sorted, x, pair_pos)
    T, Hd = x.shape
    if tuple(x_sorted.shape) != (T * top_k, Hd) or x_sorted.dtype != x.dtype or pair_pos.numel() != T * top_k:
        raise PaError(PA_EINVAL, "x_sorted must be [T*K, hidden] of x's dtype; pair_pos T*K entries")
    _call("pa_moe_permute", load().pa_moe_permute(_ptr(x_sorted), _ptr(x), _ptr(pair_pos), T, int(top_k), Hd,
                                                  _dtype_code(x.dtype), _stream(stream, x.device)))


def pa_moe_combine(out, y_sorted, topk_weights, pair_pos, stream=None):
    """out[t] = sum_j topk_weights[t, j] * y_sorted[pair_pos[t*K + j]] (fp32 accumulation, order j)."""
    _gpu_contig(out, y_sorted, topk_weights, pair_pos)
    T, K = topk_weights.shape
    Hd = out.shape[1]
    if tuple(y_sorted.shape) != (T * K, Hd) or y_sorted.dtype != out.dtype or pair_pos.numel() != T * K:
        raise PaError(PA_EINVAL, "y_sorted must be [T*K, hidden] of out's dtype; pair_pos T*K entries")
    _call("pa_moe_combine", load().pa_moe_combine(_ptr(out), _ptr(y_sorted), _ptr(topk_weights), _ptr(pair_pos), T, K,
                                                  Hd, _dtype_code(out.dtype), _stream(stream, out.device)))


# ---------------------------------------------------------------- measurement kernels
def pa_probe_empty(start=None, stop=None, stream=None):
    """An empty launch (one wave), optionally with events attached to its dispatch."""
    import torch
    sp = _stream(stream, torch.device("cuda", torch.cuda.current_device()))
    _call("pa_probe_empty", load().pa_probe_empty(ctypes.c_void_p(start), ctypes.c_void_p(stop), sp))


def probe_read_grid(num_ids: int, num_kv_heads: int, units_per_wg: int) -> int:
    r = int(load().pa_probe_paged_read_grid(int(num_ids), int(num_kv_heads), int(units_per_wg)))
    _call("pa_probe_paged_read_grid", r if r < 0 else 0)
    return r


def pa_probe_paged_read(k_cache, v_cache, block_ids, units_per_wg, sink, start=None, stop=None, stream=None):
    """Read-only pass over the K/V bytes of `block_ids` (int32, every KV head), no math."""
    import torch
    _gpu_contig(k_cache, v_cache, block_ids, sink)
    if block_ids.dtype != torch.int32 or sink.dtype != torch.int32:
        raise PaError(PA_EINVAL, "block_ids and sink must be int32")
    NB, Hkv, BS, D = k_cache.shape
    _call("pa_probe_paged_read", load().pa_probe_paged_read(
        _ptr(k_cache), _ptr(v_cache), _ptr(block_ids), int(block_ids.numel()), int(Hkv), int(D),
        int(k_cache.element_size()), int(NB), int(units_per_wg), _ptr(sink), int(sink.numel()),
        ctypes.c_void_p(start), ctypes.c_void_p(stop), _stream(stream, k_cache.device)))


class HipEvents:
    """Raw hipEvent_t handles for the *_timed entry points.

    The handles come from the HIP runtime this process already has mapped (the
    one the library itself is linked against), opened without loading a
    second copy. They are freed by close().
    """

    # hipEventCreateWithFlags: a timing-only event that records without a
    # system-scope cache write-back and invalidate (the HIP runtime documents
    # this flag for precise timing; the decode's results stay on the device).
    DISABLE_SYSTEM_FENCE = 0x20000000

    def __init__(self, flags: int = 0):
        load()  # maps the runtime the library is linked against
        self.ct = ctypes
        self.flags = int(flags)
        self.hip = ctypes.CDLL("libamdhip64.so.7", mode=os.RTLD_NOLOAD | os.RTLD_GLOBAL)
        self.hip.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.made = []

    def new(self) -> int:
        h = self.ct.c_void_p()
        if self.hip.hipEventCreateWithFlags(self.ct.byref(h), self.flags) != 0:
            raise RuntimeError("hipEventCreateWithFlags failed")
        self.made.append(h.value)
        return h.value

    def record(self, event: int, stream) -> None:
        """Record `event` on a torch stream (or a raw hipStream_t int)."""
        sp = getattr(stream, "cuda_stream", stream)
        if self.hip.hipEventRecord(self.ct.c_void_p(event), self.ct.c_void_p(int(sp))) != 0:
            raise RuntimeError("hipEventRecord failed")

    def ms(self, a: int, b: int) -> float:
        out = self.ct.c_float()
        if self.hip.hipEventElapsedTime(self.ct.byref(out), self.ct.c_void_p(a), self.ct.c_void_p(b)) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return float(out.value)

    def close(self):
        for h in self.made:
            self.hip.hipEventDestroy(self.ct.c_void_p(h))
        self.made = []
