"""C-ABI checks that need no GPU: the library loads, exports what the header
declares, and rejects every invalid argument with its documented status
before touching the device."""
import ctypes

import pytest

from paged_attention_decode_06_amd import _lib as L


@pytest.fixture(scope="module")
def lib():
    return L.load()


def shape(**kw):
    base = dict(num_seqs=2, num_heads=16, num_kv_heads=2, head_dim=128, block_size=16,
                max_blocks_per_seq=100, num_blocks=1000, dtype=L.PA_BF16)
    base.update(kw)
    return L.PaShape(**base)


A = 0x10000   # fake, well-aligned device addresses: validation never dereferences them


def check(lib, sh, mode=L.MODE_AUTO, **ptrs):
    p = dict(out=A, q=A, k=A, v=A, bt=A, sl=A, es=A, ml=A, to=A)
    p.update(ptrs)
    c = lambda x: None if x is None else ctypes.c_void_p(x)
    return lib.pa_check_args(c(p["out"]), c(p["q"]), c(p["k"]), c(p["v"]), c(p["bt"]), c(p["sl"]),
                             ctypes.byref(sh), c(p["es"]), c(p["ml"]), c(p["to"]), mode)


def test_exports_every_header_function(lib):
    names = L.header_functions()
    assert len(names) >= 10
    for n in names:
        assert hasattr(lib, n), n
    assert lib.pa_version() == 1


def test_header_constants_match_binding():
    text = open(L.HEADER).read()
    assert "#define PA_PARTITION_SIZE 512" in text
    assert "#define PA_V2_THRESHOLD 8192" in text
    assert "#define PA_BLOCK_SIZE 16" in text


def test_valid_args_pass(lib):
    assert check(lib, shape()) == L.PA_OK
    assert check(lib, shape(dtype=L.PA_F32, head_dim=256, num_heads=2, num_kv_heads=1)) == L.PA_OK
    assert check(lib, shape(dtype=L.PA_F16)) == L.PA_OK
    # single pass needs no partial buffers
    assert check(lib, shape(), L.MODE_V1, es=None, ml=None, to=None) == L.PA_OK


@pytest.mark.parametrize("kw,status", [
    (dict(num_heads=15), L.PA_EINVAL),            # H % Hkv != 0
    (dict(num_heads=0), L.PA_EINVAL),
    (dict(num_kv_heads=0), L.PA_EINVAL),
    (dict(num_seqs=-1), L.PA_EINVAL),
    (dict(max_blocks_per_seq=0), L.PA_EINVAL),
    (dict(num_blocks=0), L.PA_EINVAL),
    (dict(head_dim=64), L.PA_EUNSUPPORTED),
    (dict(head_dim=192), L.PA_EUNSUPPORTED),
    (dict(block_size=32), L.PA_EUNSUPPORTED),
    (dict(dtype=7), L.PA_EUNSUPPORTED),
    (dict(num_heads=34, num_kv_heads=2), L.PA_EUNSUPPORTED),   # G = 17 > 16
    (dict(partition_size=300), L.PA_EUNSUPPORTED),             # only 512 (0) and 256
    (dict(partition_size=128), L.PA_EUNSUPPORTED),
    (dict(partition_size=-512), L.PA_EUNSUPPORTED),
])
def test_bad_shapes(lib, kw, status):
    assert check(lib, shape(**kw)) == status


def test_empty_batch_is_a_noop(lib):
    assert check(lib, shape(num_seqs=0), out=None, q=None, k=None, v=None, bt=None, sl=None,
                 es=None, ml=None, to=None) == L.PA_OK


def test_bad_mode(lib):
    assert check(lib, shape(), 9) == L.PA_EUNSUPPORTED


@pytest.mark.parametrize("name", ["out", "q", "k", "v", "bt", "sl", "es", "ml", "to"])
def test_null_pointers(lib, name):
    assert check(lib, shape(), **{name: None}) == L.PA_EINVAL


@pytest.mark.parametrize("name,addr", [("q", A + 8), ("k", A + 4), ("v", A + 2), ("out", A + 8),
                                       ("to", A + 8), ("bt", A + 2), ("sl", A + 1), ("es", A + 2)])
def test_misaligned(lib, name, addr):
    assert check(lib, shape(), **{name: addr}) == L.PA_EALIGN


def test_grid_limit(lib):
    big = shape(num_seqs=1 << 20, max_blocks_per_seq=1 << 20)
    assert check(lib, big) == L.PA_EUNSUPPORTED


def test_entry_points_reject_before_launch(lib):
    """Every entry point validates first: with a null q nothing reaches HIP."""
    sh = shape()
    n = None
    a = ctypes.c_void_p(A)
    assert lib.pa_decode(a, n, a, a, a, a, ctypes.byref(sh), 1.0, a, a, a, n) == L.PA_EINVAL
    assert lib.pa_decode_v1(a, n, a, a, a, a, ctypes.byref(sh), 1.0, n) == L.PA_EINVAL
    assert lib.pa_decode_v2(a, a, a, a, a, a, ctypes.byref(sh), 1.0, n, a, a, n) == L.PA_EINVAL
    assert lib.pa_decode_partitions(a, n, a, a, a, a, ctypes.byref(sh), 1.0, a, a, a, 0, n) == L.PA_EINVAL
    assert lib.pa_lse_reduce(a, n, a, a, a, ctypes.byref(sh), 2, n) == L.PA_EINVAL
    bad = shape(head_dim=96)
    assert lib.pa_lse_reduce(a, a, a, a, a, ctypes.byref(bad), 2, n) == L.PA_EUNSUPPORTED
    assert lib.pa_decode_partitions_debug(a, a, a, a, a, a, ctypes.byref(sh), 1.0, a, a, a, 0,
                                          ctypes.c_void_p(A + 2), n, n) == L.PA_EALIGN
    assert lib.pa_decode(a, a, a, a, a, a, None, 1.0, a, a, a, n) == L.PA_EINVAL


def test_partition_arithmetic(lib):
    # Pmax = ceil(MB * 16 / 512): 6250 blocks (100000 tokens) -> 196 partitions
    assert lib.pa_max_partitions(ctypes.byref(shape(max_blocks_per_seq=6250))) == 196
    assert lib.pa_max_partitions(ctypes.byref(shape(max_blocks_per_seq=32))) == 1
    assert lib.pa_max_partitions(ctypes.byref(shape(max_blocks_per_seq=33))) == 2
    sh = shape(num_seqs=3, num_heads=16, max_blocks_per_seq=2048, head_dim=256)
    assert lib.pa_partials_elems(ctypes.byref(sh), 0) == 3 * 16 * 64
    assert lib.pa_partials_elems(ctypes.byref(sh), 1) == 3 * 16 * 64 * 256
    assert lib.pa_partials_elems(ctypes.byref(sh), 5) == L.PA_EINVAL
    assert lib.pa_max_partitions(ctypes.byref(shape(head_dim=5))) == L.PA_EUNSUPPORTED


def test_opt_in_partition_size(lib):
    """partition_size 0 is the 512-token default; 256 doubles the partition count."""
    assert check(lib, shape(partition_size=256)) == L.PA_OK
    assert check(lib, shape(partition_size=512)) == L.PA_OK
    for mb, p512, p256 in [(6250, 196, 391), (16, 1, 1), (32, 1, 2), (33, 2, 3), (2048, 64, 128)]:
        assert lib.pa_max_partitions(ctypes.byref(shape(max_blocks_per_seq=mb))) == p512
        assert lib.pa_max_partitions(ctypes.byref(shape(max_blocks_per_seq=mb, partition_size=512))) == p512
        assert lib.pa_max_partitions(ctypes.byref(shape(max_blocks_per_seq=mb, partition_size=256))) == p256
    sh = shape(num_seqs=3, max_blocks_per_seq=2048, head_dim=256, partition_size=256)
    assert lib.pa_partials_elems(ctypes.byref(sh), 1) == 3 * 16 * 128 * 256


def test_shape_struct_layout():
    """The binding's struct matches the header's field order (40 bytes, the
    partition size filling what was tail padding)."""
    assert ctypes.sizeof(L.PaShape) == 40
    assert L.PaShape.num_blocks.offset == 24
    assert L.PaShape.dtype.offset == 32
    assert L.PaShape.partition_size.offset == 36


def test_status_strings(lib):
    for st in (0, -1, -2, -3, -4):
        assert lib.pa_status_string(st)
    assert b"unknown" in lib.pa_status_string(-99)


def test_library_missing_fails_loudly(tmp_path):
    with pytest.raises(RuntimeError, match="missing"):
        L.load(str(tmp_path / "nope.so"))


def test_prefill_validation(lib):
    a = ctypes.c_void_p(A)
    n = None

    def call(sh, T=10, maxq=5, **ptrs):
        p = dict(out=A, q=A, k=A, v=A, bt=A, sl=A, qsl=A)
        p.update(ptrs)
        c = lambda x: None if x is None else ctypes.c_void_p(x)
        # validation fails before any launch, so these fake addresses are never touched
        return lib.pa_prefill(c(p["out"]), c(p["q"]), c(p["k"]), c(p["v"]), c(p["bt"]), c(p["sl"]), c(p["qsl"]),
                              ctypes.byref(sh), T, maxq, ctypes.c_float(1.0), n)

    assert call(shape(dtype=L.PA_F32)) == L.PA_EUNSUPPORTED
    assert call(shape(head_dim=64)) == L.PA_EUNSUPPORTED
    assert call(shape(num_heads=15)) == L.PA_EINVAL
    for name in ("out", "q", "k", "v", "bt", "sl", "qsl"):
        assert call(shape(), **{name: None}) == L.PA_EINVAL, name
    assert call(shape(), q=A + 8) == L.PA_EALIGN
    assert call(shape(), qsl=A + 2) == L.PA_EALIGN
    assert call(shape(), T=-1) == L.PA_EINVAL
    assert call(shape(), maxq=-3) == L.PA_EINVAL
    assert call(shape(num_seqs=1 << 30, num_heads=16, num_kv_heads=16), maxq=1 << 30) == L.PA_EUNSUPPORTED
    # empty work: nothing to read, every pointer may be NULL (nothing is launched on the null stream)
    assert lib.pa_prefill(n, n, n, n, n, n, n, ctypes.byref(shape(num_seqs=0)), 0, 0, ctypes.c_float(1.0), n) == L.PA_OK
    assert a is not None


def test_moe_validation(lib):
    n = None
    a = ctypes.c_void_p(A)
    f = ctypes.c_float
    # top-k softmax: sizes, pointers, alignment
    assert lib.pa_moe_topk_softmax(a, a, a, 10, 2000, 8, 1, n) == L.PA_EUNSUPPORTED      # E > 1024
    assert lib.pa_moe_topk_softmax(a, a, a, 10, 256, 40, 1, n) == L.PA_EUNSUPPORTED      # K > 32
    assert lib.pa_moe_topk_softmax(a, a, a, 10, 4, 8, 1, n) == L.PA_EUNSUPPORTED         # K > E
    assert lib.pa_moe_topk_softmax(a, a, a, -1, 256, 8, 1, n) == L.PA_EINVAL
    assert lib.pa_moe_topk_softmax(n, a, a, 10, 256, 8, 1, n) == L.PA_EINVAL
    assert lib.pa_moe_topk_softmax(a, a, ctypes.c_void_p(A + 2), 10, 256, 8, 1, n) == L.PA_EALIGN
    assert lib.pa_moe_topk_softmax(n, n, n, 0, 256, 8, 1, n) == L.PA_OK                   # T = 0: no-op
    # sort workspace: (chunks * E + pairs + E) int32
    assert lib.pa_moe_sort_workspace_bytes(16384, 256, 8) == (128 * 256 + 131072 + 256) * 4
    assert lib.pa_moe_sort_workspace_bytes(1, 256, 8) == (1 * 256 + 8 + 256) * 4
    assert lib.pa_moe_sort_workspace_bytes(10, 0, 8) == L.PA_EINVAL
    ws = lib.pa_moe_sort_workspace_bytes(100, 16, 4)
    assert lib.pa_moe_sort_by_expert(a, a, a, a, 100, 16, 4, a, ws - 4, n) == L.PA_EINVAL   # workspace too small
    assert lib.pa_moe_sort_by_expert(a, n, a, a, 100, 16, 4, a, ws, n) == L.PA_EINVAL
    assert lib.pa_moe_sort_by_expert(a, a, a, a, 100, 16, 4, ctypes.c_void_p(A + 1), ws, n) == L.PA_EALIGN
    # permute / combine: row bytes must be a multiple of 16, dtype known
    assert lib.pa_moe_permute(a, a, a, 10, 8, 2047, L.PA_BF16, n) == L.PA_EALIGN
    assert lib.pa_moe_permute(a, a, a, 10, 8, 2048, 9, n) == L.PA_EUNSUPPORTED
    assert lib.pa_moe_permute(a, ctypes.c_void_p(A + 8), a, 10, 8, 2048, L.PA_BF16, n) == L.PA_EALIGN
    assert lib.pa_moe_combine(a, a, a, n, 10, 8, 2048, L.PA_BF16, n) == L.PA_EINVAL
    assert lib.pa_moe_combine(a, a, a, a, 10, 40, 2048, L.PA_BF16, n) == L.PA_EUNSUPPORTED
    assert lib.pa_moe_combine(n, n, n, n, 0, 8, 2048, L.PA_F32, n) == L.PA_OK
    assert f is not None


def test_load_binds_to_one_hip_runtime():
    """Loading the library before torch must still leave one HIP runtime in
    the process (two runtimes make every launch on torch's streams fail)."""
    import os
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    code = ("from paged_attention_decode_06_amd import _lib as L\n"
            "L.load()\n"
            "print(len(L._hip_runtimes()))\n")
    res = subprocess.run([sys.executable, "-c", code], cwd=root, capture_output=True, text=True, timeout=300)
    assert res.returncode == 0, res.stderr
    assert res.stdout.strip().splitlines()[-1] == "1"


def test_binding_checks_buffer_sizes_before_launch():
    """The binding compares every decode buffer with the shape it passes, on
    the host: partials allocated for 512-token partitions and a call that
    opts into 256-token ones (twice the partitions) raise instead of letting
    the kernel write past tmp_out's end."""
    import torch
    S, H, Hkv, D, MB = 2, 16, 2, 128, 100
    sh512 = shape(num_seqs=S, max_blocks_per_seq=MB)
    sh256 = shape(num_seqs=S, max_blocks_per_seq=MB, partition_size=256)
    P512 = (MB * 16 + 511) // 512
    es = torch.empty((S, H, P512))
    ml = torch.empty((S, H, P512))
    to = torch.empty((S, H, P512, D))
    out = torch.empty((S, H, D))
    sl = torch.zeros(S, dtype=torch.int32)
    L.check_sizes(sh512, out=out, seq_lens=sl, partials=(es, ml, to))          # consistent: no error
    with pytest.raises(L.PaError, match="tmp_out|exp_sums") as e:
        L.check_sizes(sh256, out=out, seq_lens=sl, partials=(es, ml, to))
    assert e.value.status == L.PA_EINVAL
    with pytest.raises(L.PaError, match="seq_lens"):
        L.check_sizes(sh512, out=out, seq_lens=torch.zeros(S + 1, dtype=torch.int32))
    with pytest.raises(L.PaError, match="out"):
        L.check_sizes(sh512, out=torch.empty((S, H, D // 2)), seq_lens=sl)
    with pytest.raises(L.PaError, match="tmp_out"):
        L.check_sizes(sh512, partials=(es, ml, torch.empty((S, H, P512 - 1, D))))
    with pytest.raises(L.PaError, match="cache"):
        L.check_sizes(sh512, k_cache=torch.empty((999, Hkv, 16, D)))
    L.check_sizes(sh512, k_cache=torch.empty((1000, Hkv, 16, D)))


def test_noalloc_rejects_partials_beyond_its_scratch(lib):
    """pa_decode_noalloc refuses, before any HIP call, a shape whose partials
    (S * H * Pmax * (D + 2) floats, each array 256-byte aligned) exceed the
    library's 64 MiB array; a single-pass-only shape needs no partials."""
    a = ctypes.c_void_p(A)
    n = None
    # 64 sequences x 16 heads x 128 partitions x (128 + 2) floats = 68.2 MB > 64 MiB
    big = shape(num_seqs=64, max_blocks_per_seq=4096)
    assert lib.pa_decode_noalloc(a, a, a, a, a, a, ctypes.byref(big), 1.0, n) == L.PA_ESCRATCH
    assert b"scratch" in lib.pa_status_string(L.PA_ESCRATCH)
    assert lib.pa_decode_noalloc(a, n, a, a, a, a, ctypes.byref(shape()), 1.0, n) == L.PA_EINVAL
    assert lib.pa_decode_noalloc(a, a, a, a, a, a, ctypes.byref(shape(head_dim=96)), 1.0, n) == L.PA_EUNSUPPORTED
    assert lib.pa_decode_noalloc(a, a, a, a, a, a, ctypes.byref(shape(num_seqs=0)), 1.0, n) == L.PA_OK
    # the arithmetic of the limit at 128 partitions of 16 heads: 63 sequences
    # fit (130 * 129024 floats), 64 do not
    assert 2 * 63 * 16 * 128 + 63 * 16 * 128 * 128 <= L.NOALLOC_SCRATCH_BYTES // 4
    assert 2 * 64 * 16 * 128 + 64 * 16 * 128 * 128 > L.NOALLOC_SCRATCH_BYTES // 4
