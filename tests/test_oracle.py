"""Pins for the fp64 oracle (CPU only).

Each check compares the oracle against something other than itself: exact
40-digit brute force, torch's fp64 scaled_dot_product_attention, closed forms,
invariants, and values the pages fix (tests/golden/). The last group plants
plausible mistakes in the oracle and asserts that some pin catches each one.
"""
import math
from decimal import Decimal, getcontext

import numpy as np
import pytest

import oracle
import oracle.attention as oa

BS = 16


# ---------------------------------------------------------------- helpers
def maxerr(a, b):
    """max |a - b|, with any NaN counted as an infinite error."""
    e = np.abs(np.asarray(a, dtype=np.float64) - np.asarray(b, dtype=np.float64))
    return float("inf") if np.isnan(e).any() else float(e.max(initial=0.0))


def paged_from_dense(dense_k, dense_v, rng, pool_extra=3, garbage=np.nan):
    """Scatter per-sequence dense K/V ([L, Hkv, D] each) into a shuffled paged pool.

    Written from the layout's definition in the scatter direction (dense ->
    pool), independent of the oracle's gather. Slots no context covers hold
    `garbage`.
    """
    lens = [k.shape[0] for k in dense_k]
    Hkv, D = dense_k[0].shape[1], dense_k[0].shape[2]
    need = [(L + BS - 1) // BS for L in lens]
    nb = sum(need) + pool_extra
    perm = rng.permutation(nb)
    kc = np.full((nb, Hkv, BS, D), garbage, dtype=np.float32)
    vc = np.full((nb, Hkv, BS, D), garbage, dtype=np.float32)
    mb = max(max(need), 1) + 2
    tables = np.full((len(lens), mb), nb - 1, dtype=np.int32)   # padding -> an unused block
    pos = 0
    for s, L in enumerate(lens):
        for i in range(need[s]):
            b = int(perm[pos]); pos += 1
            tables[s, i] = b
            for slot in range(BS):
                t = i * BS + slot
                if t < L:
                    kc[b, :, slot, :] = dense_k[s][t]
                    vc[b, :, slot, :] = dense_v[s][t]
    # padding entries must point at a block no sequence uses
    used = set(tables[s, i] for s in range(len(lens)) for i in range(need[s]))
    spare = [b for b in range(nb) if b not in used]
    for s in range(len(lens)):
        tables[s, need[s]:] = spare[0]
    return kc, vc, tables, np.asarray(lens, dtype=np.int32)


def random_case(rng, lens, H, Hkv, D, scale=None, garbage=np.nan):
    dk = [rng.standard_normal((L, Hkv, D)).astype(np.float32) for L in lens]
    dv = [rng.standard_normal((L, Hkv, D)).astype(np.float32) for L in lens]
    q = rng.standard_normal((len(lens), H, D)).astype(np.float32)
    kc, vc, tables, sl = paged_from_dense(dk, dv, rng, garbage=garbage)
    scale = 1.0 / math.sqrt(D) if scale is None else scale
    return q, dk, dv, kc, vc, tables, sl, scale


def brute_decimal(qh, K, V, scale):
    """softmax(scale * q.K) V with 40 significant digits, no max shift."""
    getcontext().prec = 40
    L, D = K.shape
    sc = Decimal(float(scale))
    z = [sc * sum(Decimal(float(qh[d])) * Decimal(float(K[t, d])) for d in range(D)) for t in range(L)]
    e = [zi.exp() for zi in z]
    tot = sum(e)
    return np.array([float(sum(e[t] * Decimal(float(V[t, d])) for t in range(L)) / tot) for d in range(D)])


def check_bruteforce(mod, seed=0):
    rng = np.random.default_rng(seed)
    worst = 0.0
    for lens, H, Hkv, D in [([37, 1, 70], 4, 2, 4), ([16, 17], 2, 1, 8), ([33], 6, 3, 4)]:
        q, dk, dv, kc, vc, tables, sl, scale = random_case(rng, lens, H, Hkv, D)
        out = mod.attend_dense(q, kc, vc, tables, sl, scale, "f32")
        G = H // Hkv
        for s, L in enumerate(lens):
            for h in range(H):
                ref = brute_decimal(q[s, h], dk[s][:, h // G].astype(np.float64), dv[s][:, h // G].astype(np.float64), scale)
                worst = max(worst, maxerr(out[s, h], ref))
    return worst


def check_sdpa(mod, seed=1):
    import torch
    rng = np.random.default_rng(seed)
    worst = 0.0
    for lens, H, Hkv, D in [([37, 200, 5], 16, 2, 128), ([513, 1], 8, 8, 64), ([64], 2, 1, 256)]:
        q, dk, dv, kc, vc, tables, sl, scale = random_case(rng, lens, H, Hkv, D, scale=0.37)
        out = mod.attend_dense(q, kc, vc, tables, sl, scale, "f32")
        G = H // Hkv
        for s, L in enumerate(lens):
            k = torch.from_numpy(dk[s].astype(np.float64)).permute(1, 0, 2).repeat_interleave(G, dim=0)
            v = torch.from_numpy(dv[s].astype(np.float64)).permute(1, 0, 2).repeat_interleave(G, dim=0)
            qq = torch.from_numpy(q[s].astype(np.float64)).unsqueeze(1)             # [H, 1, D]
            ref = torch.nn.functional.scaled_dot_product_attention(qq, k, v, scale=scale)[:, 0].numpy()
            worst = max(worst, maxerr(out[s], ref))
    return worst


def check_v1_v2(mod, seed=2):
    rng = np.random.default_rng(seed)
    q, dk, dv, kc, vc, tables, sl, scale = random_case(rng, [37, 513, 1, 1100], 8, 2, 32)
    dense = mod.attend_dense(q, kc, vc, tables, sl, scale, "f32")
    worst = 0.0
    for P in (1, 7, 16, 256, 512, 1100, 1101):
        v2 = mod.attend_v2(q, kc, vc, tables, sl, scale, "f32", P)
        worst = max(worst, maxerr(v2, dense))
    return worst


def check_closed_form_combine(mod):
    a = np.array([1.0, -2.0, 0.5]); b = np.array([3.0, 4.0, -1.0])
    # weights exp(0 - ln3) * 1 : exp(ln3 - ln3) * 1 = 1/3 : 1  ->  (a + 3 b) / 4
    got = mod.lse_combine(np.array([0.0, math.log(3.0)]), np.array([1.0, 1.0]), np.stack([a, b]))
    e1 = maxerr(got, (a + 3 * b) / 4)
    # exp-sums enter linearly: l = (2, 6) at equal maxima -> (a + 3 b) / 4 again
    got = mod.lse_combine(np.array([5.0, 5.0]), np.array([2.0, 6.0]), np.stack([a, b]))
    e2 = maxerr(got, (a + 3 * b) / 4)
    # single partition: the partition output itself
    e3 = maxerr(mod.lse_combine(np.array([7.0]), np.array([3.0]), a[None]), a)
    return max(e1, e2, e3)


# ---------------------------------------------------------------- pins
def test_p1_bruteforce_decimal():
    assert check_bruteforce(oracle) < 1e-12


def test_p2_torch_sdpa_fp64():
    assert check_sdpa(oracle) < 1e-12


def test_p3_v1_equals_v2_any_partition_size():
    assert check_v1_v2(oracle) < 1e-12


def test_lse_combine_closed_forms():
    assert check_closed_form_combine(oracle) < 1e-14


def test_partition_stats_definition():
    """m_p is the partition max of the scaled logits, l_p = sum exp(z - m_p), o_p normalised."""
    rng = np.random.default_rng(3)
    q, dk, dv, kc, vc, tables, sl, scale = random_case(rng, [1100], 2, 1, 8)
    m, l, o = oracle.partition_stats(q[0], kc, vc, tables[0, :69], 1100, scale, "f32", 512)
    assert m.shape == (2, 3) and o.shape == (2, 3, 8)
    K = dk[0][:, 0].astype(np.float64); V = dv[0][:, 0].astype(np.float64)
    for h in range(2):
        for p, (lo, hi) in enumerate([(0, 512), (512, 1024), (1024, 1100)]):
            z = [scale * float(np.dot(q[0, h].astype(np.float64), K[t])) for t in range(lo, hi)]
            assert m[h, p] == pytest.approx(max(z), abs=1e-12)
            w = [math.exp(x - max(z)) for x in z]
            assert l[h, p] == pytest.approx(math.fsum(w), rel=1e-12)
            ref = sum(wt * V[lo + i] for i, wt in enumerate(w)) / math.fsum(w)
            assert np.abs(o[h, p] - ref).max() < 1e-12


def test_p4_constant_v():
    rng = np.random.default_rng(4)
    q, dk, dv, kc, vc, tables, sl, scale = random_case(rng, [37, 300], 8, 2, 16)
    c = np.float32(1.625)
    vc2 = np.where(np.isnan(vc), vc, c).astype(np.float32)
    for fn in (oracle.attend_dense, lambda *a: oracle.attend_v2(*a, 7)):
        out = fn(q, kc, vc2, tables, sl, scale, "f32")
        assert np.abs(out - float(c)).max() <= 1e-14 * float(c)


def test_p5_single_token_returns_v0_exactly():
    rng = np.random.default_rng(5)
    q, dk, dv, kc, vc, tables, sl, scale = random_case(rng, [1, 1], 4, 2, 32)
    out = oracle.attend_dense(q, kc, vc, tables, sl, scale, "f32")
    for s in range(2):
        for h in range(4):
            assert np.array_equal(out[s, h], dv[s][0, h // 2].astype(np.float64))


def test_p6_block_permutation_is_bitwise_invariant():
    rng = np.random.default_rng(6)
    q, dk, dv, kc, vc, tables, sl, scale = random_case(rng, [37, 100, 5], 8, 2, 16)
    base = oracle.attend_dense(q, kc, vc, tables, sl, scale, "f32")
    perm = rng.permutation(kc.shape[0])          # new position of old block b is perm[b]
    kc2 = np.empty_like(kc); vc2 = np.empty_like(vc)
    kc2[perm] = kc; vc2[perm] = vc
    t2 = perm[tables].astype(np.int32)
    assert np.array_equal(oracle.attend_dense(q, kc2, vc2, t2, sl, scale, "f32"), base)


def test_p7_zero_query_or_zero_scale_gives_mean_of_v():
    rng = np.random.default_rng(7)
    q, dk, dv, kc, vc, tables, sl, scale = random_case(rng, [37, 129], 4, 2, 8)
    out0 = oracle.attend_dense(q, kc, vc, tables, sl, 0.0, "f32")
    outq = oracle.attend_dense(np.zeros_like(q), kc, vc, tables, sl, scale, "f32")
    for s, L in enumerate(sl):
        for h in range(4):
            mean = dv[s][:, h // 2].astype(np.float64).mean(axis=0)
            assert np.abs(out0[s, h] - mean).max() < 1e-14
            assert np.abs(outq[s, h] - mean).max() < 1e-14


def test_p8_dominant_key_selects_its_value():
    rng = np.random.default_rng(8)
    L, D = 50, 16
    dk = [rng.standard_normal((L, 1, D)).astype(np.float32)]
    dv = [rng.standard_normal((L, 1, D)).astype(np.float32)]
    q = rng.standard_normal((1, 1, D)).astype(np.float32)
    j = 23
    beta = 200.0
    dk[0][j, 0] = (beta * q[0, 0] / np.dot(q[0, 0], q[0, 0])).astype(np.float32)   # q.k_j = beta
    kc, vc, tables, sl = paged_from_dense(dk, dv, rng)
    out = oracle.attend_dense(q, kc, vc, tables, sl, 1.0, "f32")
    # all other logits are O(10): their weights are below exp(-150) relative to k_j
    assert np.abs(out[0, 0] - dv[0][j, 0]).max() < 1e-12


def test_p9_gqa_equals_replicated_kv_heads():
    rng = np.random.default_rng(9)
    q, dk, dv, kc, vc, tables, sl, scale = random_case(rng, [37, 70], 16, 2, 8)
    g = oracle.attend_dense(q, kc, vc, tables, sl, scale, "f32")
    rep = oracle.attend_dense(q, np.repeat(kc, 8, axis=1), np.repeat(vc, 8, axis=1), tables, sl, scale, "f32")
    # same values; only the BLAS blocking (8-row vs 1-row products) may reorder roundings
    assert np.abs(g - rep).max() < 1e-14


def test_p10_gather_list_matches_table_prefix():
    tables = np.array([[5, 9, 2, 7], [3, 0, 0, 0], [1, 4, 6, 0]], dtype=np.int32)
    got = oracle.gather_list(tables, np.array([49, 16, 33]))
    assert [g.tolist() for g in got] == [[5, 9, 2, 7], [3], [1, 4, 6]]
    got = oracle.gather_list(tables, np.array([0, 1, 17]))
    assert [g.tolist() for g in got] == [[], [3], [1, 4]]


def test_zero_length_context_gives_zeros():
    q = np.ones((1, 2, 4), np.float32)
    kc = np.full((2, 1, 16, 4), np.nan, np.float32)
    out = oracle.attend_dense(q, kc, kc, np.zeros((1, 1), np.int32), np.array([0]), 1.0, "f32")
    assert np.array_equal(out, np.zeros((1, 2, 4)))


def test_unreferenced_and_tail_slots_never_read():
    """NaN in every slot outside the contexts leaves the output finite (C8 reading)."""
    rng = np.random.default_rng(10)
    q, dk, dv, kc, vc, tables, sl, scale = random_case(rng, [37, 5, 100], 4, 2, 8, garbage=np.nan)
    assert np.isnan(kc).any()
    out = oracle.attend_dense(q, kc, vc, tables, sl, scale, "f32")
    assert np.isfinite(out).all()


def test_widen_f16_values():
    v = np.array([1.0, -2.5, 65504.0, 2.0 ** -24, np.inf], dtype=np.float16)
    w = oracle.widen(v, "f16")
    assert w.tolist()[:4] == [1.0, -2.5, 65504.0, 2.0 ** -24] and np.isinf(w[4])


def test_widen_bf16_bit_patterns():
    bits = np.array([0x3F80, 0xC000, 0x7F80, 0x0001, 0x3E80], dtype=np.uint16)
    w = oracle.widen(bits, "bf16")
    assert w[0] == 1.0 and w[1] == -2.0 and w[2] == np.inf and w[4] == 0.25
    assert w[3] == 2.0 ** -133        # smallest bf16 subnormal


def test_large_logits_stay_finite_and_match_decimal():
    """Logits near 700/scale: the max shift must keep exp finite (outlier-K workload)."""
    rng = np.random.default_rng(11)
    L, D = 40, 4
    dk = [(rng.standard_normal((L, 1, D)) * 300).astype(np.float32)]
    dv = [rng.standard_normal((L, 1, D)).astype(np.float32)]
    q = (rng.standard_normal((1, 1, D)) * 3).astype(np.float32)
    kc, vc, tables, sl = paged_from_dense(dk, dv, rng)
    out = oracle.attend_dense(q, kc, vc, tables, sl, 1.0, "f32")
    ref = brute_decimal(q[0, 0], dk[0][:, 0].astype(np.float64), dv[0][:, 0].astype(np.float64), 1.0)
    assert np.isfinite(out).all()
    assert np.abs(out[0, 0] - ref).max() < 1e-12


def _golden_rows(name):
    import os
    path = os.path.join(os.path.dirname(__file__), "golden", name)
    with open(path) as f:
        return [line.split() for line in f if line.strip() and not line.startswith("#")]


def test_golden_dispatch_and_partition_counts():
    for L, path, P, last in _golden_rows("dispatch_partitions.txt"):
        L, P, last = int(L), int(P), int(last)
        assert oracle.choose_path(L) == path
        assert oracle.num_partitions(L) == P
        assert L - (P - 1) * oracle.PARTITION_SIZE == last


# ---------------------------------------------------------------- planted mistakes
def _mut_kv_mapping(q_s, k_cache, v_cache, block_ids, L, scale, dtype):
    """attend_seq with query head h reading KV head h % Hkv (interleaved instead of grouped)."""
    H, D = q_s.shape
    Hkv = k_cache.shape[1]
    out = np.zeros((H, D))
    qf = oa.widen(q_s, dtype)
    for h in range(H):
        K = oa.gather_kv(k_cache, block_ids, h % Hkv, L, dtype)
        V = oa.gather_kv(v_cache, block_ids, h % Hkv, L, dtype)
        z = scale * (qf[h:h + 1] @ K.T)
        out[h] = oa._softmax_weighted_sum(z, V)[2][0]
    return out


def _mut_gather_slot(cache, block_ids, kv_head, L, dtype):
    """gather_kv reading slot (t + 1) % 16 instead of t % 16."""
    D = cache.shape[-1]
    rows = cache[block_ids, kv_head]
    rows = np.roll(rows, -1, axis=1).reshape(-1, D)[:L]
    return oa.widen(rows, dtype)


def _mut_softmax_no_scale_sum(z, V):
    m = z.max(axis=1); w = np.exp(z - m[:, None]); l = w.sum(axis=1)
    return m, l, (w @ V)            # partial output left unnormalised


def _mut_combine_sign(m, l, o):
    M = m.max(); c = np.exp(M - m) * l
    return (c[:, None] * o).sum(axis=0) / c.sum()


def _mut_combine_no_l(m, l, o):
    M = m.max(); c = np.exp(m - M)
    return (c[:, None] * o).sum(axis=0) / c.sum()


def _mut_transposed_v(z, V):
    m = z.max(axis=1); w = np.exp(z - m[:, None]); l = w.sum(axis=1)
    Vt = V[::-1]                     # values paired with the wrong tokens
    return m, l, (w @ Vt) / l[:, None]


@pytest.mark.parametrize("target,mutant", [
    ("attend_seq", _mut_kv_mapping),
    ("gather_kv", _mut_gather_slot),
    ("_softmax_weighted_sum", _mut_softmax_no_scale_sum),
    ("lse_combine", _mut_combine_sign),
    ("lse_combine", _mut_combine_no_l),
    ("_softmax_weighted_sum", _mut_transposed_v),
])
def test_planted_mistake_is_caught(monkeypatch, target, mutant):
    monkeypatch.setattr(oa, target, mutant)
    errs = [check_v1_v2(oa), check_closed_form_combine(oa)]
    if target != "lse_combine":
        errs += [check_bruteforce(oa), check_sdpa(oa)]
    assert max(errs) > 1e-6, f"planted mistake in {target} went unnoticed: {errs}"
