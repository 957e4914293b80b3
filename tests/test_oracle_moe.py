"""Pins for the MoE routing oracle (CPU only): brute force, torch's topk and
softmax, a dense routing-matrix formulation of the combine, closed forms,
and planted mistakes that some pin must catch."""
import math

import numpy as np
import pytest

import oracle.moe as om


def brute_topk(logits, k, renormalize=False):
    T, E = logits.shape
    W = np.zeros((T, k)); I = np.zeros((T, k), dtype=np.int32)
    for t in range(T):
        row = [float(v) for v in logits[t]]
        mx = max(row)
        ex = [math.exp(v - mx) for v in row]
        tot = math.fsum(ex)
        pick = sorted(range(E), key=lambda e: (-row[e], e))[:k]
        ws = [ex[e] / tot for e in pick]
        if renormalize:
            s = math.fsum(ws)
            ws = [v / s for v in ws]
        W[t] = ws; I[t] = pick
    return W, I


def brute_sort(ids, E):
    flat = [int(v) for v in ids.reshape(-1)]
    order = []
    offsets = [0]
    for e in range(E):
        order += [a for a in range(len(flat)) if flat[a] == e]
        offsets.append(len(order))
    return np.array(order), np.array(offsets)


def check_topk_brute(mod, seed=0):
    rng = np.random.default_rng(seed)
    worst = 0.0
    for T, E, k in [(7, 16, 4), (3, 64, 8), (5, 8, 8)]:
        lg = rng.standard_normal((T, E)).astype(np.float32)
        for ren in (False, True):
            w, i = mod.topk_softmax(lg, k, ren)
            bw, bi = brute_topk(lg, k, ren)
            if not np.array_equal(i, bi):
                return float("inf")
            worst = max(worst, float(np.abs(w - bw).max()))
    return worst


def check_topk_torch(mod, seed=1):
    import torch
    rng = np.random.default_rng(seed)
    lg = rng.standard_normal((50, 256)).astype(np.float32)
    w, i = mod.topk_softmax(lg, 8)
    p = torch.softmax(torch.from_numpy(lg.astype(np.float64)), dim=1)
    tw, ti = torch.topk(p, 8, dim=1)
    if not np.array_equal(i, ti.numpy()):
        return float("inf")
    return float(np.abs(w - tw.numpy()).max())


def check_sort_brute(mod, seed=2):
    rng = np.random.default_rng(seed)
    for T, K, E in [(40, 8, 16), (9, 2, 4), (100, 4, 256)]:
        ids = rng.integers(0, E, size=(T, K)).astype(np.int32)
        sp, pp, off = mod.sort_by_expert(ids, E)
        bo, boff = brute_sort(ids, E)
        if not (np.array_equal(sp, bo) and np.array_equal(off, boff) and np.array_equal(pp[sp], np.arange(T * K))):
            return float("inf")
    return 0.0


def check_combine_dense(mod, seed=3):
    """out = R Y per token, with R the dense [T, E] routing matrix: no sorted order involved."""
    rng = np.random.default_rng(seed)
    T, E, K, Hd = 30, 16, 4, 8
    lg = rng.standard_normal((T, E)).astype(np.float32)
    w, ids = mod.topk_softmax(lg, K, True)
    sp, pp, off = mod.sort_by_expert(ids, E)
    Y = rng.standard_normal((E, T, Hd))
    y_sorted = np.array([Y[ids.reshape(-1)[a], a // K] for a in sp])
    out = mod.combine(y_sorted, w, pp)
    R = np.zeros((T, E))
    for t in range(T):
        for j in range(K):
            R[t, ids[t, j]] += w[t, j]
    ref = np.einsum("te,eth->th", R, Y)
    return float(np.abs(out - ref).max())


def check_permute(mod, seed=4):
    rng = np.random.default_rng(seed)
    T, K, E, Hd = 20, 3, 5, 6
    ids = rng.integers(0, E, size=(T, K)).astype(np.int32)
    x = rng.standard_normal((T, Hd))
    sp, pp, off = mod.sort_by_expert(ids, E)
    xs = mod.permute_rows(x, sp, K)
    for e in range(E):
        toks = [t for t in range(T) for j in range(K) if ids[t, j] == e]
        if not np.array_equal(xs[off[e]:off[e + 1]], x[toks]):
            return float("inf")
    return 0.0


PINS = [check_topk_brute, check_topk_torch, check_sort_brute, check_combine_dense, check_permute]


@pytest.mark.parametrize("pin", PINS, ids=lambda f: f.__name__)
def test_moe_oracle_pins(pin):
    assert pin(om) <= 1e-14


def test_topk_ties_go_to_the_lower_id():
    lg = np.array([[1.0, 3.0, 3.0, 0.0]], dtype=np.float32)
    w, i = om.topk_softmax(lg, 2)
    assert i.tolist() == [[1, 2]]
    e = math.e
    assert abs(w[0, 0] - e ** 3 / (e + 2 * e ** 3 + 1)) < 1e-15
    w2, _ = om.topk_softmax(lg, 2, renormalize=True)
    assert np.allclose(w2, 0.5, atol=1e-15, rtol=0)


def test_softmax_sums_to_one_over_all_experts():
    rng = np.random.default_rng(5)
    lg = rng.standard_normal((10, 32)).astype(np.float32)
    w, _ = om.topk_softmax(lg, 32)
    assert np.abs(w.sum(axis=1) - 1).max() < 1e-14


def test_offsets_partition_the_pairs():
    rng = np.random.default_rng(6)
    ids = rng.integers(0, 256, size=(1000, 8)).astype(np.int32)
    sp, pp, off = om.sort_by_expert(ids, 256)
    flat = ids.reshape(-1)
    assert off[0] == 0 and off[-1] == flat.size and (np.diff(off) >= 0).all()
    for e in (0, 17, 255):
        seg = sp[off[e]:off[e + 1]]
        assert (flat[seg] == e).all() and (np.diff(seg) > 0).all()     # stable: ascending pair index


# ---------------------------------------------------------------- planted mistakes
def _mut_ties_high(logits, k, renormalize=False):
    lg = np.asarray(logits, dtype=np.float32).astype(np.float64)
    p = np.exp(lg - lg.max(axis=1, keepdims=True)); p /= p.sum(axis=1, keepdims=True)
    order = np.argsort(-lg[:, ::-1], axis=1, kind="stable")[:, :k]
    order = lg.shape[1] - 1 - order
    w = np.take_along_axis(p, order, axis=1)
    return (w / w.sum(axis=1, keepdims=True) if renormalize else w), order.astype(np.int32)


def _mut_softmax_over_chosen(logits, k, renormalize=False):
    w, i = _ORIG_TOPK(logits, k, True)
    return w, i


def _mut_unstable_sort(topk_ids, num_experts):
    sp, pp, off = _ORIG_SORT(topk_ids, num_experts)
    for e in range(num_experts):
        sp[off[e]:off[e + 1]] = sp[off[e]:off[e + 1]][::-1].copy()
    pp = np.empty_like(sp); pp[sp] = np.arange(sp.size)
    return sp, pp, off


def _mut_combine_wrong_inverse(y_sorted, weights, pair_pos):
    sp = np.argsort(pair_pos)            # sorted_pairs instead of pair_pos
    return _ORIG_COMBINE(y_sorted, weights, sp.astype(np.int32))


_ORIG_TOPK, _ORIG_SORT, _ORIG_COMBINE = om.topk_softmax, om.sort_by_expert, om.combine


@pytest.mark.parametrize("target,mutant", [
    ("topk_softmax", _mut_ties_high),
    ("topk_softmax", _mut_softmax_over_chosen),
    ("sort_by_expert", _mut_unstable_sort),
    ("combine", _mut_combine_wrong_inverse),
])
def test_planted_mistake_is_caught(monkeypatch, target, mutant):
    monkeypatch.setattr(om, target, mutant)
    errs = [pin(om) for pin in PINS]
    try:
        test_topk_ties_go_to_the_lower_id()
        errs.append(0.0)
    except AssertionError:
        errs.append(float("inf"))
    assert max(errs) > 1e-6, f"planted mistake in {target} went unnoticed: {errs}"
