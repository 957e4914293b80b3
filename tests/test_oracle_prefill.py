"""Pins for the fp64 prefix/chunked-prefill oracle (CPU only).

Each check compares oracle.prefill against something other than itself:
40-digit brute force, torch's fp64 scaled_dot_product_attention with an
explicit mask and with is_causal, the decode oracle (pinned on its own in
test_oracle.py) for single tokens, and invariants. Planted mistakes in the
oracle (an exclusive mask, a position off by one, interleaved KV heads) must
each be caught.
"""
import math

import numpy as np
import pytest

import oracle
import oracle.prefill as op
from test_oracle import brute_decimal, maxerr, paged_from_dense


def prefill_case(rng, lens, qlens, H, Hkv, D, scale=None, garbage=np.nan):
    """Dense per-sequence K/V scattered into a paged pool, plus packed chunk queries."""
    dk = [rng.standard_normal((L, Hkv, D)).astype(np.float32) for L in lens]
    dv = [rng.standard_normal((L, Hkv, D)).astype(np.float32) for L in lens]
    T = int(sum(qlens))
    q = rng.standard_normal((T, H, D)).astype(np.float32)
    qsl = np.concatenate([[0], np.cumsum(qlens)]).astype(np.int32)
    kc, vc, tables, sl = paged_from_dense(dk, dv, rng, garbage=garbage)
    scale = 1.0 / math.sqrt(D) if scale is None else scale
    return q, qsl, dk, dv, kc, vc, tables, sl, scale


CASES = [([5, 37], [3, 37], 4, 2, 8), ([16, 20], [16, 1], 2, 1, 8), ([33], [17], 6, 3, 4)]


def check_bruteforce(mod, seed=0):
    rng = np.random.default_rng(seed)
    worst = 0.0
    for lens, qlens, H, Hkv, D in CASES:
        q, qsl, dk, dv, kc, vc, tables, sl, scale = prefill_case(rng, lens, qlens, H, Hkv, D)
        out = mod.attend_prefill(q, kc, vc, tables, sl, qsl, scale, "f32")
        G = H // Hkv
        for s, (L, Q) in enumerate(zip(lens, qlens)):
            for i in range(Q):
                pos = L - Q + i
                for h in range(H):
                    K = dk[s][:pos + 1, h // G].astype(np.float64)
                    V = dv[s][:pos + 1, h // G].astype(np.float64)
                    ref = brute_decimal(q[qsl[s] + i, h], K, V, scale)
                    worst = max(worst, maxerr(out[qsl[s] + i, h], ref))
    return worst


def check_sdpa_masked(mod, seed=1):
    """Library routine: fp64 SDPA with the causal-over-context mask spelled out as a boolean matrix."""
    import torch
    rng = np.random.default_rng(seed)
    worst = 0.0
    for lens, qlens, H, Hkv, D in [([300, 40], [64, 40], 16, 2, 128), ([129], [1], 8, 8, 64),
                                   ([77, 512], [33, 200], 4, 1, 256)]:
        q, qsl, dk, dv, kc, vc, tables, sl, scale = prefill_case(rng, lens, qlens, H, Hkv, D, scale=0.41)
        out = mod.attend_prefill(q, kc, vc, tables, sl, qsl, scale, "f32")
        G = H // Hkv
        for s, (L, Q) in enumerate(zip(lens, qlens)):
            k = torch.from_numpy(dk[s].astype(np.float64)).permute(1, 0, 2).repeat_interleave(G, dim=0)
            v = torch.from_numpy(dv[s].astype(np.float64)).permute(1, 0, 2).repeat_interleave(G, dim=0)
            qq = torch.from_numpy(q[qsl[s]:qsl[s + 1]].astype(np.float64)).permute(1, 0, 2)   # [H, Q, D]
            mask = torch.zeros((Q, L), dtype=torch.bool)
            for i in range(Q):
                mask[i, :L - Q + i + 1] = True
            ref = torch.nn.functional.scaled_dot_product_attention(qq, k, v, attn_mask=mask, scale=scale)
            worst = max(worst, maxerr(out[qsl[s]:qsl[s + 1]], ref.permute(1, 0, 2).numpy()))
    return worst


def check_sdpa_causal(mod, seed=2):
    """No prefix (Q = L): plain causal attention, torch's is_causal path."""
    import torch
    rng = np.random.default_rng(seed)
    worst = 0.0
    for L, H, Hkv, D in [(100, 8, 2, 64), (17, 2, 1, 128)]:
        q, qsl, dk, dv, kc, vc, tables, sl, scale = prefill_case(rng, [L], [L], H, Hkv, D)
        out = mod.attend_prefill(q, kc, vc, tables, sl, qsl, scale, "f32")
        G = H // Hkv
        k = torch.from_numpy(dk[0].astype(np.float64)).permute(1, 0, 2).repeat_interleave(G, dim=0)
        v = torch.from_numpy(dv[0].astype(np.float64)).permute(1, 0, 2).repeat_interleave(G, dim=0)
        qq = torch.from_numpy(q.astype(np.float64)).permute(1, 0, 2)
        ref = torch.nn.functional.scaled_dot_product_attention(qq, k, v, is_causal=True, scale=scale)
        worst = max(worst, maxerr(out, ref.permute(1, 0, 2).numpy()))
    return worst


def check_tokens_are_decodes(mod, seed=3):
    """Each chunk token equals decode attention over the context up to its own position."""
    rng = np.random.default_rng(seed)
    q, qsl, dk, dv, kc, vc, tables, sl, scale = prefill_case(rng, [90, 33], [25, 33], 8, 2, 32)
    out = mod.attend_prefill(q, kc, vc, tables, sl, qsl, scale, "f32")
    lists = oracle.gather_list(tables, sl)
    worst = 0.0
    for s in range(2):
        L, Q = int(sl[s]), int(qsl[s + 1] - qsl[s])
        for i in range(Q):
            dec = oracle.attend_seq(q[qsl[s] + i], kc, vc, lists[s], L - Q + i + 1, scale, "f32")
            worst = max(worst, maxerr(out[qsl[s] + i], dec))
    return worst


PINS = [check_bruteforce, check_sdpa_masked, check_sdpa_causal, check_tokens_are_decodes]


@pytest.mark.parametrize("pin", PINS, ids=lambda f: f.__name__)
def test_prefill_oracle_pins(pin):
    assert pin(op) <= 1e-12


def test_single_token_chunk_is_decode():
    rng = np.random.default_rng(4)
    lens = [1, 37, 600]
    q, qsl, dk, dv, kc, vc, tables, sl, scale = prefill_case(rng, lens, [1, 1, 1], 16, 2, 128)
    out = op.attend_prefill(q, kc, vc, tables, sl, qsl, scale, "f32")
    dec = oracle.attend_dense(q, kc, vc, tables, sl, scale, "f32")
    assert maxerr(out, dec) <= 1e-13


def test_chunk_longer_than_context_gives_zeros_for_negative_positions():
    rng = np.random.default_rng(5)
    q, qsl, dk, dv, kc, vc, tables, sl, scale = prefill_case(rng, [4], [4], 2, 1, 8)
    qsl = np.array([0, 6], dtype=np.int32)
    q = np.concatenate([rng.standard_normal((2, 2, 8)).astype(np.float32), q])
    out = op.attend_prefill(q, kc, vc, tables, sl, qsl, scale, "f32")
    assert (out[:2] == 0).all()                       # positions -2, -1 see no keys
    ref = op.attend_prefill(q[2:], kc, vc, tables, sl, np.array([0, 4]), scale, "f32")
    assert np.array_equal(out[2:], ref)


def test_block_permutation_is_bitwise_invariant():
    rng = np.random.default_rng(6)
    q, qsl, dk, dv, kc, vc, tables, sl, scale = prefill_case(rng, [70, 50], [30, 50], 4, 2, 16)
    base = op.attend_prefill(q, kc, vc, tables, sl, qsl, scale, "f32")
    perm = rng.permutation(kc.shape[0])
    k2 = np.empty_like(kc); v2 = np.empty_like(vc)
    k2[perm] = kc; v2[perm] = vc
    again = op.attend_prefill(q, k2, v2, perm[tables].astype(np.int32), sl, qsl, scale, "f32")
    assert np.array_equal(base, again)


def test_garbage_outside_contexts_never_reaches_output():
    rng = np.random.default_rng(7)
    q, qsl, dk, dv, kc, vc, tables, sl, scale = prefill_case(rng, [21, 40], [9, 40], 4, 2, 8, garbage=np.inf)
    out = op.attend_prefill(q, kc, vc, tables, sl, qsl, scale, "f32")
    assert np.isfinite(out).all()


def test_constant_v_gives_the_constant():
    rng = np.random.default_rng(8)
    q, qsl, dk, dv, kc, vc, tables, sl, scale = prefill_case(rng, [50], [20], 4, 1, 8)
    vc[:] = 0.75
    out = op.attend_prefill(q, kc, vc, tables, sl, qsl, scale, "f32")
    assert np.abs(out - 0.75).max() <= 1e-14


def test_row_form_matches_batch_form():
    rng = np.random.default_rng(9)
    q, qsl, dk, dv, kc, vc, tables, sl, scale = prefill_case(rng, [300], [100], 8, 2, 64)
    out = op.attend_prefill(q, kc, vc, tables, sl, qsl, scale, "f32")
    ids = oracle.gather_list(tables, sl)[0]
    for i in (0, 1, 57, 99):
        row = op.attend_prefill_row(q[i], kc, vc, ids, 300 - 100 + i, scale, "f32")
        assert maxerr(row, out[i]) <= 1e-13


def test_bf16_inputs_widen_exactly():
    """bf16 bit patterns go through the same widening as decode: a bf16 copy of an
    fp32 case whose values are bf16-representable gives the same result."""
    rng = np.random.default_rng(10)
    q, qsl, dk, dv, kc, vc, tables, sl, scale = prefill_case(rng, [40], [12], 4, 2, 16, garbage=0.0)
    rb = lambda a: (np.asarray(a, np.float32).view(np.uint32) >> 16).astype(np.uint16)
    wid = lambda b: (b.astype(np.uint32) << 16).view(np.float32)
    qb, kb, vb = rb(q), rb(kc), rb(vc)
    f = op.attend_prefill(wid(qb), wid(kb), wid(vb), tables, sl, qsl, scale, "f32")
    b = op.attend_prefill(qb, kb, vb, tables, sl, qsl, scale, "bf16")
    assert np.array_equal(f, b)


# ---------------------------------------------------------------- planted mistakes
def _mut_exclusive_mask(q_rows, k_cache, v_cache, block_ids, L, scale, dtype):
    """Tokens attend to keys strictly before their own position (drops the diagonal)."""
    Q, H, D = q_rows.shape
    out = np.zeros((Q, H, D))
    Hkv = k_cache.shape[1]; G = H // Hkv
    pos = op.query_positions(L, Q)
    qf = op.widen(q_rows, dtype)
    for kv in range(Hkv):
        K = op.gather_kv(k_cache, block_ids, kv, L, dtype); V = op.gather_kv(v_cache, block_ids, kv, L, dtype)
        for g in range(G):
            z = scale * (qf[:, kv * G + g] @ K.T)
            z = np.where(np.arange(L)[None, :] < pos[:, None], z, -np.inf)   # a row at pos 0 becomes NaN
            with np.errstate(invalid="ignore"):
                w = np.exp(z - z.max(axis=1, keepdims=True))
            out[:, kv * G + g] = (w @ V) / w.sum(axis=1, keepdims=True)
    return out


def _mut_position_off_by_one(L, Q):
    return np.arange(L - Q + 1, L + 1, dtype=np.int64)


def _mut_interleaved_heads(q_rows, k_cache, v_cache, block_ids, L, scale, dtype):
    """Query head h reads KV head h % Hkv (interleaved instead of grouped)."""
    Q, H, D = q_rows.shape
    out = np.zeros((Q, H, D))
    Hkv = k_cache.shape[1]
    pos = op.query_positions(L, Q)
    qf = op.widen(q_rows, dtype)
    allowed = np.arange(L)[None, :] <= pos[:, None]
    for h in range(H):
        K = op.gather_kv(k_cache, block_ids, h % Hkv, L, dtype); V = op.gather_kv(v_cache, block_ids, h % Hkv, L, dtype)
        z = np.where(allowed, scale * (qf[:, h] @ K.T), -np.inf)
        w = np.exp(z - z.max(axis=1, keepdims=True))
        out[:, h] = (w @ V) / w.sum(axis=1, keepdims=True)
    return out


@pytest.mark.parametrize("target,mutant", [
    ("attend_prefill_seq", _mut_exclusive_mask),
    ("query_positions", _mut_position_off_by_one),
    ("attend_prefill_seq", _mut_interleaved_heads),
])
def test_planted_mistake_is_caught(monkeypatch, target, mutant):
    monkeypatch.setattr(op, target, mutant)
    errs = [pin(op) for pin in PINS]
    assert max(errs) > 1e-6, f"planted mistake in {target} went unnoticed: {errs}"
