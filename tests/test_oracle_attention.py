"""Pins of the oracle's paged verify attention (oracle/attention.py) to values fixed by the
mathematics, not by the oracle itself:

* a library routine (torch scaled_dot_product_attention, CPU, float64) on the same keys laid
  out contiguously, with the query heads' KV heads expanded by repeat_interleave;
* hand-computed closed forms: a zero query averages the visible values, so values equal to
  their position give (lo + t) / 2 with lo, t written out as numbers below;
* invariants: a permuted page pool with the matching table changes nothing; a window at least
  as long as the context equals global attention; a window of 1 returns the query's own value.
"""
import math

import numpy as np
import pytest
import torch

import oracle


def paged_from_contiguous(keys_per_seq, page_size, hkv, d, rng, spare=3):
    """Scatter per-sequence contiguous [T_b, Hkv, D] arrays into a shuffled page pool."""
    need = [math.ceil(k.shape[0] / page_size) for k in keys_per_seq]
    P = sum(need) + spare
    perm = rng.permutation(P)
    pool = rng.standard_normal((P, hkv, page_size, d))  # garbage in unused slots
    table = np.full((len(keys_per_seq), max(need) + 2), -1, dtype=np.int32)
    base = 0
    for b, k in enumerate(keys_per_seq):
        for j in range(need[b]):
            page = perm[base + j]
            table[b, j] = page
            chunk = k[j * page_size:(j + 1) * page_size]
            pool[page, :, :chunk.shape[0], :] = np.transpose(chunk, (1, 0, 2))
        base += need[b]
    return pool, table


@pytest.mark.parametrize("window", [0, 5, 13, 1000])
def test_matches_sdpa_on_contiguous_keys(window):
    rng = np.random.default_rng(7)
    B, K1, Hq, Hkv, D, ps = 3, 4, 6, 2, 8, 4
    ctx = [9, 23, 4]
    ks = [rng.standard_normal((c, Hkv, D)) for c in ctx]
    vs = [rng.standard_normal((c, Hkv, D)) for c in ctx]
    rng2 = np.random.default_rng(8)
    kp, table = paged_from_contiguous(ks, ps, Hkv, D, rng2)
    rng2 = np.random.default_rng(8)
    vp, table2 = paged_from_contiguous(vs, ps, Hkv, D, rng2)
    assert (table == table2).all()
    q = rng.standard_normal((B, K1, Hq, D))
    scale = 1 / math.sqrt(D)
    got = oracle.verify_attention(q, kp, vp, table, ctx, window, scale)
    for b in range(B):
        T = ctx[b]
        kk = torch.from_numpy(ks[b]).permute(1, 0, 2).repeat_interleave(Hq // Hkv, dim=0)
        vv = torch.from_numpy(vs[b]).permute(1, 0, 2).repeat_interleave(Hq // Hkv, dim=0)
        qq = torch.from_numpy(q[b]).permute(1, 0, 2)           # [Hq, K1, D]
        pos_q = torch.arange(T - K1, T)[:, None]
        pos_k = torch.arange(T)[None, :]
        mask = pos_k <= pos_q
        if window > 0:
            mask &= (pos_q - pos_k) < window
        ref = torch.nn.functional.scaled_dot_product_attention(
            qq, kk, vv, attn_mask=mask, scale=scale)           # [Hq, K1, D]
        np.testing.assert_allclose(got[b], ref.permute(1, 0, 2).numpy(), rtol=0, atol=1e-12)


def _position_values(P, hkv, ps, d, table, ctx):
    """Pools whose value vectors equal the logical position of the key (all dims)."""
    v = np.full((P, hkv, ps, d), -1e9)
    for b, c in enumerate(ctx):
        for s in range(c):
            v[table[b, s // ps], :, s % ps, :] = s
    return v


def test_zero_query_averages_visible_positions():
    # ctx 40, K1 3 -> query positions t = 37, 38, 39.
    ps, hkv, d = 8, 1, 2
    table = np.array([[4, 0, 3, 1, 2]], dtype=np.int32)
    ctx = [40]
    P = 5
    k = np.random.default_rng(0).standard_normal((P, hkv, ps, d))
    v = _position_values(P, hkv, ps, d, table, ctx)
    q = np.zeros((1, 3, 2, d))
    glob = oracle.verify_attention(q, k, v, table, ctx, 0, 1.0)
    # global: mean of 0..t
    np.testing.assert_allclose(glob[0, :, 0, 0], [18.5, 19.0, 19.5], atol=1e-12)
    slid = oracle.verify_attention(q, k, v, table, ctx, 8, 1.0)
    # window 8: positions t-7..t -> means 33.5, 34.5, 35.5
    np.testing.assert_allclose(slid[0, :, 1, 1], [33.5, 34.5, 35.5], atol=1e-12)
    one = oracle.verify_attention(q, k, v, table, ctx, 1, 1.0)
    np.testing.assert_allclose(one[0, :, 0, 0], [37.0, 38.0, 39.0], atol=1e-12)


def test_two_keys_closed_form():
    # one sequence of 2 tokens, K1 = 1: the query sees keys 0 and 1.
    k = np.zeros((1, 1, 2, 2))
    k[0, 0, 0] = [1.0, 0.0]
    k[0, 0, 1] = [0.0, 1.0]
    v = np.zeros((1, 1, 2, 2))
    v[0, 0, 0] = [10.0, 0.0]
    v[0, 0, 1] = [0.0, 20.0]
    q = np.array([[[[2.0, 0.5]]]])
    out = oracle.verify_attention(q, k, v, np.array([[0]]), [2], 0, 0.5)
    # scores 1.0 and 0.25 -> weights e/(e+e^0.25), e^0.25/(e+e^0.25)
    w0 = math.e / (math.e + math.exp(0.25))
    np.testing.assert_allclose(out[0, 0, 0], [10 * w0, 20 * (1 - w0)], atol=1e-12)


def test_page_permutation_and_long_window_invariance():
    rng = np.random.default_rng(3)
    B, K1, Hq, Hkv, D, ps = 2, 3, 4, 2, 16, 16
    ctx = [50, 37]
    P = 8
    table = np.array([[0, 1, 2, 3], [4, 5, 6, -1]], dtype=np.int32)
    kp = rng.standard_normal((P, Hkv, ps, D))
    vp = rng.standard_normal((P, Hkv, ps, D))
    q = rng.standard_normal((B, K1, Hq, D))
    base = oracle.verify_attention(q, kp, vp, table, ctx, 0, 0.25)
    perm = rng.permutation(P)
    inv = np.argsort(perm)          # new page index of old page j is inv[j]
    kp2, vp2 = kp[perm], vp[perm]
    table2 = np.where(table >= 0, inv[np.maximum(table, 0)], -1)
    moved = oracle.verify_attention(q, kp2, vp2, table2, ctx, 0, 0.25)
    np.testing.assert_allclose(moved, base, atol=1e-12)
    long_window = oracle.verify_attention(q, kp, vp, table, ctx, 64, 0.25)
    np.testing.assert_allclose(long_window, base, atol=1e-12)


def test_invalid_page_hides_its_keys_and_empty_rows_are_zero():
    ps, d = 4, 2
    table = np.array([[0, 99]], dtype=np.int32)   # second page id is outside the pool
    k = np.zeros((1, 1, ps, d))
    v = np.zeros((1, 1, ps, d))
    v[0, 0, :, 0] = [1.0, 2.0, 3.0, 4.0]
    q = np.zeros((1, 2, 1, d))
    out = oracle.verify_attention(q, k, v, table, [6], 0, 1.0)
    # queries at 4 and 5 see positions 0..3 only (page 99 missing): mean 2.5
    np.testing.assert_allclose(out[0, :, 0, 0], [2.5, 2.5], atol=1e-12)
    out2 = oracle.verify_attention(q, k, v, table, [6], 1, 1.0)
    np.testing.assert_allclose(out2, 0.0)
