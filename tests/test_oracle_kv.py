"""Pins of the KV bookkeeping oracle (oracle/kv.py) against a list model of each sequence
(brute force): a sequence's committed tokens are its prefix followed, per step, by the last
committed token's successors that were accepted; rows land where the page table says."""
import numpy as np

from oracle import kv


def test_append_places_rows_through_the_page_table():
    P, Hkv, ps, D = 6, 2, 4, 3
    kp = np.zeros((P, Hkv, ps, D)); vp = np.zeros((P, Hkv, ps, D))
    table = np.array([[5, 2, 0], [1, 3, -1]])
    ctx = np.array([7, 2])
    kn = np.arange(2 * 3 * Hkv * D, dtype=float).reshape(2, 3, Hkv, D) + 1
    kv.append(kp, vp, table, ctx, kn, -kn)
    # sequence 0, K1 = 3 -> positions 4, 5, 6: page 2 (table[0][1]) slots 0, 1, 2
    np.testing.assert_array_equal(kp[2, :, 0:3], np.transpose(kn[0], (1, 0, 2)))
    np.testing.assert_array_equal(vp[2, :, 0:3], -np.transpose(kn[0], (1, 0, 2)))
    # sequence 1: positions -1 (skipped), 0, 1 -> page 1 slots 0, 1
    np.testing.assert_array_equal(kp[1, :, 0:2], np.transpose(kn[1, 1:], (1, 0, 2)))
    assert kp[5].sum() == 0 and kp[0].sum() == 0


def test_commit_arithmetic():
    assert list(kv.commit([10, 10, 10], [0, 1, 2], 3)) == [8, 9, 10]
    assert list(kv.commit([10], [7], 3)) == [10]         # clamped: all drafts kept
    assert list(kv.commit([10], [-4], 3)) == [8]


def test_multi_step_matches_list_model():
    rng = np.random.default_rng(0)
    ps, Hkv, D, K1, steps = 4, 1, 2, 3, 6
    maxp, P = 16, 20
    table = np.array([rng.permutation(P)[:maxp]])
    kp = np.zeros((P, Hkv, ps, D)); vp = np.zeros((P, Hkv, ps, D))
    model = []                                          # committed rows, as a list
    ctx = np.array([0])
    for t in range(steps):
        rows = rng.standard_normal((1, K1, Hkv, D))
        ctx = ctx + K1
        kv.append(kp, vp, table, ctx, rows, rows)
        n = int(rng.integers(0, K1))
        ctx = kv.commit(ctx, [n], K1)
        model.extend(list(rows[0, :n + 1]))             # last committed token + n drafts
        got = kv.committed_rows(kp, table, ctx[0], 0)
        assert len(model) == ctx[0] == got.shape[0]
        np.testing.assert_array_equal(got, np.array(model))
