"""Pins of the oracle's lm-head and row distributions (oracle/lm_head.py):

* hand-computed products of small integer tables, and a pure-Python triple loop on a tiny
  random case (brute force);
* softmax closed forms: logits (0, ln 2, ln 3) give (1/6, 2/6, 3/6); temperature divides the
  logits; huge logits do not overflow; rows sum to one;
* greedy rows: one-hot at the first maximal index; the low-temperature limit approaches it.
"""
import math

import numpy as np

import oracle


def test_small_integer_product():
    hidden = np.array([[1.0, 2.0], [-1.0, 0.5]])
    table = np.array([[3.0, 4.0], [5.0, 6.0], [0.0, -1.0]])
    np.testing.assert_array_equal(oracle.logits(hidden, table),
                                  [[11.0, 17.0, -2.0], [-1.0, -2.0, -0.5]])


def test_brute_force_triple_loop():
    rng = np.random.default_rng(1)
    R, H, V = 3, 7, 11
    x = rng.standard_normal((R, H))
    w = rng.standard_normal((V, H))
    ref = [[sum(x[r][h] * w[v][h] for h in range(H)) for v in range(V)] for r in range(R)]
    np.testing.assert_allclose(oracle.logits(x, w), ref, rtol=0, atol=1e-12)
    sub = oracle.logits(x, w, rows=[2], vocab_rows=[4, 9])
    np.testing.assert_allclose(sub, [[ref[2][4], ref[2][9]]], atol=1e-12)


def test_softmax_closed_forms():
    z = np.array([[0.0, math.log(2), math.log(3)],
                  [0.0, 2 * math.log(2), 2 * math.log(3)],
                  [1000.0, 1000.0 + math.log(3), -1000.0]])
    p = oracle.probabilities(z, [1.0, 2.0, 1.0])
    np.testing.assert_allclose(p[0], [1 / 6, 2 / 6, 3 / 6], atol=1e-15)
    np.testing.assert_allclose(p[1], [1 / 6, 2 / 6, 3 / 6], atol=1e-15)
    np.testing.assert_allclose(p[2], [0.25, 0.75, 0.0], atol=1e-15)


def test_rows_sum_to_one_and_shift_invariance():
    rng = np.random.default_rng(2)
    z = rng.standard_normal((4, 1000)) * 3
    t = [1.0, 0.7, 2.5, 1e-2]
    p = oracle.probabilities(z, t)
    np.testing.assert_allclose(p.sum(axis=1), 1.0, atol=1e-12)
    np.testing.assert_allclose(oracle.probabilities(z + 17.0, t), p, atol=1e-14)


def test_greedy_rows_and_low_temperature_limit():
    z = np.array([[1.0, 3.0, 3.0, 2.0], [5.0, -1.0, 0.0, 4.0]])
    p = oracle.probabilities(z, [0.0, 0.0])
    np.testing.assert_array_equal(p, [[0, 1, 0, 0], [1, 0, 0, 0]])
    cold = oracle.probabilities(z[1:], [1e-3])
    assert cold[0, 0] > 1 - 1e-12
