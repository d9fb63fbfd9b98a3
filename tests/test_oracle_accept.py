"""Pins of the oracle's accept / reject and correction / bonus draw (oracle/accept.py).

1. Lossless, by exhaustive enumeration (the pages' claim that the output is distributionally
   identical to decoding with the target alone): with tiny vocabularies and random dyadic
   target / drafter tables indexed by the prefix, the exact measure of the uniforms leading to
   each outcome of the oracle's decision and draw is taken (all 2^24 uniform values, or
   equivalently the bisected boundaries of those monotone functions, checked against the full
   enumeration), composed over verify steps until N tokens are out, and the
   resulting distribution over V^N must equal prod_t p(y_t | y_<t) within the 2^-24
   quantisation of the uniforms.
2. Closed form: P(accept at a position) = sum_v min(p, q), by exact enumeration and by Monte
   Carlo; E[n + 1] = (1 - a^(k+1)) / (1 - a) for positions with equal acceptance a.
3. Greedy: with temperature 0, n is the longest prefix where the draft equals the target's
   argmax and the emitted token is the target's argmax at n (an independent routine).
4. Exactness of the draw: brute-force inverse CDF, exact counts of every outcome over all
   2^24 uniforms, strict comparison, q(d) = 0, out-of-range drafts, empty residual.
"""
import itertools
import math
import zlib
from functools import lru_cache

import numpy as np
import pytest

import oracle
from oracle.accept import accept_test, sample_weights, uniform_index, acceptance_probability

M_ALL = np.arange(2 ** 24, dtype=np.uint64)
U_ALL = (np.arange(2 ** 24, dtype=np.float64) / 2 ** 24).astype(np.float32)


def dyadic_dist(rng, V, bits=10):
    """Random distribution whose entries are multiples of 2^-bits, all entries > 0."""
    cuts = np.sort(rng.choice(np.arange(1, 2 ** bits), size=V - 1, replace=False))
    parts = np.diff(np.concatenate([[0], cuts, [2 ** bits]]))
    return (parts / 2 ** bits).astype(np.float32)


class Tables:
    def __init__(self, V, seed):
        self.V, self.seed = V, seed
        self.cache = {}

    def get(self, who, prefix):
        key = (who, prefix)
        if key not in self.cache:
            h = zlib.crc32(repr((self.seed, who, prefix)).encode())
            self.cache[key] = dyadic_dist(np.random.default_rng(h), self.V)
        return self.cache[key]


def accept_measure_full(qd: float, pd: float) -> float:
    """Exact measure of the uniforms the oracle accepts: all 2^24 values probed."""
    return float(accept_test(U_ALL, qd, pd).sum()) / 2 ** 24


def draw_measure_full(weights: np.ndarray) -> np.ndarray:
    ys = oracle.sample_index(weights, M_ALL)
    return np.bincount(ys, minlength=weights.size) / 2 ** 24


def _first_m(pred):
    """Smallest m in [0, 2^24] with pred(m) true, for pred monotone false -> true."""
    lo, hi = 0, 2 ** 24
    while lo < hi:
        mid = (lo + hi) // 2
        if pred(mid):
            hi = mid
        else:
            lo = mid + 1
    return lo


@lru_cache(maxsize=None)
def accept_measure(qd: float, pd: float) -> float:
    """Same measure, by bisecting the oracle's decision (which rejects from some u on)."""
    rej = lambda m: not bool(accept_test(np.float32(m / 2 ** 24), qd, pd))  # noqa: E731
    b = _first_m(lambda m: m >= 2 ** 24 or rej(m))
    assert b == 0 or not rej(b - 1)
    return b / 2 ** 24


_draw_cache = {}


def draw_measure(weights: np.ndarray) -> np.ndarray:
    """Same measure of every drawn index, by bisecting the oracle's (monotone) draw."""
    key = weights.tobytes()
    if key not in _draw_cache:
        V = weights.size
        y = lambda m: oracle.sample_index(weights, m) if m < 2 ** 24 else V  # noqa: E731
        starts = [0] + [_first_m(lambda m, j=j: y(m) >= j) for j in range(1, V)] + [2 ** 24]
        for j in range(1, V):
            assert starts[j] == 0 or y(starts[j] - 1) < j
        _draw_cache[key] = np.diff(np.array(starts, dtype=np.float64)) / 2 ** 24
    return _draw_cache[key]


def test_bisection_measures_match_full_enumeration():
    rng = np.random.default_rng(4)
    for _ in range(3):
        p = dyadic_dist(rng, 3)
        q = dyadic_dist(rng, 3)
        for d in range(3):
            assert accept_measure(float(q[d]), float(p[d])) == \
                accept_measure_full(float(q[d]), float(p[d]))
        w = sample_weights(p, q)
        np.testing.assert_array_equal(draw_measure(w), draw_measure_full(w))


def one_step(tab, prefix, k):
    """Distribution of the tokens one verify step emits from `prefix`: {tuple: prob}."""
    V = tab.V
    out = {}
    for draft in itertools.product(range(V), repeat=k):
        pd = 1.0
        for i in range(k):
            pd *= float(tab.get("q", prefix + draft[:i])[draft[i]])
        if pd == 0:
            continue
        reach = pd
        for n in range(k + 1):
            ctxn = prefix + draft[:n]
            if n < k:
                qd = float(tab.get("q", ctxn)[draft[n]])
                a = accept_measure(qd, float(tab.get("p", ctxn)[draft[n]]))
                p_stop = reach * (1 - a)
                w = sample_weights(tab.get("p", ctxn), tab.get("q", ctxn))
            else:
                p_stop = reach
                w = sample_weights(tab.get("p", ctxn))
            if p_stop > 0:
                ys = draw_measure(w)
                for y in range(V):
                    if ys[y] > 0:
                        key = draft[:n] + (y,)
                        out[key] = out.get(key, 0.0) + p_stop * ys[y]
            if n < k:
                reach *= a
    return out


def emitted_distribution(tab, k, N, prefix=()):
    if N <= 0:
        return {(): 1.0}
    out = {}
    for seq, pr in one_step(tab, prefix, k).items():
        seq = seq[:N]
        rest = emitted_distribution(tab, k, N - len(seq), prefix + seq)
        for tail, pt in rest.items():
            key = seq + tail
            out[key] = out.get(key, 0.0) + pr * pt
    return out


@pytest.mark.parametrize("V,k,seed", [(2, 1, 0), (2, 2, 1), (3, 2, 2), (2, 3, 3), (4, 1, 5)])
def test_lossless_by_enumeration(V, k, seed):
    tab = Tables(V, seed)
    N = k + 1
    got = emitted_distribution(tab, k, N)
    worst = 0.0
    for seq in itertools.product(range(V), repeat=N):
        target = 1.0
        for t in range(N):
            target *= float(tab.get("p", seq[:t])[seq[t]])
        worst = max(worst, abs(got.get(seq, 0.0) - target))
    assert abs(sum(got.values()) - 1.0) < 1e-9
    # each decision and draw is quantised to 2^-24; a few steps of them compose
    assert worst < 64 * 2 ** -24, worst


def test_enumeration_detects_a_wrong_residual():
    """A plausible mistake (resampling from the drafter's excess q - p) breaks losslessness."""
    V, k = 2, 1
    tab = Tables(V, 11)
    p0, q0 = tab.get("p", ()), tab.get("q", ())
    total_good, total_bad = np.zeros(V), np.zeros(V)
    for d in range(V):
        a = accept_measure(float(q0[d]), float(p0[d]))
        good = draw_measure(sample_weights(p0, q0))
        bad = draw_measure(sample_weights(q0, p0))
        total_good[d] += q0[d] * a
        total_bad[d] += q0[d] * a
        total_good += q0[d] * (1 - a) * good
        total_bad += q0[d] * (1 - a) * bad
    assert np.abs(total_good - p0).max() < 4 * 2 ** -24
    assert np.abs(total_bad - p0).max() > 1e-3


def test_acceptance_closed_form_by_exact_enumeration():
    rng = np.random.default_rng(5)
    V = 40
    for trial in range(5):
        p = rng.dirichlet(np.ones(V)).astype(np.float32)
        q = rng.dirichlet(np.ones(V)).astype(np.float32)
        measure = accept_measure_full if trial == 0 else accept_measure
        exact = sum(float(q[d]) * measure(float(q[d]), float(p[d])) for d in range(V))
        assert abs(exact - acceptance_probability(p, q)) < V * 2 ** -24


def test_acceptance_closed_form_by_monte_carlo():
    rng = np.random.default_rng(6)
    V, trials = 64, 1_000_000
    p = rng.dirichlet(np.ones(V) * 0.5).astype(np.float32)
    q = rng.dirichlet(np.ones(V) * 0.5).astype(np.float32)
    d = rng.choice(V, size=trials, p=q.astype(np.float64) / q.sum())
    u = rng.random(trials, dtype=np.float32)
    rate = accept_test(u, q[d], p[d]).mean()
    a = acceptance_probability(p, q)
    sd = math.sqrt(a * (1 - a) / trials)
    assert abs(rate - a) < 4 * sd + V * 2 ** -24


def test_mean_emitted_tokens_closed_form():
    """Positions with the same (p, q): E[n + 1] = (1 - a^(k+1)) / (1 - a)."""
    rng = np.random.default_rng(8)
    V, B, k = 12, 20000, 2
    p1 = rng.dirichlet(np.ones(V)).astype(np.float32)
    q1 = rng.dirichlet(np.ones(V)).astype(np.float32)
    p = np.broadcast_to(p1, (B, k + 1, V))
    q = np.broadcast_to(q1, (B, k, V))
    draft = rng.choice(V, size=(B, k), p=q1.astype(np.float64) / q1.sum()).astype(np.int32)
    u = rng.random((B, k + 1), dtype=np.float32)
    n, tokens = oracle.verify_accept(draft, q, p, u)
    a = acceptance_probability(p1, q1)
    mean = (1 - a ** (k + 1)) / (1 - a)
    sd = np.std(n + 1) / math.sqrt(B)
    assert abs(np.mean(n + 1) - mean) < 4 * sd
    # tokens: accepted drafts, then one sampled token, then padding
    for b in range(50):
        nb = n[b]
        assert list(tokens[b, :nb]) == list(draft[b, :nb])
        assert 0 <= tokens[b, nb] < V
        assert (tokens[b, nb + 1:] == -1).all()


def test_greedy_equals_argmax_prefix_matching():
    rng = np.random.default_rng(9)
    B, k, V = 200, 4, 7
    zq = rng.integers(0, 5, size=(B, k, V)).astype(np.float64)
    zp = zq + (rng.random((B, k + 1, V))[:, :k] < 0.15) * rng.integers(-3, 4, size=(B, k, V))
    zp = np.concatenate([zp, rng.integers(0, 5, size=(B, 1, V))], axis=1)
    q = oracle.probabilities(zq.reshape(-1, V), 0.0).reshape(B, k, V).astype(np.float32)
    p = oracle.probabilities(zp.reshape(-1, V), 0.0).reshape(B, k + 1, V).astype(np.float32)
    draft = np.argmax(zq, axis=2).astype(np.int32)
    u = rng.random((B, k + 1), dtype=np.float32)
    n, tokens = oracle.verify_accept(draft, q, p, u)

    def greedy(drafts, target_rows):
        j = 0
        while j < len(drafts) and drafts[j] == int(np.argmax(target_rows[j])):
            j += 1
        return j, int(np.argmax(target_rows[j]))

    for b in range(B):
        nb, y = greedy(draft[b], zp[b])
        assert n[b] == nb and tokens[b, nb] == y


def test_inverse_cdf_brute_force():
    rng = np.random.default_rng(10)
    for _ in range(200):
        w = rng.integers(0, 5, size=rng.integers(1, 9))
        if w.sum() == 0:
            continue
        m = int(rng.integers(0, 2 ** 24))
        t = (m * int(w.sum())) // 2 ** 24
        j, acc = 0, int(w[0])
        while acc <= t:
            j += 1
            acc += int(w[j])
        assert oracle.sample_index(w, m) == j


def test_draw_counts_over_all_uniforms():
    """#{m : y = j} = ceil(C_j 2^24 / W) - ceil(C_{j-1} 2^24 / W), C the running sums."""
    w = np.array([5, 0, 7, 1, 3], dtype=np.int64) * 12345
    counts = np.bincount(oracle.sample_index(w, M_ALL), minlength=w.size)
    C = np.concatenate([[0], np.cumsum(w)])
    W = int(C[-1])
    expect = [-(-int(C[j + 1]) * 2 ** 24 // W) - (-(-int(C[j]) * 2 ** 24 // W))
              for j in range(w.size)]
    assert list(counts) == expect
    assert counts[1] == 0


def test_decision_edge_cases():
    # strict comparison: u * q == p rejects
    assert not accept_test(np.float32(0.5), 0.5, 0.25)
    assert accept_test(np.float32(0.5) - np.float32(2 ** -24), 0.5, 0.25)
    # q(d) = 0: accept iff p(d) > 0
    assert accept_test(np.float32(0.99), 0.0, 1e-30)
    assert not accept_test(np.float32(0.0), 0.0, 0.0)
    # out-of-range drafts are rejected; uniforms index from floor(u * 2^24)
    p = np.full((1, 2, 4), 0.25, np.float32)
    q = np.full((1, 1, 4), 0.25, np.float32)
    n, tokens = oracle.verify_accept(np.array([[7]]), q, p, np.array([[0.0, 0.0]], np.float32))
    assert n[0] == 0 and tokens[0, 0] == 0 and tokens[0, 1] == -1
    assert uniform_index(np.float32(1.0) - np.float32(2 ** -24)) == 2 ** 24 - 1


def test_empty_residual_falls_back_to_target():
    p = np.array([0.5, 0.25, 0.25], np.float32)
    w = sample_weights(p, p.copy())
    assert list(w) == list(oracle.integer_weights(p))
    # p == q exactly: rejection has probability 0, and the fallback draws from p
    assert accept_measure(0.25, 0.25) == 1.0


def test_k_zero_is_plain_sampling():
    p = np.array([[[0.125, 0.5, 0.375]]], np.float32)
    q = np.zeros((1, 0, 3), np.float32)
    ys = [oracle.verify_accept(np.zeros((1, 0), np.int32), q, p,
                               np.array([[u]], np.float32))[1][0, 0]
          for u in (0.0, 0.124, 0.125, 0.6249, 0.625, 0.99)]
    assert ys == [0, 0, 1, 1, 2, 2]
