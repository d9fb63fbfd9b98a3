"""Oracle: lossless accept / reject of the drafts, with the correction or bonus token.

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).

What the pages state.  The target verifies the k drafts in one forward; where a draft is
wrong, only the tokens before it are confirmed and the target generates the token at that
position itself, which keeps the output distributionally identical to decoding without a
drafter ([wiki] "투기적 디코딩의 기본 구조"; [guide] §4 "실행 흐름", accept/reject step:
drafts from the first rejected one on are discarded and the target generates the token).  If
the target agrees with the whole draft it accepts it and generates one more token in the same
forward ([geeknews] "MTP가 동작하는 방식"; [damoang] "추측적 해독은 어떻게 작동하는가").  The
pages name Leviathan et al. (2022) for the rule; restated:

  for i = 0 .. k-1:   accept d_i  iff  u_i < min(1, p_i(d_i) / q_i(d_i));  stop at the first
                      rejection; n = number of accepted drafts
  n < k:  emit y ~ norm(max(0, p_n - q_n))      (correction token)
  n = k:  emit y ~ p_k                           (bonus token)
  output: d_0 .. d_{n-1}, y

Exact evaluation (readings of what the pages leave open; the GPU path uses the same ones):
  * u_i is an fp32 value in [0, 1); the test is u_i * q < p, evaluated in float64, where the
    product of two fp32 values is exact, so the comparison is exact.  For q > 0 this equals
    u < min(1, p/q); for q = 0 it accepts iff p > 0.  A draft id outside [0, V) is rejected.
  * Sampling is an inverse CDF over integer weights, so the result does not depend on the
    order of any sum: P_j = floor(p_j * 2^38), Q_j = floor(q_j * 2^38); weights are
    max(0, P_j - Q_j) for a correction and P_j for a bonus; if every correction weight is 0
    the weights fall back to P_j.  With W = sum_j w_j and m = floor(u_k * 2^24), the
    threshold is floor(m * W / 2^24) and y is the smallest j whose running weight sum exceeds
    it.  (norm(.) is then implicit: the weights are never divided.)
  * Uniforms: u_0 .. u_{k-1} drive the k tests and u_k the one final draw, whatever n is.
"""
from __future__ import annotations

import numpy as np

FIXED_BITS = 38     # fixed-point scale of the integer sampling weights
UNIFORM_BITS = 24   # resolution of the sampling uniform


def _f64(x) -> np.ndarray:
    if hasattr(x, "detach"):
        import torch
        x = x.detach().to("cpu").to(torch.float64).numpy()
    return np.asarray(x, dtype=np.float64)


def accept_mask(draft, q, p, u) -> np.ndarray:
    """a[b, i] = [u_i * q_i(d_i) < p_i(d_i)] for i < k, bool [B, k].

    draft [B, k] int; q [B, k, V]; p [B, k+1, V] (or [B, k, V]); u [B, >=k].
    """
    draft = np.asarray(draft, dtype=np.int64)
    B, k = draft.shape
    V = q.shape[-1]
    a = np.zeros((B, k), dtype=bool)
    for b in range(B):
        for i in range(k):
            d = int(draft[b, i])
            if d < 0 or d >= V:
                continue
            a[b, i] = bool(accept_test(u[b, i], q[b, i, d], p[b, i, d]))
    return a


def accept_test(u, q_d, p_d):
    """[u * q(d) < p(d)] for fp32 u, q(d), p(d) (scalars or arrays), evaluated in float64.

    The float64 product of two fp32 values is exact (24 + 24 significant bits), so this is the
    exact comparison u < min(1, p/q) for q > 0, and p > 0 for q = 0.
    """
    u = np.asarray(u, dtype=np.float32).astype(np.float64)
    return u * np.float64(np.float32(q_d)) < np.float64(np.float32(p_d))


def first_rejection(a: np.ndarray) -> np.ndarray:
    """n[b] = index of the first False in a[b], or k if all are True."""
    B, k = a.shape
    n = np.full(B, k, dtype=np.int64)
    for b in range(B):
        for i in range(k):
            if not a[b, i]:
                n[b] = i
                break
    return n


def integer_weights(row) -> np.ndarray:
    """floor(row * 2^38) as int64; exact for fp32 inputs in [0, 1]."""
    r = _f64(row)
    return np.floor(r * float(2 ** FIXED_BITS)).astype(np.int64)


def sample_weights(p_row, q_row=None) -> np.ndarray:
    """Correction weights max(0, P - Q) (bonus: P), with the all-zero fallback to P."""
    P = integer_weights(p_row)
    if q_row is None:
        return P
    w = np.maximum(P - integer_weights(q_row), 0)
    return w if int(w.sum()) > 0 else P


def uniform_index(u: float) -> int:
    """m = floor(u * 2^24), clamped to [0, 2^24 - 1]."""
    m = int(np.floor(np.float64(np.float32(u)) * float(2 ** UNIFORM_BITS)))
    return min(max(m, 0), 2 ** UNIFORM_BITS - 1)


def sample_index(weights: np.ndarray, m):
    """Smallest j with sum_{i<=j} w_i > floor(m * W / 2^24), W = sum w (exact integers).

    m is one integer in [0, 2^24) or an array of them (then an array of indices is returned).
    m * W < 2^24 * 2^40 fits uint64.  If W = 0 (no entry reaches 2^-38, not a distribution)
    the index is 0.
    """
    w = np.asarray(weights, dtype=np.int64)
    running = np.cumsum(w).astype(np.uint64)
    total = int(running[-1]) if running.size else 0
    scalar = np.ndim(m) == 0
    m = np.atleast_1d(np.asarray(m, dtype=np.uint64))
    if total == 0:
        y = np.zeros(m.shape, dtype=np.int64)
    else:
        t = (m * np.uint64(total)) >> np.uint64(UNIFORM_BITS)
        y = np.searchsorted(running, t, side="right").astype(np.int64)
    return int(y[0]) if scalar else y


def verify_accept(draft, q, p, u):
    """Accept counts n [B] and emitted tokens [B, k+1] (padding -1).

    draft [B, k]; q [B, k, V] drafter probabilities; p [B, k+1, V] target probabilities;
    u [B, k+1] uniforms.  p and q are the fp32 arrays the GPU consumes (converted exactly).
    """
    draft = np.asarray(draft, dtype=np.int64)
    B, k = draft.shape
    u = np.asarray(u, dtype=np.float32)
    n = first_rejection(accept_mask(draft, q, p, u)) if k > 0 else np.zeros(B, np.int64)
    tokens = np.full((B, k + 1), -1, dtype=np.int64)
    for b in range(B):
        nb = int(n[b])
        w = sample_weights(p[b, nb], q[b, nb] if nb < k else None)
        y = sample_index(w, uniform_index(u[b, k]))
        tokens[b, :nb] = draft[b, :nb]
        tokens[b, nb] = y
    return n, tokens


def acceptance_probability(p_row, q_row) -> float:
    """Closed form of P(accept) at one position when d ~ q: sum_v min(p(v), q(v)).

    (sum_v q(v) * min(1, p(v)/q(v)); the identity min(p, q) + max(0, p - q) = p is what makes
    the correction draw restore p exactly.)
    """
    return float(np.minimum(_f64(p_row), _f64(q_row)).sum())
