"""Oracle: lm-head contraction and the target's row distributions, float64.

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).

What it computes.  Each verified position needs the target's own distribution over the whole
vocabulary, against which the draft is compared ([guide] §4 "실행 흐름", parallel
verification: the target checks the draft sequence against its own distribution in one
forward).  The distribution comes from the vocab x hidden output table, which at a 256k
vocabulary is a large part of the cost ([guide] §1: the final 256k-vocabulary logit
projection; [damoang] section on the drafters' internals: the final logit computation is a
major bottleneck on the edge models).

  logits[r, v] = sum_h hidden[r, h] * W[v, h]
  p[r]         = softmax(logits[r] / T_r)                       for T_r > 0
  p[r]         = one-hot at the first index of max(logits[r])   for T_r <= 0 (greedy)

Readings: W is [V, H] row-major with no bias and no soft-capping; the temperature is a
per-row argument; greedy ties go to the lowest index.
"""
from __future__ import annotations

import numpy as np


def _f64(x) -> np.ndarray:
    if hasattr(x, "detach"):
        import torch
        x = x.detach().to("cpu").to(torch.float64).numpy()
    return np.asarray(x, dtype=np.float64)


def logits(hidden, weight, rows=None, vocab_rows=None) -> np.ndarray:
    """hidden [R, H] times weight[V, H] transposed: [R, V] float64.

    `rows` / `vocab_rows` restrict the product to a subset (index arrays), for sampled checks
    of large cases.
    """
    x = _f64(hidden)
    w = weight
    if vocab_rows is not None:
        w = w[vocab_rows]
    w = _f64(w)
    if rows is not None:
        x = x[rows]
    return x @ w.T


def probabilities(z, temperature) -> np.ndarray:
    """Row distributions of logits z [R, V] at per-row temperatures [R]."""
    z = np.asarray(z, dtype=np.float64)
    t = np.broadcast_to(np.asarray(temperature, dtype=np.float64), (z.shape[0],))
    p = np.zeros_like(z)
    for r in range(z.shape[0]):
        if t[r] > 0:
            e = np.exp((z[r] - z[r].max()) / t[r])
            p[r] = e / e.sum()
        else:
            p[r, int(np.argmax(z[r]))] = 1.0   # argmax returns the first maximal index
    return p
