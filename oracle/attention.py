"""Oracle: (k+1)-query causal grouped-query attention over a paged KV cache, float64.

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).

What it computes.  The target scores the k drafted tokens and the bonus position in one
forward pass ([wiki] "투기적 디코딩의 기본 구조": the target processes the k proposed tokens at
once; [guide] §4 "실행 흐름", parallel verification step).  The K/V of all those positions are
already in the shared cache ([guide] §1 table, KV-cache row: the drafter and the target share
one KV-cache pool), so each verified position is an ordinary causal query against the cache:

  query i of sequence b sits at position t = ctx_b - K1 + i (the last K1 cache positions);
  it sees key positions s with lo <= s <= t, where lo = 0 for a global layer and
  lo = max(0, t - window + 1) for a sliding-window layer (window keys, itself included);
  head h reads KV head floor(h / G), G = Hq / Hkv (contiguous query-head groups);
  o = sum_s softmax_s(scale * <q, k_s>) v_s.

Heads of dim 256 with a sliding window and heads of dim 512 attending globally are the two
layer kinds of the target ([guide] §7 settings table: local 256 / global 512 head dims).

Readings of points the pages leave open:
  * key position s lives at physical page page_table[b, s // page_size], slot s % page_size,
    of pools laid out [P, Hkv, page_size, D];
  * scale is an argument (1/sqrt(D) in every workload); no soft-capping, no QK norm;
  * a page id outside [0, P) makes the keys on it invisible, and a query with no visible key
    returns zeros.
"""
from __future__ import annotations

import numpy as np


def _f64(x) -> np.ndarray:
    if hasattr(x, "detach"):
        x = x.detach().to("cpu")
        import torch
        x = x.to(torch.float64).numpy()
    return np.asarray(x, dtype=np.float64)


def visible_range(ctx: int, k1: int, i: int, window: int):
    """Key positions [lo, t] seen by query i of a sequence with ctx cached tokens."""
    t = ctx - k1 + i
    lo = max(0, t - window + 1) if window > 0 else 0
    return lo, t


def verify_attention(q, k_pool, v_pool, page_table, ctx_lens, window: int, scale: float,
                     rows=None) -> np.ndarray:
    """Attention output [B, K1, Hq, D] in float64.

    q [B, K1, Hq, D]; k_pool, v_pool [P, Hkv, page_size, D]; page_table [B, max_pages];
    ctx_lens [B].  `rows`, if given, is an iterable of (b, i) pairs to compute; the other
    entries of the result are left as NaN (used to sample large cases).
    """
    q = _f64(q)
    kp = _f64(k_pool)
    vp = _f64(v_pool)
    table = np.asarray(page_table, dtype=np.int64)
    ctx_lens = np.asarray(ctx_lens, dtype=np.int64)
    B, K1, Hq, D = q.shape
    P, Hkv, ps, _ = kp.shape
    G = Hq // Hkv
    kv_head = np.arange(Hq) // G
    out = np.full((B, K1, Hq, D), np.nan)
    if rows is None:
        rows = [(b, i) for b in range(B) for i in range(K1)]
    for b, i in rows:
        lo, t = visible_range(int(ctx_lens[b]), K1, i, window)
        pos = np.arange(lo, t + 1)
        pos = pos[(pos >= 0) & (pos // ps < table.shape[1])]
        pages = table[b, pos // ps]
        ok = (pages >= 0) & (pages < P)
        pos, pages = pos[ok], pages[ok]
        if pos.size == 0:
            out[b, i] = 0.0
            continue
        slots = pos % ps
        keys = kp[pages, :, slots, :]          # [n, Hkv, D]
        vals = vp[pages, :, slots, :]
        for h in range(Hq):
            g = kv_head[h]
            scores = scale * (keys[:, g, :] @ q[b, i, h])
            w = np.exp(scores - scores.max())
            out[b, i, h] = (w / w.sum()) @ vals[:, g, :]
    return out
