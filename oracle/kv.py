"""Oracle: KV-cache bookkeeping around the verify step (append, commit), on host arrays.

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).

What it models ([guide] §4 "실행 흐름", accept/reject step; [wiki] "투기적 디코딩의 기본 구조"):
the verify forward's K1 input positions are the last committed token and the k drafts; their
K/V are written to the cache; after n drafts are accepted the last committed token and those n
drafts stay and the k - n rejected ones are dropped (the correction or bonus token's K/V arrive
with the next step).

  append: for every sequence b and i < K1, the K/V rows of input position i go to cache
          position ctx_b - K1 + i (ctx already counts them), i.e. page table[b][pos // 16],
          slot pos % 16; positions outside the table or on an invalid page are skipped.
  commit: ctx_b <- ctx_b - (K1 - 1 - n_b), n_b clamped to [0, K1 - 1].
"""
from __future__ import annotations

import numpy as np


def append(k_pool, v_pool, page_table, ctx_lens, k_new, v_new):
    """In-place on numpy pools [P, Hkv, page, D]; k_new/v_new [B, K1, Hkv, D]."""
    P, Hkv, ps, D = k_pool.shape
    B, K1 = k_new.shape[:2]
    table = np.asarray(page_table)
    for b in range(B):
        for i in range(K1):
            pos = int(ctx_lens[b]) - K1 + i
            if pos < 0 or pos >= table.shape[1] * ps:
                continue
            page = int(table[b, pos // ps])
            if page < 0 or page >= P:
                continue
            k_pool[page, :, pos % ps, :] = k_new[b, i]
            v_pool[page, :, pos % ps, :] = v_new[b, i]


def commit(ctx_lens, n_accepted, K1: int):
    ctx = np.asarray(ctx_lens, dtype=np.int64).copy()
    n = np.clip(np.asarray(n_accepted, dtype=np.int64), 0, K1 - 1)
    return ctx - (K1 - 1 - n)


def committed_rows(pool, page_table, ctx, b):
    """The K (or V) rows of sequence b's committed positions 0 .. ctx-1, in order [ctx, Hkv, D]."""
    ps = pool.shape[2]
    pos = np.arange(int(ctx))
    pages = np.asarray(page_table)[b, pos // ps]
    return pool[pages, :, pos % ps, :]
