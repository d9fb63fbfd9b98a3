"""Oracle: the counter-based generator Philox4x32-10 and the verify step's uniforms drawn from it.

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).

Philox4x32-10 (Salmon, Moraes, Dror, Shaw, "Parallel Random Numbers: As Easy as 1, 2, 3",
SC'11): a 128-bit counter (four 32-bit words) and a 64-bit key (two words) go through ten
rounds; each round multiplies counter words 0 and 2 by the published constants 0xD2511F53 and
0xCD9E8D57 into 64-bit products, and the new counter is
  (hi(word 2 product) ^ word 1 ^ key 0, lo(word 2 product),
   hi(word 0 product) ^ word 3 ^ key 1, lo(word 0 product));
between rounds the key words grow by the Weyl constants 0x9E3779B9 and 0xBB67AE85 (mod 2^32).

Uniforms of the verify step (the accept rule needs u in [0, 1) for the k tests and the one draw
of every sequence; the pages name Leviathan et al. for the rule and say nothing about the
generator, so this is a reading): u[b][i] = (word (i mod 4) of Philox4x32-10 at counter
(i div 4, b, offset low 32 bits, offset high 32 bits) and key (seed low, seed high)) >> 8,
times 2^-24 — a multiple of 2^-24, as the accept step expects.
"""
from __future__ import annotations

import numpy as np

M0, M1 = 0xD2511F53, 0xCD9E8D57
W0, W1 = 0x9E3779B9, 0xBB67AE85
MASK = 0xFFFFFFFF


def philox4x32_10(counter, key):
    """Four output words (Python ints) for counter (c0, c1, c2, c3) and key (k0, k1)."""
    c0, c1, c2, c3 = (int(x) & MASK for x in counter)
    k0, k1 = (int(x) & MASK for x in key)
    for r in range(10):
        if r:
            k0 = (k0 + W0) & MASK
            k1 = (k1 + W1) & MASK
        p0 = M0 * c0
        p1 = M1 * c2
        c0, c1, c2, c3 = ((p1 >> 32) ^ c1 ^ k0, p1 & MASK, (p0 >> 32) ^ c3 ^ k1, p0 & MASK)
    return c0, c1, c2, c3


def uniforms(seed: int, offset: int, B: int, K1: int) -> np.ndarray:
    """u [B, K1] float32 of the reading above."""
    u = np.empty((B, K1), np.float32)
    key = (seed & MASK, (seed >> 32) & MASK)
    for b in range(B):
        for blk in range((K1 + 3) // 4):
            words = philox4x32_10((blk, b, offset & MASK, (offset >> 32) & MASK), key)
            for j in range(4):
                i = 4 * blk + j
                if i < K1:
                    u[b, i] = np.float32((words[j] >> 8) * 2.0 ** -24)
    return u
