"""Seeded synthetic inputs for the verify step.

Both the fp64 oracle and the HIP library read what these functions produce; the module holds
random-number recipes only (no attention, no softmax, no acceptance arithmetic).  Every draw
is keyed by (workload seed, step, stream[, layer]) through numpy's SeedSequence, so any input
can be regenerated alone:

    stream 0  queries and the paged K/V pools
    stream 1  lm-head hidden states and the vocab x hidden table
    stream 2  base logits
    stream 3  logit noise
    stream 4  drafted tokens
    stream 5  acceptance / sampling uniforms
    stream 6  context lengths and the page permutation

Small arrays come from numpy's Philox generator.  Bulk tensors (K/V pools, the lm-head table)
come from torch's generator on the device they are needed on, so a multi-GB table never has
to cross PCIe to be created; a test that needs them on the host copies them once.
"""
from __future__ import annotations

import math

import numpy as np

from .configs import Workload, noise_sigma

STREAM_QKV, STREAM_LMHEAD, STREAM_BASE, STREAM_NOISE = 0, 1, 2, 3
STREAM_DRAFT, STREAM_UNIFORM, STREAM_LAYOUT, STREAM_DRAFTER_Q = 4, 5, 6, 7


def seed_words(w: Workload, stream: int, step: int = 0, sub: int = 0) -> np.random.SeedSequence:
    return np.random.SeedSequence([int(w.seed), int(step), int(stream), int(sub)])


def rng(w: Workload, stream: int, step: int = 0, sub: int = 0) -> np.random.Generator:
    return np.random.Generator(np.random.Philox(seed_words(w, stream, step, sub)))


def torch_seed(w: Workload, stream: int, step: int = 0, sub: int = 0) -> int:
    a, b = seed_words(w, stream, step, sub).generate_state(2, dtype=np.uint32)
    return int((int(a) << 31) ^ int(b)) & ((1 << 63) - 1)


# ----------------------------------------------------------------------------- layout

def context_lengths(w: Workload, step: int = 0) -> np.ndarray:
    """Tokens in each sequence's cache, the K1 positions being verified included."""
    kind, *args = w.ctx.split(":")
    g = rng(w, STREAM_LAYOUT, step, 0)
    if kind == "fixed":
        out = np.full(w.batch, int(args[0]))
    elif kind == "uniform":
        lo, hi = int(args[0]), int(args[1])
        out = g.integers(lo, hi + 1, size=w.batch)
    elif kind == "loguniform":
        lo, hi = int(args[0]), int(args[1])
        out = np.floor(np.exp(g.uniform(math.log(lo), math.log(hi), size=w.batch)))
    else:
        raise ValueError(w.ctx)
    return np.maximum(out, w.k1).astype(np.int32)


def max_context(w: Workload) -> int:
    kind, *args = w.ctx.split(":")
    return int(args[0]) if kind == "fixed" else int(args[1])


def page_tables(w: Workload, ctx_lens: np.ndarray, step: int = 0, spare: float = 0.1,
                max_pages: int | None = None):
    """Page table [B, max_pages] int32 and the pool size P.

    All sequences draw their pages from one pool that holds exactly the pages they need plus
    `spare` unused ones; the physical page of every logical page is a seeded random
    permutation of the pool.  A contiguous cache (w.paged False) is the identity table.
    Unused table entries hold -1.
    """
    ps = w.page_size
    need = [(int(c) + ps - 1) // ps for c in ctx_lens]
    if max_pages is None:
        max_pages = (max_context(w) + ps - 1) // ps
    total = int(sum(need))
    table = np.full((w.batch, max_pages), -1, dtype=np.int32)
    if not w.paged:
        base = 0
        for b, n in enumerate(need):
            table[b, :n] = np.arange(base, base + n, dtype=np.int32)
            base += n
        return table, total
    pool = total + int(math.ceil(spare * total))
    perm = rng(w, STREAM_LAYOUT, step, 1).permutation(pool).astype(np.int32)
    base = 0
    for b, n in enumerate(need):
        table[b, :n] = perm[base:base + n]
        base += n
    return table, pool


# ----------------------------------------------------------------------------- tensors

def _torch_dtype(name: str):
    import torch
    return {"f32": torch.float32, "bf16": torch.bfloat16}[name]


def normal_tensor(shape, seed: int, device, dtype: str, std: float = 1.0):
    """N(0, std^2) samples, drawn in fp32 by torch's generator on `device`, then cast."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    t = torch.randn(tuple(shape), generator=g, device=device, dtype=torch.float32)
    if std != 1.0:
        t.mul_(std)
    return t.to(_torch_dtype(dtype))


def queries(w: Workload, layer: int, device="cpu", step: int = 0):
    L = w.layers[layer]
    return normal_tensor((w.batch, w.k1, L.hq, L.head_dim),
                         torch_seed(w, STREAM_QKV, step, 3 * layer), device, w.dtype)


def drafter_queries(w: Workload, layer: int, hq: int, draft_step: int, device="cpu",
                    step: int = 0):
    """Queries [B, 1, hq, D] of one drafter step that reads layer `layer`'s KV pool: one query
    position per sequence, the drafter's own head count over the target's KV heads."""
    L = w.layers[layer]
    return normal_tensor((w.batch, 1, hq, L.head_dim),
                         torch_seed(w, STREAM_DRAFTER_Q, step, 64 * layer + draft_step), device,
                         w.dtype)


def kv_pools(w: Workload, layer: int, num_pages: int, device="cpu", step: int = 0):
    """K and V pools, each [P, Hkv, page_size, head_dim], entries N(0, 1)."""
    L = w.layers[layer]
    shape = (num_pages, L.hkv, w.page_size, L.head_dim)
    k = normal_tensor(shape, torch_seed(w, STREAM_QKV, step, 3 * layer + 1), device, w.dtype)
    v = normal_tensor(shape, torch_seed(w, STREAM_QKV, step, 3 * layer + 2), device, w.dtype)
    return k, v


def hidden_states(w: Workload, device="cpu", step: int = 0, rows: int | None = None):
    """Final hidden states entering the lm-head, [R, H], entries N(0, 1)."""
    r = w.rows if rows is None else rows
    return normal_tensor((r, w.hidden), torch_seed(w, STREAM_LMHEAD, step, 0), device, w.dtype)


def lm_head_table(w: Workload, device="cpu", step: int = 0):
    """Vocab x hidden output table [V, H], entries N(0, 1/H)."""
    return normal_tensor((w.vocab, w.hidden), torch_seed(w, STREAM_LMHEAD, step, 1), device,
                         w.dtype, std=1.0 / math.sqrt(w.hidden))


def drafter_hidden_noise(w: Workload, device="cpu", step: int = 0, rows: int | None = None):
    """N(0, 1) perturbation of the hidden states, [R, H], for a drafter sharing the table."""
    r = w.rows if rows is None else rows
    return normal_tensor((r, w.hidden), torch_seed(w, STREAM_NOISE, step, 7), device, "f32")


# ----------------------------------------------------------------------------- logits

def logit_pairs(w: Workload, step: int = 0, vocab: int | None = None, batch: int | None = None):
    """Drafter logits z_q [B, k, V] and target logits z_p [B, K1, V], float64.

    "gauss": z_q ~ N(0, 1); z_p = z_q + N(0, sigma^2) on the first k rows, and the bonus row
             of z_p is its own N(0, 1 + sigma^2) draw built the same way from a base row.
    "zipf":  per row a base b_j = -1.1 ln(rank_j) over a seeded permutation of the ranks
             1..V; z_q = b + N(0, sigma^2) and z_p = b + N(0, sigma^2), independent noise.
    """
    V = w.vocab if vocab is None else vocab
    B = w.batch if batch is None else batch
    sigma = noise_sigma(w)
    gb = rng(w, STREAM_BASE, step)
    gn = rng(w, STREAM_NOISE, step)
    if w.logit_recipe == "gauss":
        base = gb.standard_normal((B, w.k1, V))
        z_q = base[:, : w.k].copy()
        z_p = base + sigma * gn.standard_normal((B, w.k1, V))
    elif w.logit_recipe == "zipf":
        ranks = np.empty((B, w.k1, V))
        for b in range(B):
            for i in range(w.k1):
                ranks[b, i] = gb.permutation(V) + 1.0
        base = -1.1 * np.log(ranks)
        z_q = base[:, : w.k] + sigma * gn.standard_normal((B, w.k, V))
        z_p = base + sigma * gn.standard_normal((B, w.k1, V))
    else:
        raise ValueError(w.logit_recipe)
    return z_q, z_p


def temperatures(w: Workload, batch: int | None = None) -> np.ndarray:
    B = w.batch if batch is None else batch
    return np.array([w.temperature_of(b) for b in range(B)], dtype=np.float32)


def row_temperatures(w: Workload, batch: int | None = None) -> np.ndarray:
    """Temperature of every lm-head row (b-major, K1 rows per sequence)."""
    return np.repeat(temperatures(w, batch), w.k1).astype(np.float32)


def uniforms(w: Workload, step: int = 0, batch: int | None = None) -> np.ndarray:
    """[B, K1] float32 uniforms in [0, 1): k acceptance tests plus one sampling draw.

    numpy's float32 draw keeps 24 random bits, so every value is a multiple of 2^-24.
    """
    B = w.batch if batch is None else batch
    return rng(w, STREAM_UNIFORM, step).random((B, w.k1), dtype=np.float32)


def draw_drafts(w: Workload, q: np.ndarray, temps: np.ndarray, step: int = 0) -> np.ndarray:
    """Drafted tokens [B, k] int32 drawn from the drafter's distributions q [B, k, V].

    Greedy sequences (temperature 0) take the first maximal entry; the others are inverse-CDF
    draws on float64 running sums of q.
    """
    B, k, V = q.shape
    g = rng(w, STREAM_DRAFT, step)
    u = g.random((B, k))
    out = np.empty((B, k), dtype=np.int32)
    for b in range(B):
        for i in range(k):
            row = np.asarray(q[b, i], dtype=np.float64)
            if temps[b] <= 0:
                out[b, i] = int(np.argmax(row))
            else:
                c = np.cumsum(row)
                j = int(np.searchsorted(c, u[b, i] * c[-1], side="right"))
                out[b, i] = min(j, V - 1)
    return out
