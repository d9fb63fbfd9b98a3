"""Builders of seeded verify-step inputs for the GPU parity tests (inputs from workloads.gen;
expected values from the oracle only)."""
from __future__ import annotations

import math
import sys

import numpy as np
import torch

import oracle
from workloads import WORKLOADS, gen

# Tolerances.  Attention outputs and logits: max-abs 1e-2 for bf16 inputs and 1e-5 for fp32
# inputs, both accumulated in fp32.  p: max-abs 1e-5 (entries are at most 1; a logit error e
# moves p by at most p * e / T, and the fp32 exp/normalise adds a few ulp).
TOL = {"bf16": 1e-2, "f32": 1e-5}
P_TOL = 1e-5
# Regression bound on top of TOL: errors measured on MI355X are ~1e-6 (attention) and ~6e-6
# (logits) with bf16 inputs, and a one-key slip of the sliding window at the 8K batch-1 shape
# moves attention outputs by ~7e-3, inside the 1e-2 bar; 1e-4 catches such indexing errors.
REG_TOL = {"bf16": 1e-4, "f32": 1e-5}


def say(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def dev():
    return torch.device("cuda", 0)


def attn_inputs(w, layer: int, device, step: int = 0, ctx=None, table=None, num_pages=None):
    L = w.layers[layer]
    ctx = gen.context_lengths(w, step) if ctx is None else np.asarray(ctx, dtype=np.int32)
    if table is None:
        table, P = gen.page_tables(w, ctx, step)
    else:
        P = num_pages
    q = gen.queries(w, layer, device, step)
    k, v = gen.kv_pools(w, layer, P, device, step)
    return dict(q=q, k_pool=k, v_pool=v,
                page_table=torch.from_numpy(np.ascontiguousarray(table)).to(device),
                ctx_lens=torch.from_numpy(np.ascontiguousarray(ctx)).to(device),
                window=L.window, scale=1.0 / math.sqrt(L.head_dim))


def to_host(inp):
    return {k: (v.cpu() if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}


def oracle_attn(inp, rows=None):
    h = to_host(inp)
    return oracle.verify_attention(h["q"], h["k_pool"], h["v_pool"], h["page_table"].numpy(),
                                   h["ctx_lens"].numpy(), h["window"], h["scale"], rows=rows)


def accept_inputs(w, step: int = 0, batch=None, vocab=None, temps=None):
    """fp32 p [B, K1, V], q [B, k, V], drafts and uniforms for the accept stage.

    p and q are the oracle's float64 distributions of the workload's logit recipe, rounded to
    fp32: the identical arrays both sides consume.
    """
    B = w.batch if batch is None else batch
    V = w.vocab if vocab is None else vocab
    zq, zp = gen.logit_pairs(w, step, vocab=V, batch=B)
    t = gen.temperatures(w, B) if temps is None else np.asarray(temps, np.float32)
    k = w.k
    q = np.empty((B, k, V), np.float32)
    p = np.empty((B, k + 1, V), np.float32)
    for b in range(B):
        if k:
            q[b] = oracle.probabilities(zq[b], np.full(k, t[b])).astype(np.float32)
        p[b] = oracle.probabilities(zp[b], np.full(k + 1, t[b])).astype(np.float32)
    draft = gen.draw_drafts(w, q, t, step) if k else np.zeros((B, 0), np.int32)
    u = gen.uniforms(w, step, batch=B)
    return draft, q, p, u


def gpu_accept(draft, q, p, u, device):
    import speculative_decoding_decode_amd as sv
    n, tok = sv.accept(torch.from_numpy(draft).to(device), torch.from_numpy(q).to(device),
                       torch.from_numpy(p).to(device), torch.from_numpy(u).to(device))
    torch.cuda.synchronize(device)
    return n.cpu().numpy(), tok.cpu().numpy()


def explain_difference(draft, q, p_ref32, u, n_gpu, tok_gpu, n_ref, tok_ref, p_tol=1e-5):
    """Return None if the GPU chain's accept result equals the oracle chain's, else a reason the
    difference is a floating-point knife edge (decision margin or draw threshold within the p
    tolerance), or raise AssertionError if it is not."""
    from oracle.accept import sample_weights, uniform_index
    B, k = np.asarray(draft).shape
    V = p_ref32.shape[-1]
    reasons = []
    for b in range(B):
        if n_gpu[b] == n_ref[b] and np.array_equal(tok_gpu[b], tok_ref[b]):
            continue
        nmin = int(min(n_gpu[b], n_ref[b]))
        if n_gpu[b] != n_ref[b]:
            d = int(draft[b, nmin])
            margin = abs(float(u[b, nmin]) * float(q[b, nmin, d]) - float(p_ref32[b, nmin, d]))
            assert margin <= p_tol, f"sequence {b}: accept decision differs with margin {margin}"
            reasons.append(f"seq {b}: decision at position {nmin} within {margin:.2e}")
            continue
        w = sample_weights(p_ref32[b, nmin], q[b, nmin] if nmin < k else None)
        W = int(w.sum())
        t = (uniform_index(u[b, k]) * W) >> 24
        cum = np.cumsum(w)
        yg = int(tok_gpu[b, nmin])
        assert 0 <= yg < V and w[yg] > 0, f"sequence {b}: drawn token {yg} has no weight"
        gap = min(abs(int(cum[yg]) - t), abs(int(cum[yg] - w[yg]) - t)) / W
        assert gap <= p_tol, f"sequence {b}: draw differs, threshold {gap} from the boundary"
        reasons.append(f"seq {b}: draw threshold within {gap:.2e} of a boundary")
    return reasons or None
