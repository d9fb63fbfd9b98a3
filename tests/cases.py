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
