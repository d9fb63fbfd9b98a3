"""Oracle: one whole verify step (attention layers, lm-head, row softmax, accept), float64.

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).  Composes attention.py, lm_head.py and
accept.py in the order of the verify step ([guide] §4 "실행 흐름": one target forward over the
draft, comparison with the target's own distribution, accept/reject).  The target's p enters
the acceptance as float32, the precision the GPU path hands between its calls.
"""
from __future__ import annotations

import numpy as np

from .attention import verify_attention
from .lm_head import logits, probabilities
from .accept import verify_accept


def verify_step(attn_layers, hidden, weight, row_temperature, draft, q, u):
    """attn_layers: list of dicts with q, k_pool, v_pool, page_table, ctx_lens, window, scale.

    Returns (attention outputs per layer, logits [R, V], p [B, K1, V] float64, n, tokens).
    """
    outs = [verify_attention(**a) for a in attn_layers]
    z = logits(hidden, weight)
    p = probabilities(z, row_temperature)
    B, k = np.asarray(draft).shape
    p32 = p.astype(np.float32).reshape(B, k + 1, -1)
    n, tokens = verify_accept(draft, q, p32, u)
    return outs, z, p.reshape(B, k + 1, -1), n, tokens
