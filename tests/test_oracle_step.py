"""Pins of the oracle's composed verify step (oracle/step.py: attention layers, lm-head, row
softmax, accept) to results fixed independently of the oracle's own modules:

* greedy decoding (temperature 0): the number of accepted drafts is the length of the prefix
  on which the drafts equal the target's argmax, and the emitted token is the target's argmax
  at the first mismatch; the logits here come from a pure-Python dot-product loop over the
  rows b * K1 + i (sequence-major), so a transposed row order or a wrong reshape fails;
* attention: every layer's output equals torch's scaled_dot_product_attention (CPU, float64)
  on the keys laid out contiguously with an explicit causal / window mask;
* a uniform of 0 accepts every draft with p(d) > 0 and draws the first index with a nonzero
  integer weight (the threshold is 0);
* the target's p reaches the accept step rounded to fp32 (the precision the calls hand over):
  a bonus draw is constructed whose integer weights select different tokens for the fp32 and
  the float64 p, and the step must draw the fp32 one.
"""
import math

import numpy as np
import torch

from oracle.step import verify_step

FP32_BITS = 38


def contiguous_layer(rng, B, K1, Hq, Hkv, D, ctx, window):
    """A layer whose cache is an identity page table over [B * pages] pages of 4 tokens."""
    ps = 4
    pages = max(-(-c // ps) for c in ctx)
    P = B * pages
    kp = rng.standard_normal((P, Hkv, ps, D))
    vp = rng.standard_normal((P, Hkv, ps, D))
    table = np.arange(P, dtype=np.int32).reshape(B, pages)
    q = rng.standard_normal((B, K1, Hq, D))
    return dict(q=q, k_pool=kp, v_pool=vp, page_table=table, ctx_lens=np.array(ctx, np.int32),
                window=window, scale=1 / math.sqrt(D))


def sdpa_reference(layer, K1, Hq, Hkv):
    q, kp, vp, table, ctx = (layer[x] for x in ("q", "k_pool", "v_pool", "page_table", "ctx_lens"))
    window = layer["window"]
    outs = []
    for b in range(q.shape[0]):
        T = int(ctx[b])
        # keys of sequence b in position order: page table row b, 4 slots per page
        kk = np.concatenate([kp[table[b, j]] for j in range(table.shape[1])], axis=1)[:, :T]
        vv = np.concatenate([vp[table[b, j]] for j in range(table.shape[1])], axis=1)[:, :T]
        kk = torch.from_numpy(kk).repeat_interleave(Hq // Hkv, dim=0)      # [Hq, T, D]
        vv = torch.from_numpy(vv).repeat_interleave(Hq // Hkv, dim=0)
        qq = torch.from_numpy(q[b]).permute(1, 0, 2)                        # [Hq, K1, D]
        pos_q = torch.arange(T - K1, T)[:, None]
        pos_k = torch.arange(T)[None, :]
        mask = pos_k <= pos_q
        if window:
            mask &= (pos_q - pos_k) < window
        o = torch.nn.functional.scaled_dot_product_attention(qq, kk, vv, attn_mask=mask,
                                                             scale=layer["scale"])
        outs.append(o.permute(1, 0, 2).numpy())
    return np.stack(outs)


def loop_logits(hidden, weight):
    R, H = hidden.shape
    V = weight.shape[0]
    z = np.zeros((R, V))
    for r in range(R):
        for v in range(V):
            s = 0.0
            for h in range(H):
                s += float(hidden[r, h]) * float(weight[v, h])
            z[r, v] = s
    return z


def test_greedy_step_is_argmax_prefix_and_attention_is_sdpa():
    rng = np.random.default_rng(41)
    B, k, H, V = 3, 3, 6, 9
    K1 = k + 1
    layers = [contiguous_layer(rng, B, K1, 4, 2, 8, [11, 6, 17], 0),
              contiguous_layer(rng, B, K1, 4, 2, 8, [11, 6, 17], 3)]
    hidden = rng.integers(-3, 4, size=(B * K1, H)).astype(np.float64)
    weight = rng.integers(-3, 4, size=(V, H)).astype(np.float64)
    weight[:, 0] += np.arange(V) * 0.01                  # no exact ties between vocab rows
    z = loop_logits(hidden, weight)
    target_argmax = [[int(np.argmax(z[b * K1 + i])) for i in range(K1)] for b in range(B)]
    # drafts: sequence 0 agrees everywhere, sequence 1 disagrees at position 1, sequence 2 at 0
    draft = np.array([target_argmax[0][:k],
                      [target_argmax[1][0], (target_argmax[1][1] + 1) % V, target_argmax[1][2]],
                      [(target_argmax[2][0] + 2) % V] + target_argmax[2][1:k]], dtype=np.int32)
    q = np.zeros((B, k, V), np.float32)
    for b in range(B):
        for i in range(k):
            q[b, i, draft[b, i]] = 1.0                    # greedy drafter: one-hot at its draft
    u = rng.random((B, K1), dtype=np.float32)
    outs, zo, p, n, tokens = verify_step(layers, hidden, weight, np.zeros(B * K1), draft, q, u)

    np.testing.assert_allclose(zo, z, rtol=0, atol=1e-9)
    for li, L in enumerate(layers):
        np.testing.assert_allclose(outs[li], sdpa_reference(L, K1, 4, 2), rtol=0, atol=1e-12)
    for b in range(B):
        j = 0
        while j < k and draft[b, j] == target_argmax[b][j]:
            j += 1
        assert n[b] == j
        assert list(tokens[b, :j]) == list(draft[b, :j])
        assert tokens[b, j] == target_argmax[b][j]
        assert (tokens[b, j + 1:] == -1).all()
    assert list(n) == [3, 1, 0]


def test_zero_uniforms_accept_everything_and_draw_the_first_weighted_index():
    rng = np.random.default_rng(5)
    B, k, H, V = 2, 2, 5, 12
    K1 = k + 1
    layers = [contiguous_layer(rng, B, K1, 2, 1, 4, [8, 5], 0)]
    hidden = rng.standard_normal((B * K1, H))
    weight = rng.standard_normal((V, H))
    weight[0] = -40.0 * np.sign(hidden[1])               # row 0 has a tiny p in row 1 only
    draft = rng.integers(0, V, size=(B, k)).astype(np.int32)
    q = np.full((B, k, V), 1.0 / V, np.float32)
    u = np.zeros((B, K1), np.float32)
    _, _, p, n, tokens = verify_step(layers, hidden, weight, np.ones(B * K1), draft, q, u)
    assert list(n) == [k, k]
    for b in range(B):
        assert list(tokens[b, :k]) == list(draft[b])
        # the bonus row is row b * K1 + k; its first index whose floor(p * 2^38) is positive
        pk = np.exp(hidden[b * K1 + k] @ weight.T - (hidden[b * K1 + k] @ weight.T).max())
        pk = (pk / pk.sum()).astype(np.float32)
        first = int(np.flatnonzero(np.floor(pk.astype(np.float64) * 2.0 ** FP32_BITS) > 0)[0])
        assert tokens[b, k] == first


def _inverse_cdf(weights, m):
    """Smallest j whose running weight sum exceeds floor(m * W / 2^24) (exact integers)."""
    t = (m * int(sum(weights))) >> 24
    run = 0
    for j, x in enumerate(weights):
        run += x
        if run > t:
            return j
    raise AssertionError("threshold beyond the total")


def test_target_probability_is_handed_over_in_fp32():
    # k = 0, V = 2: the bonus row z = (a, 0) has p(0) = 1 / (1 + e^-a).  Find a and a draw
    # index m where the integer weights floor(p * 2^38) of the fp32 p and of the float64 p
    # select different tokens; the step must follow the fp32 p.
    case = None
    for a in np.linspace(0.05, 2.0, 4001):
        p64 = 1.0 / (1.0 + math.exp(-a))
        w64 = [math.floor(p64 * 2.0 ** 38), math.floor((1.0 - p64) * 2.0 ** 38)]
        p32 = [float(np.float32(p64)), float(np.float32(1.0 - p64))]
        w32 = [math.floor(x * 2.0 ** 38) for x in p32]
        c = int(p64 * 2 ** 24)
        for m in range(c - 3, c + 4):
            if _inverse_cdf(w32, m) != _inverse_cdf(w64, m):
                case = (a, m, _inverse_cdf(w32, m))
                break
        if case:
            break
    assert case is not None
    a, m, y32 = case
    rng = np.random.default_rng(3)
    layers = [contiguous_layer(rng, 1, 1, 2, 1, 4, [6], 0)]
    hidden = np.array([[a, 0.0]])
    weight = np.array([[1.0, 0.0], [0.0, 1.0]])
    draft = np.zeros((1, 0), np.int32)
    q = np.zeros((1, 0, 2), np.float32)
    u = np.array([[m / 2 ** 24]], np.float32)
    _, _, p, n, tokens = verify_step(layers, hidden, weight, np.ones(1), draft, q, u)
    assert abs(p[0, 0, 0] - 1.0 / (1.0 + math.exp(-a))) < 1e-15   # p itself stays float64
    assert n[0] == 0 and tokens[0, 0] == y32
