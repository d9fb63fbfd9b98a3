"""End to end: the GPU chain (verify attention per layer, lm-head + softmax, accept on the GPU's
own p) against the oracle chain (the same steps in float64, accept on the oracle's own p
rounded to fp32).  Attention outputs, logits and p must be within tolerance; accept counts and
tokens must be equal, or differ only where the oracle shows a floating-point knife edge."""
import numpy as np
import pytest
import torch

import oracle
import speculative_decoding_decode_amd as sv
from workloads import WORKLOADS, gen
from cases import TOL, REG_TOL, P_TOL, attn_inputs, oracle_attn, explain_difference, say, dev

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name,rows_sample", [("tiny_fp32_b1_k2", None),
                                               ("b1_k2_sliding256_8k", None),
                                               ("b1_k4_global512_32k", None),
                                               ("b8_ragged_k5_hybrid", None),
                                               ("b32_k2_mixed_16k", [0, 7, 31])])
def test_verify_step_chain(name, rows_sample):
    w = WORKLOADS[name]
    d = dev()
    B, k, K1, V = w.batch, w.k, w.k1, w.vocab
    say(f"[step] {name}: B={B} k={k} layers={len(w.layers)}")
    for li in range(len(w.layers)):
        inp = attn_inputs(w, li, d, step=5)
        out = sv.verify_attn(**inp)
        torch.cuda.synchronize()
        rows = None if rows_sample is None else [(b, i) for b in rows_sample for i in range(K1)]
        ref = oracle_attn(inp, rows=rows)
        got = out.cpu().numpy().astype(np.float64)
        if rows is not None:
            sel = tuple(np.array(rows).T)
            got, ref = got[sel], ref[sel]
        err = np.abs(got - ref).max()
        assert err <= TOL[w.dtype] and err <= REG_TOL[w.dtype]

    x = gen.hidden_states(w, d, step=5)
    W = gen.lm_head_table(w, d, step=5)
    rt = gen.row_temperatures(w)
    _, p = sv.lm_head(x, W, torch.from_numpy(rt).to(d))
    # drafter distributions and drafts of the workload's recipe (inputs, from the oracle side)
    zq, _ = gen.logit_pairs(w, step=5)
    temps = gen.temperatures(w)
    q = np.stack([oracle.probabilities(zq[b], np.full(k, temps[b])) for b in range(B)]).astype(np.float32)
    draft = gen.draw_drafts(w, q, temps, step=5)
    u = gen.uniforms(w, step=5)
    n_g, tok_g = sv.accept(torch.from_numpy(draft).to(d), torch.from_numpy(q).to(d),
                           p.view(B, K1, V), torch.from_numpy(u).to(d))
    torch.cuda.synchronize()

    z_ref = oracle.logits(x.cpu(), W.cpu())
    del W
    p_ref = oracle.probabilities(z_ref, rt)
    assert np.abs(p.cpu().numpy() - p_ref).max() <= P_TOL
    p_ref32 = p_ref.astype(np.float32).reshape(B, K1, V)
    n_r, tok_r = oracle.verify_accept(draft, q, p_ref32, u)
    why = explain_difference(draft, q, p_ref32, u, n_g.cpu().numpy(), tok_g.cpu().numpy(), n_r, tok_r)
    say(f"    n={n_g.cpu().tolist()[:8]}  differences: {why}")
