"""The verify step captured in a HIP graph (torch.cuda.CUDAGraph) and replayed: every call of
the library only enqueues kernels on the caller's stream and allocates nothing when its
workspace is given, so a captured step replays.  Each replay follows eager work and a
synchronisation, runs on uniforms and drafts rewritten in place since the capture, and must
give the bits of the same calls made eagerly."""
import numpy as np
import pytest
import torch

import speculative_decoding_decode_amd as sv
from workloads import WORKLOADS, gen
from cases import attn_inputs, say, dev

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name", ["b1_k2_sliding256_8k", "b8_ragged_k5_hybrid"])
def test_step_replays_from_a_graph(name):
    w = WORKLOADS[name]
    d = dev()
    B, k, K1, V, H = w.batch, w.k, w.k1, w.vocab, w.hidden
    L = w.layers[0]
    inp = attn_inputs(w, 0, d, step=6)
    max_pages = inp["page_table"].shape[1]
    x = gen.hidden_states(w, d, step=6)
    W = gen.lm_head_table(w, d, step=6)
    t = torch.from_numpy(gen.row_temperatures(w)).to(d)
    rng = np.random.default_rng(6)
    q = torch.from_numpy(rng.dirichlet(np.ones(V), size=(B, k)).astype(np.float32)).to(d)
    draft = torch.from_numpy(rng.integers(0, V, size=(B, k)).astype(np.int32)).to(d)
    u = torch.from_numpy(rng.random((B, K1), dtype=np.float32)).to(d)

    ws_a = torch.empty(sv.verify_attn_workspace_bytes(B, K1, L.hq, L.hkv, L.head_dim, max_pages,
                                                      L.window), dtype=torch.uint8, device=d)
    ws_l = torch.empty(sv.lm_head_accept_workspace_bytes(B, k, H, V), dtype=torch.uint8, device=d)
    out_g = torch.empty((B, K1, L.hq, L.head_dim), dtype=torch.float32, device=d)
    n_g = torch.empty((B,), dtype=torch.int32, device=d)
    tok_g = torch.empty((B, K1), dtype=torch.int32, device=d)

    def step(out, n, tok):
        sv.verify_attn(**inp, out=out, workspace=ws_a)
        sv.lm_head_accept(x, W, t, draft, q, u, n_accepted=n, tokens=tok, workspace=ws_l)

    step(out_g, n_g, tok_g)                      # eager first call: per-device set-up done here
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step(out_g, n_g, tok_g)
    torch.cuda.synchronize()

    for rep in range(4):
        # new uniforms and drafts in the captured buffers, some unrelated eager work
        u.copy_(torch.from_numpy(rng.random((B, K1), dtype=np.float32)).to(d))
        draft.copy_(torch.from_numpy(rng.integers(0, V, size=(B, k)).astype(np.int32)).to(d))
        junk = torch.randn(1 << 20, device=d).sum()
        torch.cuda.synchronize()
        out_e = torch.empty_like(out_g)
        n_e = torch.empty_like(n_g)
        tok_e = torch.empty_like(tok_g)
        step(out_e, n_e, tok_e)
        torch.cuda.synchronize()
        out_g.fill_(float("nan"))
        n_g.fill_(-7)
        tok_g.fill_(-7)
        g.replay()
        torch.cuda.synchronize()
        say(f"[graph] {name} replay {rep}: n {n_g.cpu().tolist()[:8]} (junk {float(junk):.1f})")
        assert torch.equal(out_g, out_e)
        assert torch.equal(n_g, n_e) and torch.equal(tok_g, tok_e)
