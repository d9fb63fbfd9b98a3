"""GPU parity of spec_lm_head_accept (the lm-head contraction and the accept step in one call,
p formed from the contraction's statistics instead of a finalize pass): n and tokens equal
spec_lm_head followed by spec_accept bit for bit (the definition the fused call keeps), on
every workload, with array and Philox uniforms, greedy and tempered rows, k = 0, one and two
MFMA passes, vocabularies of one and many statistics groups, out-of-range drafts, and a
workspace filled with junk and reused across calls of other sizes (no call needs its contents).
Against the oracle chain (float64 p rounded to fp32), the result must be equal or differ only
at a floating-point knife edge."""
import math

import numpy as np
import pytest
import torch

import oracle
import speculative_decoding_decode_amd as sv
from workloads import WORKLOADS, gen
from cases import explain_difference, say, dev

pytestmark = pytest.mark.gpu


def drafter(p, k, recipe_q, seed):
    """q [B, k, V]: the target's own rows for even sequences (every draft accepted), the
    recipe's drafter rows for odd ones; drafts drawn from q on the host."""
    B = p.shape[0]
    q = recipe_q.copy()
    q[0::2] = p[0::2, :k]
    rng = np.random.default_rng(seed)
    draft = np.zeros((B, k), np.int32)
    for b in range(B):
        for i in range(k):
            row = q[b, i].astype(np.float64)
            draft[b, i] = int(rng.choice(row.size, p=row / row.sum()))
    return q, draft


def run_both(x, W, temps, draft, q, u, seed=None, offset=0):
    d = dev()
    B, k = draft.shape
    V = W.shape[0]
    t = torch.as_tensor(np.asarray(temps, np.float32), device=d)
    dr = torch.from_numpy(np.ascontiguousarray(draft)).to(d)
    qt = torch.from_numpy(np.ascontiguousarray(q)).to(d) if k else None
    _, p = sv.lm_head(x, W, t)
    pk = p.view(B, k + 1, V)
    if seed is None:
        ut = torch.from_numpy(u).to(d)
        n2, tok2 = sv.accept(dr, qt, pk, ut)
        n1, tok1, _ = sv.lm_head_accept(x, W, t, dr, qt, ut)
    else:
        n2, tok2, u2 = sv.accept_philox(dr, qt, pk, seed, offset, return_uniforms=True)
        n1, tok1, u1 = sv.lm_head_accept(x, W, t, dr, qt, None, seed, offset, return_uniforms=True)
        torch.cuda.synchronize()
        assert torch.equal(u1, u2)
    torch.cuda.synchronize()
    return (n1.cpu().numpy(), tok1.cpu().numpy()), (n2.cpu().numpy(), tok2.cpu().numpy()), p


@pytest.mark.parametrize("name", ["tiny_fp32_b1_k2", "b1_k2_sliding256_8k", "b1_k4_global512_32k",
                                  "b8_ragged_k5_hybrid", "b32_k2_mixed_16k"])
@pytest.mark.parametrize("philox", [False, True])
def test_workloads_equal_two_calls(name, philox):
    w = WORKLOADS[name]
    d = dev()
    B, k, K1, V = w.batch, w.k, w.k1, w.vocab
    x = gen.hidden_states(w, d, step=3)
    W = gen.lm_head_table(w, d, step=3)
    rt = gen.row_temperatures(w)
    _, p = sv.lm_head(x, W, torch.from_numpy(rt).to(d))
    zq, _ = gen.logit_pairs(w, step=3)
    tq = gen.temperatures(w)
    recipe_q = np.stack([oracle.probabilities(zq[b], np.full(k, tq[b])) for b in range(B)]).astype(np.float32)
    q, draft = drafter(p.view(B, K1, V).cpu().numpy(), k, recipe_q, seed=B + k)
    u = gen.uniforms(w, step=3)
    say(f"[fused] {name} philox={philox}: B={B} k={k} V={V}")
    (n1, t1), (n2, t2), pg = run_both(x, W, rt, draft, q, u, seed=0xFEED if philox else None, offset=9)
    say(f"    n = {n1.tolist()[:16]}")
    assert np.array_equal(n1, n2) and np.array_equal(t1, t2)
    if name in ("tiny_fp32_b1_k2", "b1_k2_sliding256_8k") and not philox:
        # the oracle chain: its own p (rounded to fp32) with the same drafts, q and uniforms
        z_ref = oracle.logits(x.cpu(), W.cpu())
        p_ref32 = oracle.probabilities(z_ref, rt).astype(np.float32).reshape(B, K1, V)
        n_r, t_r = oracle.verify_accept(draft, q, p_ref32, u)
        why = explain_difference(draft, q, p_ref32, u, n1, t1, n_r, t_r)
        say(f"    against the oracle chain: {why or 'equal'}")


@pytest.mark.parametrize("B,k,H,V,dtype,temps", [
    (1, 0, 264, 5003, "bf16", (1.0,)),          # k = 0: a plain sampling step
    (3, 2, 64, 17, "f32", (1.0, 0.0, 0.5)),     # a vocabulary smaller than one block
    (33, 2, 136, 1000, "bf16", (0.0, 0.7, 1.0, 2.0)),   # 99 rows: two MFMA passes
    (2, 9, 2568, 777, "bf16", (0.0, 1.0)),
    (5, 3, 72, 70001, "f32", (0.7,)),           # many blocks, a ragged last group
    (1, 1, 8, 1, "bf16", (1.0,)),               # one vocabulary entry
    (48, 2, 64, 262144, "bf16", (1.0, 0.0, 0.7)),   # 32 chunks of 8192 per row
    (96, 2, 64, 262144, "bf16", (1.0,)),        # 16 chunks of 16384 per row, 288 rows
])
def test_ragged_shapes_equal_two_calls(B, k, H, V, dtype, temps):
    d = dev()
    K1 = k + 1
    td = torch.float32 if dtype == "f32" else torch.bfloat16
    g = torch.Generator().manual_seed(B * 131 + V)
    x = torch.randn(B * K1, H, generator=g).to(td).to(d)
    W = (torch.randn(V, H, generator=g) / math.sqrt(H)).to(td).to(d)
    rt = np.array([temps[(r // K1) % len(temps)] for r in range(B * K1)], np.float32)
    _, p = sv.lm_head(x, W, torch.from_numpy(rt).to(d))
    rng = np.random.default_rng(V)
    recipe_q = rng.dirichlet(np.ones(V), size=(B, k)).astype(np.float32) if k else np.zeros((B, 0, V), np.float32)
    q, draft = drafter(p.view(B, K1, V).cpu().numpy(), k, recipe_q, seed=V)
    if k:
        draft[B - 1, 0] = V + 3                     # out of range: rejected without a read
    u = rng.random((B, K1), dtype=np.float32)
    say(f"[fused] ragged B={B} k={k} H={H} V={V} {dtype}")
    (n1, t1), (n2, t2), _ = run_both(x, W, rt, draft, q, u)
    assert np.array_equal(n1, n2) and np.array_equal(t1, t2)


def test_max_rows_per_call():
    # B (k + 1) = 65535 rows, the most one call takes, against the two calls and the oracle chain
    d = dev()
    B, k, H, V = 13107, 4, 16, 64
    K1 = k + 1
    g = torch.Generator().manual_seed(13107)
    x = torch.randn(B * K1, H, generator=g).to(torch.bfloat16).to(d)
    W = (torch.randn(V, H, generator=g) / math.sqrt(H)).to(torch.bfloat16).to(d)
    rt = np.array([(0.0, 0.8, 1.0)[(r // K1) % 3] for r in range(B * K1)], np.float32)
    _, p = sv.lm_head(x, W, torch.from_numpy(rt).to(d))
    rng = np.random.default_rng(7)
    recipe_q = rng.dirichlet(np.ones(V), size=(B, k)).astype(np.float32)
    q, draft = drafter(p.view(B, K1, V).cpu().numpy(), k, recipe_q, seed=11)
    u = rng.random((B, K1), dtype=np.float32)
    say(f"[fused] max rows: B={B} k={k} V={V}")
    (n1, t1), (n2, t2), _ = run_both(x, W, rt, draft, q, u)
    assert np.array_equal(n1, n2) and np.array_equal(t1, t2)
    z_ref = oracle.logits(x.cpu(), W.cpu())
    p_ref32 = oracle.probabilities(z_ref, rt).astype(np.float32).reshape(B, K1, V)
    n_r, t_r = oracle.verify_accept(draft, q, p_ref32, u)
    why = explain_difference(draft, q, p_ref32, u, n1, t1, n_r, t_r)
    say(f"    against the oracle chain: {why or 'equal'}")


def test_workspace_reused_across_sizes():
    # one workspace per entry point, filled with junk once and reused by calls of decreasing and
    # increasing size: no call needs any contents in it, whatever the layout of the call before
    d = dev()
    shapes = [(8, 5, 256, 40000), (1, 2, 256, 3000), (32, 2, 128, 9000), (1, 2, 256, 3000)]
    need = max(sv.lm_head_accept_workspace_bytes(B, k, H, V) for B, k, H, V in shapes)
    ws = torch.full((need,), 0xA5, dtype=torch.uint8, device=d)
    ws_acc = torch.full((sv.accept_workspace_bytes(32, 5, 40000),), 0x5A, dtype=torch.uint8, device=d)
    ws_lm = torch.full((sv.lm_head_workspace_bytes(48, 256, 40000),), 0xFF, dtype=torch.uint8, device=d)
    for i, (B, k, H, V) in enumerate(shapes * 2):
        K1 = k + 1
        g = torch.Generator().manual_seed(i)
        x = torch.randn(B * K1, H, generator=g).to(torch.bfloat16).to(d)
        W = (torch.randn(V, H, generator=g) / math.sqrt(H)).to(torch.bfloat16).to(d)
        t = torch.ones(B * K1, device=d)
        _, p = sv.lm_head(x, W, t, workspace=ws_lm)
        pk = p.view(B, K1, V)
        q = pk[:, :k].contiguous()
        dr = torch.argmax(q, dim=-1).to(torch.int32).contiguous()
        u = torch.rand(B, K1, generator=g).to(d)
        n2, t2 = sv.accept(dr, q, pk, u, workspace=ws_acc)
        n1, t1, _ = sv.lm_head_accept(x, W, t, dr, q, u, workspace=ws)
        torch.cuda.synchronize()
        say(f"[fused] reuse call {i}: B={B} k={k} V={V}: n={n1.cpu().tolist()[:4]}")
        assert torch.equal(n1, n2) and torch.equal(t1, t2)
        assert (n1.cpu().numpy() == k).all()          # q = p at argmax drafts: all accepted
