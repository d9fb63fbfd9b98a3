"""GPU parity of spec_accept: accept counts and emitted tokens bit-exact against the oracle,
given identical fp32 p / q and uniforms."""
import numpy as np
import pytest
import torch

import oracle
import speculative_decoding_decode_amd as sv
from workloads import WORKLOADS, gen
from cases import accept_inputs, gpu_accept, say, dev

pytestmark = pytest.mark.gpu


def compare(draft, q, p, u, label):
    say(f"[accept] {label}: B={p.shape[0]} k={p.shape[1] - 1} V={p.shape[2]}")
    n, tok = gpu_accept(draft, q, p, u, dev())
    n_ref, tok_ref = oracle.verify_accept(draft, q, p, u)
    assert np.array_equal(n, n_ref), (n, n_ref)
    assert np.array_equal(tok, tok_ref)
    say(f"    mean accepted {n.mean():.3f}, tokens/step {(n + 1).mean():.3f}")
    return n


@pytest.mark.parametrize("name,batch,vocab", [
    ("tiny_fp32_b1_k2", 256, None),
    ("b1_k2_sliding256_8k", 48, None),
    ("b1_k4_global512_32k", 12, None),
    ("b8_ragged_k5_hybrid", 8, None),
    ("b32_k2_mixed_16k", 32, None),
    ("b8_ragged_k5_hybrid", 40, 1000),
    ("b1_k2_sliding256_8k", 96, None),    # 16 chunks of 16384 per row: the widest chunks
])
def test_workload_recipes(name, batch, vocab):
    w = WORKLOADS[name]
    draft, q, p, u = accept_inputs(w, step=1, batch=batch, vocab=vocab)
    compare(draft, q, p, u, name)


def test_workspace_contents_unused():
    # a workspace full of 0xFF bytes (every chunk sum and count at its maximum) gives the same
    # n and tokens as a zeroed one
    w = WORKLOADS["b32_k2_mixed_16k"]
    draft, q, p, u = accept_inputs(w, step=5, batch=12, vocab=70001)
    d = dev()
    args = [torch.from_numpy(a).to(d) for a in (draft, q, p, u)]
    nbytes = sv.accept_workspace_bytes(12, w.k, 70001)
    n0, t0 = sv.accept(*args, workspace=torch.zeros(nbytes, dtype=torch.uint8, device=d))
    n1, t1 = sv.accept(*args, workspace=torch.full((nbytes,), 0xFF, dtype=torch.uint8, device=d))
    torch.cuda.synchronize()
    assert torch.equal(n0, n1) and torch.equal(t0, t1)
    n_ref, tok_ref = oracle.verify_accept(draft, q, p, u)
    assert np.array_equal(n1.cpu().numpy(), n_ref) and np.array_equal(t1.cpu().numpy(), tok_ref)


def test_greedy_tiny():
    w = WORKLOADS["tiny_fp32_b1_k2"]
    draft, q, p, u = accept_inputs(w, step=2, batch=128, temps=np.zeros(128))
    n = compare(draft, q, p, u, "greedy")
    # greedy: accepted prefix = drafts matching the target's argmax
    for b in range(128):
        j = 0
        while j < 2 and draft[b, j] == int(np.argmax(p[b, j])):
            j += 1
        assert n[b] == j


def test_edge_cases():
    rng = np.random.default_rng(5)
    B, k, V = 6, 3, 777
    p = rng.dirichlet(np.ones(V), size=(B, k + 1)).astype(np.float32)
    q = rng.dirichlet(np.ones(V), size=(B, k)).astype(np.float32)
    draft = rng.integers(0, V, size=(B, k)).astype(np.int32)
    u = rng.random((B, k + 1), dtype=np.float32)
    draft[0, 0] = -5                      # out of range: rejected
    draft[1, 1] = V + 3
    q[2] = p[2, :k]                       # q == p: every draft accepted, bonus draw
    draft[2] = np.argmax(p[2, :k], axis=1)
    # residual empty after flooring: q just above p everywhere, u near 1 rejects draft 0
    q[3, 0] = np.nextafter(p[3, 0], np.float32(1))
    u[3, 0] = np.float32(1 - 2 ** -24)
    u[4] = 0.0                            # smallest uniforms
    u[5] = np.float32(1 - 2 ** -24)       # largest uniforms
    n = compare(draft, q, p, u, "edge cases")
    assert n[0] == 0 and n[1] == 1 and n[2] == k and n[3] == 0


def test_maximum_k():
    # k = 63 (K1 = 64 uniforms per sequence, one wave lane per draft): sequences whose drafter
    # equals the target accept all 63 drafts and draw the bonus token; the others stop at
    # their first rejection anywhere along the 63 positions
    rng = np.random.default_rng(9)
    B, k, V = 6, 63, 300
    p = rng.dirichlet(np.ones(V) * 0.5, size=(B, k + 1)).astype(np.float32)
    q = rng.dirichlet(np.ones(V) * 0.5, size=(B, k)).astype(np.float32)
    q[:2] = p[:2, :k]                                   # q == p: every draft accepted
    mix = 0.9 * p[2:4, :k] + 0.1 * q[2:4]               # close drafter: long accepted runs
    q[2:4] = (mix / mix.sum(-1, keepdims=True)).astype(np.float32)
    draft = np.empty((B, k), np.int32)
    for b in range(B):
        for i in range(k):
            pr = q[b, i].astype(np.float64)
            draft[b, i] = rng.choice(V, p=pr / pr.sum())
    u = rng.random((B, k + 1), dtype=np.float32)
    n = compare(draft, q, p, u, "k = 63")
    assert n[0] == k and n[1] == k


def test_k_zero_plain_sampling():
    rng = np.random.default_rng(6)
    B, V = 64, 3000
    p = rng.dirichlet(np.ones(V) * 0.3, size=(B, 1)).astype(np.float32)
    u = rng.random((B, 1), dtype=np.float32)
    compare(np.zeros((B, 0), np.int32), np.zeros((B, 0, V), np.float32), p, u, "k=0")


def test_deterministic_repeat():
    w = WORKLOADS["b32_k2_mixed_16k"]
    draft, q, p, u = accept_inputs(w, step=3, vocab=50000)
    a = gpu_accept(draft, q, p, u, dev())
    b = gpu_accept(draft, q, p, u, dev())
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
