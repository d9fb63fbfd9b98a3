"""KV bookkeeping on the GPU over several verify steps (append -> attention -> accept ->
commit) against the oracle doing the same steps on host copies: pools and lengths equal
bit for bit, attention within tolerance, accept counts identical."""
import math

import numpy as np
import pytest
import torch

import oracle
from oracle import kv as okv
import speculative_decoding_decode_amd as sv
from cases import TOL, say, dev

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("dtype,D,window", [("bf16", 256, 24), ("f32", 64, 0)])
def test_multi_step_chain(dtype, D, window):
    d = dev()
    td = torch.bfloat16 if dtype == "bf16" else torch.float32
    rng = np.random.default_rng(11)
    B, k, Hq, Hkv, V, ps = 3, 3, 4, 2, 50, 16
    K1 = k + 1
    maxp, P = 12, 40
    table = np.stack([rng.permutation(P)[:maxp] for _ in range(B)]).astype(np.int32)
    g = torch.Generator().manual_seed(5)
    kp = torch.randn(P, Hkv, ps, D, generator=g).to(td)
    vp = torch.randn(P, Hkv, ps, D, generator=g).to(td)
    ctx = np.array([20, 37, 5], dtype=np.int32)
    kp_h, vp_h, ctx_h = kp.double().numpy().copy(), vp.double().numpy().copy(), ctx.copy()
    kp_d, vp_d = kp.to(d), vp.to(d)
    table_d = torch.from_numpy(table).to(d)
    ctx_d = torch.from_numpy(ctx).to(d)
    for step in range(5):
        say(f"[kv] {dtype} D={D} step {step}: ctx {ctx_h.tolist()}")
        kn = torch.randn(B, K1, Hkv, D, generator=g).to(td)
        vn = torch.randn(B, K1, Hkv, D, generator=g).to(td)
        q = torch.randn(B, K1, Hq, D, generator=g).to(td)
        ctx_d += K1
        ctx_h = ctx_h + K1
        sv.kv_append(kn.to(d), vn.to(d), kp_d, vp_d, table_d, ctx_d)
        okv.append(kp_h, vp_h, table, ctx_h, kn.double().numpy(), vn.double().numpy())
        out = sv.verify_attn(q.to(d), kp_d, vp_d, table_d, ctx_d, window=window)
        ref = oracle.verify_attention(q, kp_h, vp_h, table, ctx_h, window, 1 / math.sqrt(D))
        torch.cuda.synchronize()
        assert np.abs(out.cpu().numpy() - ref).max() <= TOL[dtype]
        p = rng.dirichlet(np.ones(V), size=(B, K1)).astype(np.float32)
        qd = rng.dirichlet(np.ones(V), size=(B, k)).astype(np.float32)
        draft = rng.integers(0, V, size=(B, k)).astype(np.int32)
        u = rng.random((B, K1), dtype=np.float32)
        n, _ = sv.accept(torch.from_numpy(draft).to(d), torch.from_numpy(qd).to(d),
                         torch.from_numpy(p).to(d), torch.from_numpy(u).to(d))
        n_ref, _ = oracle.verify_accept(draft, qd, p, u)
        assert np.array_equal(n.cpu().numpy(), n_ref)
        sv.kv_commit(ctx_d, n, K1)
        ctx_h = okv.commit(ctx_h, n_ref, K1).astype(np.int32)
        torch.cuda.synchronize()
        assert np.array_equal(ctx_d.cpu().numpy(), ctx_h)
    np.testing.assert_array_equal(kp_d.cpu().double().numpy(), kp_h)
    np.testing.assert_array_equal(vp_d.cpu().double().numpy(), vp_h)


def test_append_and_commit_edge_cases():
    """Positions before the cache start or past the page table, page ids outside the pool and
    negative table entries are skipped (nothing else in the pools changes); commit clamps n to
    [0, K1 - 1]."""
    d = dev()
    rng = np.random.default_rng(3)
    B, K1, Hkv, D, ps, maxp, P = 6, 4, 2, 128, 16, 3, 24
    table = rng.permutation(P)[:B * maxp].reshape(B, maxp).astype(np.int32)   # no page shared
    table[1, 2] = -1          # a hole in the table
    table[2, 0] = P + 5       # a page id outside the pool
    table[3, 1] = -7
    # ctx (already counting the K1 new positions): 2 < K1 (two positions before the start),
    # 49 (the last new position is past the 48-token table), 33..36 over the hole / bad ids
    ctx = np.array([2, 49, 4, 20, 36, 48], dtype=np.int32)
    g = torch.Generator().manual_seed(9)
    kp = torch.randn(P, Hkv, ps, D, generator=g).to(torch.bfloat16)
    vp = torch.randn(P, Hkv, ps, D, generator=g).to(torch.bfloat16)
    kn = torch.randn(B, K1, Hkv, D, generator=g).to(torch.bfloat16)
    vn = torch.randn(B, K1, Hkv, D, generator=g).to(torch.bfloat16)
    kp_h, vp_h = kp.double().numpy().copy(), vp.double().numpy().copy()
    okv.append(kp_h, vp_h, table, ctx, kn.double().numpy(), vn.double().numpy())
    kp_d, vp_d = kp.to(d), vp.to(d)
    sv.kv_append(kn.to(d), vn.to(d), kp_d, vp_d, torch.from_numpy(table).to(d),
                 torch.from_numpy(ctx).to(d))
    torch.cuda.synchronize()
    np.testing.assert_array_equal(kp_d.cpu().double().numpy(), kp_h)
    np.testing.assert_array_equal(vp_d.cpu().double().numpy(), vp_h)
    # commit: n below 0 and above K1 - 1 are clamped
    ctx_c = np.array([10, 49, 20, 20, 36, 48], dtype=np.int32)
    n = np.array([-3, 0, 1, 3, 4, 100], dtype=np.int32)
    ctx_d = torch.from_numpy(ctx_c.copy()).to(d)
    sv.kv_commit(ctx_d, torch.from_numpy(n).to(d), K1)
    torch.cuda.synchronize()
    assert np.array_equal(ctx_d.cpu().numpy(), okv.commit(ctx_c, n, K1))
    assert okv.commit(ctx_c, n, K1).tolist() == [7, 46, 18, 20, 36, 48]
