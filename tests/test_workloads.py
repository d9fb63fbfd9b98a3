"""Seeded generators: reproducible, in range, with the stated structure."""
import numpy as np

from workloads import WORKLOADS, ORDER, noise_sigma
from workloads import gen


def test_registry_shapes():
    assert list(ORDER) == list(WORKLOADS)
    w = WORKLOADS["b1_k2_sliding256_8k"]
    assert (w.batch, w.k1, w.rows, w.hidden, w.vocab) == (1, 3, 3, 2560, 262144)
    L = w.layers[0]
    assert (L.kind, L.hq, L.hkv, L.head_dim, L.window) == ("sliding", 8, 2, 256, 1024)
    c3 = WORKLOADS["b8_ragged_k5_hybrid"]
    assert [l.kind for l in c3.layers] == ["sliding"] * 3 + ["global"]
    assert [c3.temperature_of(b) for b in range(4)] == [0.0, 0.7, 1.0, 0.0]
    assert 1.3 < noise_sigma(w) < 1.6 and noise_sigma(WORKLOADS["tiny_fp32_b1_k2"]) == 0.7


def test_uniforms_are_24_bit_and_reproducible():
    w = WORKLOADS["b32_k2_mixed_16k"]
    u = gen.uniforms(w, step=3)
    assert u.dtype == np.float32 and u.shape == (32, 3)
    assert ((u >= 0) & (u < 1)).all()
    assert (np.floor(u.astype(np.float64) * 2 ** 24) == u.astype(np.float64) * 2 ** 24).all()
    assert (gen.uniforms(w, step=3) == u).all() and not (gen.uniforms(w, step=4) == u).all()


def test_context_lengths_and_page_tables():
    for name in ORDER:
        w = WORKLOADS[name]
        ctx = gen.context_lengths(w)
        assert (ctx >= w.k1).all() and (ctx <= gen.max_context(w)).all()
        table, P = gen.page_tables(w, ctx)
        used = []
        for b in range(w.batch):
            n = -(-int(ctx[b]) // w.page_size)
            assert (table[b, :n] >= 0).all() and (table[b, n:] == -1).all()
            used.extend(table[b, :n].tolist())
        assert len(used) == len(set(used)) and max(used) < P
        if not w.paged:
            assert used == list(range(len(used)))
    c3 = gen.context_lengths(WORKLOADS["b8_ragged_k5_hybrid"])
    assert len(set(c3.tolist())) > 1 and c3.min() >= 1024 and c3.max() <= 16384


def test_tensor_generators_reproducible():
    w = WORKLOADS["tiny_fp32_b1_k2"]
    a = gen.queries(w, 0)
    b = gen.queries(w, 0)
    assert a.shape == (1, 3, 8, 64) and bool((a == b).all())
    k, v = gen.kv_pools(w, 0, 32)
    assert k.shape == (32, 2, 16, 64) and not bool((k == v).all())
    W = gen.lm_head_table(w)
    assert W.shape == (4096, 256) and abs(float(W.float().std()) - 1 / 16) < 2e-3


def test_logit_recipes():
    w = WORKLOADS["tiny_fp32_b1_k2"]
    zq, zp = gen.logit_pairs(w)
    assert zq.shape == (1, 2, 4096) and zp.shape == (1, 3, 4096)
    assert abs(np.std(zp[:, :2] - zq) - 0.7) < 0.03
    z = WORKLOADS["b1_k4_global512_32k"]
    zq, zp = gen.logit_pairs(z, vocab=1000)
    assert zq.shape == (1, 4, 1000) and zp.shape == (1, 5, 1000)
    # Zipf base: the sorted base row is -1.1 ln(1..V)
    base = np.sort(zp[0, 0])[::-1]
    assert base[0] > base[-1] + 5


def test_draft_draws():
    w = WORKLOADS["b8_ragged_k5_hybrid"]
    rng = np.random.default_rng(0)
    q = rng.dirichlet(np.ones(50), size=(8, 5)).astype(np.float32)
    d = gen.draw_drafts(w, q, gen.temperatures(w))
    assert d.shape == (8, 5) and d.dtype == np.int32 and ((d >= 0) & (d < 50)).all()
    for i in range(5):
        assert d[0, i] == int(np.argmax(q[0, i]))       # sequence 0 is greedy
