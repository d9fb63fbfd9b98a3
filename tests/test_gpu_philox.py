"""spec_accept_philox on the GPU: the uniforms it draws equal the oracle's Philox4x32-10 bit
for bit (several seeds and offsets, k up to 63, 300 sequences), and its accept counts and
tokens equal spec_accept given those uniforms and, bit for bit, the oracle's accept rule on
the same fp32 p, q and uniforms."""
import numpy as np
import pytest
import torch

import oracle
import speculative_decoding_decode_amd as sv
from workloads import WORKLOADS
from cases import accept_inputs, gpu_accept, say, dev

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("seed,offset,B,k", [
    (0, 0, 3, 2), (0x0123456789ABCDEF, 7, 300, 5), (2 ** 64 - 1, 2 ** 40 + 3, 17, 9),
    (12345, 99, 4, 0), (7, 2 ** 32 - 1, 5, 63)])   # k = 63: 64 uniforms, counters 0..15
def test_uniforms_equal_oracle_generator(seed, offset, B, k):
    d = dev()
    V = 64
    p = torch.full((B, k + 1, V), 1.0 / V, dtype=torch.float32, device=d)
    q = torch.full((B, k, V), 1.0 / V, dtype=torch.float32, device=d)
    draft = torch.zeros((B, k), dtype=torch.int32, device=d)
    _, _, u = sv.accept_philox(draft, q, p, seed, offset, return_uniforms=True)
    torch.cuda.synchronize()
    ref = oracle.philox_uniforms(seed, offset, B, k + 1)
    say(f"[philox] seed {seed:#x} offset {offset} B={B} k={k}: u[0] = {u[0].tolist()}")
    assert np.array_equal(u.cpu().numpy(), ref)


@pytest.mark.parametrize("name,batch,vocab", [("b1_k2_sliding256_8k", 64, None),
                                              ("b8_ragged_k5_hybrid", 8, 1000)])
def test_accept_with_generated_uniforms(name, batch, vocab):
    w = WORKLOADS[name]
    d = dev()
    draft, q, p, _ = accept_inputs(w, step=5, batch=batch, vocab=vocab)
    seed, offset = 0x5EED, 11
    n, tok, u = sv.accept_philox(torch.from_numpy(draft).to(d), torch.from_numpy(q).to(d),
                                 torch.from_numpy(p).to(d), seed, offset, return_uniforms=True)
    torch.cuda.synchronize()
    u_ref = oracle.philox_uniforms(seed, offset, batch, w.k1)
    assert np.array_equal(u.cpu().numpy(), u_ref)
    n2, tok2 = gpu_accept(draft, q, p, u_ref, d)
    assert np.array_equal(n.cpu().numpy(), n2) and np.array_equal(tok.cpu().numpy(), tok2)
    # identical fp32 p, q and uniforms on both sides: the oracle's result is the unique one
    n_ref, tok_ref = oracle.verify_accept(draft, q, p, u_ref)
    say(f"[philox] {name}: n {n.cpu().tolist()[:12]}")
    assert np.array_equal(n.cpu().numpy(), n_ref)
    assert np.array_equal(tok.cpu().numpy(), tok_ref)
