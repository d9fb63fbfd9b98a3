"""Drafter cross-attention over the target's shared KV cache on the GPU: the drafter's layers
attend the target's paged pools (one pool, no copy), one query per sequence per draft step,
issued as spec_verify_attn calls with K1 = 1 over the committed context.  Parity with the
fp64 oracle for each of the k chained draft steps, on the target layers of the batch-1 and
ragged-batch workloads."""
import numpy as np
import pytest
import torch

import speculative_decoding_decode_amd as sv
from workloads import WORKLOADS, gen
from cases import TOL, attn_inputs, oracle_attn, say, dev

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name,layer,hq", [
    ("b1_k2_sliding256_8k", 0, 4), ("b1_k4_global512_32k", 0, 8),
    ("b8_ragged_k5_hybrid", 0, 8), ("b8_ragged_k5_hybrid", 3, 2)])
def test_drafter_reads_target_pool(name, layer, hq):
    w = WORKLOADS[name]
    d = dev()
    inp = attn_inputs(w, layer, d)
    # committed context: the verify positions of this step are not in the cache yet
    inp["ctx_lens"] = inp["ctx_lens"] - w.k1
    pool_before = inp["k_pool"].view(-1)[:4096].clone()
    for j in range(w.k):
        inp["q"] = gen.drafter_queries(w, layer, hq, j, d)
        say(f"[drafter] {name} layer {layer} hq {hq} draft step {j}")
        out = sv.verify_attn(**inp)
        torch.cuda.synchronize()
        ref = oracle_attn(inp)
        err = float(np.abs(out.cpu().numpy() - ref).max())
        say(f"    max |err| = {err:.3e}")
        assert out.shape == (w.batch, 1, hq, w.layers[layer].head_dim)
        assert err <= TOL[w.dtype]
    assert torch.equal(inp["k_pool"].view(-1)[:4096], pool_before)   # the drafter only reads
