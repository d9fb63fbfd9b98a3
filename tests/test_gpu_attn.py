"""GPU parity of spec_verify_attn (split-K paged GQA verify attention) against the fp64
oracle: all workload layers at full size (sampled sequences for the largest batch), plus
ragged and degenerate cases."""
import math

import numpy as np
import pytest
import torch

import speculative_decoding_decode_amd as sv
from workloads import WORKLOADS, gen
from workloads.configs import Layer, Workload
from cases import TOL, REG_TOL, attn_inputs, oracle_attn, say, dev

pytestmark = pytest.mark.gpu


def check(inp, dtype, label, rows=None):
    B, K1, Hq, D = inp["q"].shape
    say(f"[attn] {label}: B={B} K1={K1} Hq={Hq} Hkv={inp['k_pool'].shape[1]} D={D} "
        f"window={inp['window']} ctx={inp['ctx_lens'].cpu().tolist()[:8]}")
    out = sv.verify_attn(**inp)
    torch.cuda.synchronize()
    ref = oracle_attn(inp, rows=rows)
    got = out.cpu().numpy().astype(np.float64)
    if rows is not None:
        sel = tuple(np.array(rows).T)
        got, ref = got[sel], ref[sel]
    err = np.abs(got - ref).max()
    say(f"    max |err| = {err:.3e}")
    assert np.isfinite(got).all()
    assert err <= TOL[dtype]
    assert err <= REG_TOL[dtype]
    return out


def test_tiny_fp32_workload():
    w = WORKLOADS["tiny_fp32_b1_k2"]
    check(attn_inputs(w, 0, dev()), "f32", "tiny fp32")


@pytest.mark.parametrize("name", ["b1_k2_sliding256_8k", "b1_k4_global512_32k"])
def test_batch1_workloads(name):
    w = WORKLOADS[name]
    check(attn_inputs(w, 0, dev()), "bf16", name)


@pytest.mark.parametrize("layer", [0, 3])
def test_ragged_hybrid_workload(layer):
    w = WORKLOADS["b8_ragged_k5_hybrid"]
    check(attn_inputs(w, layer, dev()), "bf16", f"b8 ragged layer {layer}")


@pytest.mark.parametrize("layer", [0, 1])
def test_batch32_workload_sampled(layer):
    w = WORKLOADS["b32_k2_mixed_16k"]
    inp = attn_inputs(w, layer, dev())
    rows = [(b, i) for b in (0, 5, 13, 31) for i in range(w.k1)]
    check(inp, "bf16", f"b32 layer {layer}", rows=rows)


def small_workload(dtype, hq, hkv, d, window, k, batch=3):
    kind = "sliding" if window else "global"
    return Workload(name="ragged", batch=batch, k=k, layers=(Layer(kind, hq, hkv, d, window),),
                    ctx="fixed:16", hidden=8, vocab=8, dtype=dtype, logit_recipe="gauss",
                    noise_key="sigma:1", temperatures=(1.0,), seed=11)


@pytest.mark.parametrize("dtype,hq,hkv,d,window,k", [
    ("bf16", 6, 3, 128, 37, 3), ("f32", 4, 1, 256, 0, 1), ("f32", 8, 2, 512, 100, 5),
    ("bf16", 12, 1, 64, 0, 4), ("bf16", 4, 4, 256, 1, 2), ("f32", 16, 2, 64, 0, 9),
    # bf16 head dims 256 and 512 at one and two row tiles (head-dim-quarter and staged paths)
    ("bf16", 8, 2, 512, 50, 1), ("bf16", 8, 2, 512, 0, 5), ("bf16", 8, 2, 256, 37, 4),
    ("bf16", 8, 2, 256, 0, 3)])
def test_ragged_small(dtype, hq, hkv, d, window, k):
    w = small_workload(dtype, hq, hkv, d, window, k)
    ctx = np.array([k + 1, 333, 170], dtype=np.int32)         # minimal, ragged, page-ragged
    table, P = gen.page_tables(w, ctx, max_pages=30)
    table[1, 7] = P + 50                                       # a page id outside the pool
    inp = attn_inputs(w, 0, dev(), ctx=ctx, table=table, num_pages=P)
    check(inp, dtype, f"ragged small {dtype} hq{hq}/hkv{hkv} d{d} w{window} k{k}")


@pytest.mark.parametrize("dtype,hq,hkv,d,window", [
    ("bf16", 8, 2, 128, 0), ("bf16", 8, 2, 512, 100), ("f32", 4, 4, 64, 0)])
def test_maximum_k1(dtype, hq, hkv, d, window):
    # K1 = 64 verified positions, the most the call takes: 256 query rows per KV head (eight
    # row chunks of 32) at G = 4, two chunks at G = 1
    w = small_workload(dtype, hq, hkv, d, window, 63)
    ctx = np.array([64, 300, 1000], dtype=np.int32)
    table, P = gen.page_tables(w, ctx, max_pages=64)
    inp = attn_inputs(w, 0, dev(), ctx=ctx, table=table, num_pages=P)
    check(inp, dtype, f"K1 = 64 {dtype} hq{hq}/hkv{hkv} d{d} w{window}")


def test_context_clamped_to_table():
    # a context beyond the page table (max_pages * 16 = 64 tokens) is clamped to it, and the
    # verified positions then sit at the clamped context - K1 + i: the result equals the
    # oracle on the clamped context
    w = small_workload("bf16", 8, 2, 256, 0, 2, batch=2)
    ctx = np.array([64, 64], dtype=np.int32)
    table, P = gen.page_tables(w, ctx, max_pages=4)
    inp = attn_inputs(w, 0, dev(), ctx=ctx, table=table, num_pages=P)
    ref = oracle_attn(inp)
    inp["ctx_lens"] = torch.tensor([64, 10_000], dtype=torch.int32, device=dev())
    out = sv.verify_attn(**inp)
    torch.cuda.synchronize()
    err = np.abs(out.cpu().numpy().astype(np.float64) - ref).max()
    say(f"[attn] clamped context: max |err| against the oracle at ctx 64 = {err:.3e}")
    assert err <= REG_TOL["bf16"]


@pytest.mark.parametrize("d,window,k", [(256, 1024, 2), (512, 0, 4), (256, 37, 5)])
def test_workspace_contents_unused(d, window, k):
    # a workspace full of NaN bit patterns gives the same bits as a zeroed one: every partial
    # the merge reads is written by the same call
    w = small_workload("bf16", 8, 2, d, window, k, batch=4)
    ctx = np.array([k + 1, 1500, 700, 2100], dtype=np.int32)
    table, P = gen.page_tables(w, ctx, max_pages=140)
    inp = attn_inputs(w, 0, dev(), ctx=ctx, table=table, num_pages=P)
    nbytes = sv.verify_attn_workspace_bytes(4, k + 1, 8, 2, d, 140, window)
    zero = torch.zeros(nbytes, dtype=torch.uint8, device=dev())
    junk = torch.full((nbytes,), 0xFF, dtype=torch.uint8, device=dev())
    a = sv.verify_attn(**inp, workspace=zero).clone()
    b = sv.verify_attn(**inp, workspace=junk)
    torch.cuda.synchronize()
    assert torch.equal(a, b) and not torch.isnan(b).any()


def test_deterministic_repeat():
    w = WORKLOADS["b1_k2_sliding256_8k"]
    inp = attn_inputs(w, 0, dev(), step=4)
    a = sv.verify_attn(**inp).clone()
    b = sv.verify_attn(**inp)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


@pytest.mark.parametrize("ctx_len", [2000, 800_000])
def test_long_page_table(ctx_len):
    """A 50000-page table (800K tokens): the plan's floor on pages per piece (13 here, which
    keeps one unit's pieces within what the merge takes) sets the split of a short context,
    and a full one splits into ~100-page pieces, ~500 per unit."""
    w = small_workload("bf16", 8, 2, 128, 0, 2, batch=1)
    ctx = np.array([ctx_len], dtype=np.int32)
    table, P = gen.page_tables(w, ctx, max_pages=50_000)
    inp = attn_inputs(w, 0, dev(), ctx=ctx, table=table, num_pages=P)
    check(inp, "bf16", f"page table of 50000 pages, ctx {ctx_len}")


@pytest.mark.parametrize("dtype,window,k,d", [("bf16", 0, 2, 128), ("f32", 40, 0, 128),
                                             ("bf16", 0, 2, 512), ("bf16", 30, 1, 256)])
def test_many_sequences(dtype, window, k, d):
    """More than 64 sequences (the work split scans the context lengths 64 at a time), ragged,
    with empty contexts and contexts holding only the verified positions."""
    B = 150
    w = small_workload(dtype, 4, 2, d, window, k, batch=B)
    rng = np.random.default_rng(21)
    ctx = rng.integers(k + 1, 700, size=B).astype(np.int32)
    ctx[[3, 70, 149]] = 0                                   # nothing cached
    ctx[[5, 100]] = k + 1                                   # only the verified positions
    table, P = gen.page_tables(w, ctx, max_pages=44)
    inp = attn_inputs(w, 0, dev(), ctx=ctx, table=table, num_pages=P)
    check(inp, dtype, f"{B} ragged sequences {dtype} hd{d} window {window} k {k}")
