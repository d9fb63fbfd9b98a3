"""Benchmark of the verify step on one MI355X.

    python bench.py [--steps K] [--warmup W] [--gpus 1] [--no-cpu-baseline] [--workload NAME]
    python bench.py --sweep-k KMAX [--workload NAME] [--steps K]
    python bench.py --lm-head-rows      # the contraction at 1..8 rows, 2560 / 5376 wide
    python bench.py --calibrate-copy    # one plain copy of known size (HBM counter scaling)

Default workload (the headline line): batch 1, k = 2 drafts (3 verified positions), one
sliding-window attention layer (8 query / 2 KV heads, head dim 256, window 1024) over a paged
8192-token cache (16-token pages, randomly permuted), lm-head 2560 x 262144 bf16, temperature
1; drafter / target noise tuned for about 47% acceptance per position.  `--workload` selects any
other workload of workloads/configs.py (measured the same way; not the headline).

One step = spec_verify_attn for every attention layer -> spec_lm_head_accept (the lm-head and
the accept / reject in one call; `--two-calls`: spec_lm_head -> spec_accept, same results), on
inputs resident in HBM.  Up to 64 input sets (queries, cache regions of one shared page pool, hidden
states, drafter distributions) rotate over the steps, and every step has its own drafts and
uniforms, so KV and drafter rows are not cache-resident from the previous step.

Drafter stand-in: the drafter shares the target's vocab table (the serving guide's section 1
table: the input embedding table is shared), so its distribution q is the lm-head call applied
to the target hidden state plus N(0, sigma^2) noise; each step's drafts are drawn from q by the
accept call with k = 0.  Both are prepared before timing.

`--sweep-k KMAX` instead times the step at k = 0..KMAX drafts (k = 0: plain decoding) and
prints one JSON line with the step time per k, the tokens per step (from the per-position
acceptance measured at KMAX), verified tokens/s per k, and the k the telemetry picks.

Prints one JSON line:
  value       verified tokens/s = B x E[n + 1] / measured step time, where E[n + 1] (accepted
              drafts + the correction / bonus token) is the closed form of the timed steps'
              input sets, 1 + sum_j prod_{i<=j} sum_v min(p_i, q_i); the count actually emitted
              over the timed steps is reported beside it (value_sampled), since over a few
              steps it carries the luck of the draws;
  step_hbm_gbs  the step's algorithmic bytes (KV read + lm-head table) / step time;
  roofline    the dominant kernel (the lm-head contraction), timed with HIP events the library
              records right around it, in a separate pass of 100-500 steps after the timed one;
  hbm_ceiling the rates of the library's plain streaming read and copy probes on the same box;
  cpu_baseline  the fp64 oracle on the host cores, on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import ctypes
import dataclasses
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

DEFAULT_WORKLOAD = "b1_k2_sliding256_8k"
MAX_SETS = 64
SET_BUDGET_BYTES = 48 << 30   # KV-cache bytes allowed for all input sets together
BRACKET_MIN, BRACKET_MAX = 100, 500   # steps of the pass that brackets the contraction kernel
HBM_PEAK_GBS = 8000.0
METRIC = "verified tokens/sec and verify-step HBM GB/s (% peak), batch 1, k=2, 8K ctx"
# HBM bytes per launch of the contraction kernel from rocprofv3 FETCH_SIZE / WRITE_SIZE runs,
# scaled by a 1 GiB copy (profiles/lm_head_b1_k2_sliding256_8k_traffic.md).  Valid only
# for the default workload and the kernel source those counters were taken on.
PROFILED_TRAFFIC = {
    "workload": DEFAULT_WORKLOAD,
    "source": "speculative_decoding_decode_amd/csrc/lm_head.hip",
    "sha256": "2b016cf275d87557a856c8370a74d2af7fcf57ca9069e1838d2a93c7cfaee4c4",
    "bytes_per_launch": 1346231983,
}


class HipEvents:
    """hipEvent_t handles through the process's HIP runtime (the one torch loaded)."""

    def __init__(self, n: int):
        self.hip = ctypes.CDLL("libamdhip64.so.7")
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                 ctypes.c_void_p]
        self.hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.ev = []
        for _ in range(n):
            e = ctypes.c_void_p()
            if self.hip.hipEventCreate(ctypes.byref(e)) != 0:
                raise RuntimeError("hipEventCreate failed")
            self.ev.append(e)

    def record(self, i, stream):
        if self.hip.hipEventRecord(self.ev[i], stream) != 0:
            raise RuntimeError("hipEventRecord failed")

    def ms(self, a, b) -> float:
        out = ctypes.c_float()
        if self.hip.hipEventElapsedTime(ctypes.byref(out), self.ev[a], self.ev[b]) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return float(out.value)

    def close(self):
        for e in self.ev:
            self.hip.hipEventDestroy(e)


def profiled_traffic(workload):
    """Measured HBM bytes per launch, or None (other workload, or kernel changed since)."""
    import hashlib
    if workload != PROFILED_TRAFFIC["workload"]:
        return None
    path = os.path.join(ROOT, PROFILED_TRAFFIC["source"])
    with open(path, "rb") as f:
        ok = hashlib.sha256(f.read()).hexdigest() == PROFILED_TRAFFIC["sha256"]
    return PROFILED_TRAFFIC["bytes_per_launch"] if ok else None


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def visible_tokens(ctx, k1, window):
    lo = max(0, int(ctx) - k1 - window + 1) if window else 0
    return int(ctx) - lo


def algorithmic_bytes(w, ctx_lens):
    """KV bytes every verify step must read plus the lm-head table: the roofline numerator."""
    esz = 2 if w.dtype == "bf16" else 4
    kv = 0
    for L in w.layers:
        for c in ctx_lens:
            kv += visible_tokens(c, w.k1, L.window) * L.hkv * L.head_dim * esz * 2
    table = w.vocab * w.hidden * esz
    return kv, table


def number_of_sets(w, ctx1):
    esz = 2 if w.dtype == "bf16" else 4
    per_set = sum(int(sum(-(-int(c) // w.page_size) for c in ctx1)) * w.page_size
                  * L.hkv * L.head_dim * esz * 2 for L in w.layers)
    return int(max(1, min(MAX_SETS, SET_BUDGET_BYTES // max(per_set, 1))))


def prepare(w, device, torch, sv, gen, noise_sigma):
    """Device-resident inputs for the rotating input sets."""
    B, k, K1 = w.batch, w.k, w.k1
    ctx1 = gen.context_lengths(w)                            # [B] for one step
    nsets = number_of_sets(w, ctx1)
    # one shared page pool per layer holding the caches of all sets (nsets * B sequences)
    wpool = dataclasses.replace(w, batch=nsets * B)
    ctx_all = np.tile(ctx1, nsets).astype(np.int32)
    table_all, P = gen.page_tables(wpool, ctx_all)
    pools = [gen.kv_pools(wpool, li, P, device) for li in range(len(w.layers))]
    tables = torch.from_numpy(table_all).to(device)
    ctx_dev = torch.from_numpy(ctx_all).to(device)
    W = gen.lm_head_table(w, device)
    temps = torch.from_numpy(gen.row_temperatures(w)).to(device)
    sigma = noise_sigma(w)
    sets, alphas = [], []
    tq = temps.view(B, K1)[:, :k].reshape(-1).contiguous()
    for s in range(nsets):
        qs = [gen.queries(w, li, device, step=s) for li in range(len(w.layers))]
        x = gen.hidden_states(w, device, step=s)
        if k == 0:                                           # plain decoding: no drafter
            sets.append(dict(q=qs, x=x, qd=None, table=tables[s * B:(s + 1) * B],
                             ctx=ctx_dev[s * B:(s + 1) * B]))
            continue
        noise = gen.drafter_hidden_noise(w, device, step=s)
        xd = (x.float() + sigma * noise).to(x.dtype).view(B, K1, -1)[:, :k].reshape(B * k, -1)
        xd = xd.contiguous()
        # drafter distributions through the shared table
        _, qd = sv.lm_head(xd, W, tq)
        # closed-form acceptance of each drafted position, sum_v min(p, q), from the target's
        # rows of this set (a diagnostic of the inputs, computed before timing)
        _, pt = sv.lm_head(x, W, temps)
        alpha = torch.minimum(pt.view(B, K1, -1)[:, :k], qd.view(B, k, -1)).sum(-1)
        alphas.append(alpha)                                 # [B, k]
        sets.append(dict(q=qs, x=x, qd=qd.view(B, k, -1),
                         table=tables[s * B:(s + 1) * B], ctx=ctx_dev[s * B:(s + 1) * B]))
    torch.cuda.synchronize(device)
    alpha = (torch.stack(alphas).double().cpu().numpy() if k
             else np.zeros((nsets, B, 0)))                   # [sets, B, k]
    alpha_pos = alpha.mean(axis=(0, 1)).tolist() if k else []
    return dict(pools=pools, W=W, temps=temps, sets=sets, P=P, ctx=ctx1, nsets=nsets,
                max_pages=table_all.shape[1], alpha_pos=alpha_pos,
                expected_tokens=expected_tokens(alpha))


def expected_tokens(alpha):
    """Expected emitted tokens per sequence and input set, E[n + 1] = 1 + sum_j prod_{i<=j} a_i
    with a_i = sum_v min(p_i, q_i) the closed-form acceptance at draft position i (the rows of
    one input set do not depend on the drafted prefix, so the positions are independent).
    alpha [sets, B, k] -> [sets, B]."""
    sets, B, k = alpha.shape
    out = np.ones((sets, B))
    run = np.ones((sets, B))
    for i in range(k):
        run = run * alpha[:, :, i]
        out += run
    return out


def cpu_baseline(w, gen, seconds_target=12.0, max_steps=400):
    """The fp64 oracle (untuned) on a bounded sample of the same workload."""
    import oracle
    from oracle.step import verify_step
    from workloads import noise_sigma
    from threadpoolctl import threadpool_info, threadpool_limits
    cores = len(os.sched_getaffinity(0))
    limiter = threadpool_limits(limits=cores)       # BLAS threads = the cores this process has
    blas_threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    cpu_model = "unknown"
    with open("/proc/cpuinfo") as f:
        for line in f:
            if line.startswith("model name"):
                cpu_model = line.split(":", 1)[1].strip()
                break
    ctx = gen.context_lengths(w)
    table, P = gen.page_tables(w, ctx)
    pools = [gen.kv_pools(w, li, P, "cpu") for li in range(len(w.layers))]
    W = gen.lm_head_table(w, "cpu")
    W64 = W.double().numpy()                       # static weights: converted once, untimed
    temps = gen.row_temperatures(w)
    sigma = noise_sigma(w)
    tokens_out, t_total, steps = 0, 0.0, 0
    while steps < max_steps and (steps < 1 or t_total < seconds_target):
        x = gen.hidden_states(w, "cpu", step=steps)
        u = gen.uniforms(w, step=steps)
        # drafter stand-in (untimed): the shared table applied to a perturbed hidden state
        xd = (x.float() + sigma * gen.drafter_hidden_noise(w, "cpu", step=steps)).to(x.dtype)
        rows = [b * w.k1 + i for b in range(w.batch) for i in range(w.k)]
        zq = oracle.logits(xd, W64, rows=rows)
        qd = oracle.probabilities(zq, temps[rows]).astype(np.float32).reshape(w.batch, w.k, -1)
        draft = gen.draw_drafts(w, qd, gen.temperatures(w), step=steps)
        layers = [dict(q=gen.queries(w, li, "cpu", step=steps), k_pool=pools[li][0],
                       v_pool=pools[li][1], page_table=table, ctx_lens=ctx, window=L.window,
                       scale=1 / math.sqrt(L.head_dim)) for li, L in enumerate(w.layers)]
        t0 = time.perf_counter()
        _, _, _, n, _ = verify_step(layers, x, W64, temps, draft, qd, u)
        t_total += time.perf_counter() - t0
        tokens_out += int(np.sum(n + 1))
        steps += 1
    limiter.restore_original_limits()
    return {"value": tokens_out / t_total, "unit": "verified tokens/s", "cores": int(cores),
            "blas_threads": int(blas_threads), "cpu_model": cpu_model, "kind": "oracle",
            "sample": f"{steps} verify steps of the same workload (fp64 numpy oracle: attention, "
                      f"lm-head, softmax, accept; table converted to fp64 once, untimed), "
                      f"{t_total:.1f} s"}


def adjacent_calls(w, inp, lib, sv, gen, torch, device, sptr, dt, ws_attn, n_out, n0,
                   iters=200):
    """The calls on either side of the verify step, timed after it with HIP events on the
    same stream and pools: KV append of the K1 verified positions for every layer plus the
    commit, the drafter's cross-attention (one query per sequence and draft step, K1 = 1, over
    the committed context of the same pools), k draft steps per verify step, and the accept
    step with its uniforms read from an array or drawn in the kernels."""
    from speculative_decoding_decode_amd import _lib
    B, k, K1 = w.batch, w.k, w.k1
    esz = 2 if w.dtype == "bf16" else 4
    s0 = inp["sets"][0]
    ctx_c = (s0["ctx"] - K1).contiguous()                   # committed context of set 0
    ctx_scratch = s0["ctx"].clone()
    knew = [gen.normal_tensor((B, K1, L.hkv, L.head_dim), 99 + li, device, w.dtype)
            for li, L in enumerate(w.layers)]
    dq = [gen.drafter_queries(w, li, L.hq, 0, device) for li, L in enumerate(w.layers)]
    dout = [torch.empty((B, 1, L.hq, L.head_dim), dtype=torch.float32, device=device)
            for L in w.layers]
    ev = HipEvents(4)
    ev.record(0, sptr)
    for it in range(iters):
        for li, L in enumerate(w.layers):
            kp, vp = inp["pools"][li]
            rc = lib.spec_kv_append(knew[li].data_ptr(), knew[li].data_ptr(), kp.data_ptr(),
                                    vp.data_ptr(), s0["table"].data_ptr(), s0["ctx"].data_ptr(),
                                    B, K1, L.hkv, L.head_dim, w.page_size, inp["P"],
                                    inp["max_pages"], dt, sptr)
            if rc:
                _lib.check("spec_kv_append", rc)
        n_row = n_out[(n0 + it) % n_out.shape[0]]
        rc = lib.spec_kv_commit(ctx_scratch.data_ptr(), n_row.data_ptr(), B, K1, sptr)
        if rc:
            _lib.check("spec_kv_commit", rc)
    ev.record(1, sptr)
    for it in range(iters):
        for j in range(k):
            for li, L in enumerate(w.layers):
                kp, vp = inp["pools"][li]
                rc = lib.spec_verify_attn(
                    dq[li].data_ptr(), kp.data_ptr(), vp.data_ptr(), s0["table"].data_ptr(),
                    ctx_c.data_ptr(), dout[li].data_ptr(), B, 1, L.hq, L.hkv, L.head_dim,
                    w.page_size, inp["P"], inp["max_pages"], L.window,
                    1.0 / math.sqrt(L.head_dim), dt, ws_attn.data_ptr(), ws_attn.numel(), sptr)
                if rc:
                    _lib.check("spec_verify_attn", rc)
    ev.record(2, sptr)
    # the accept step with uniforms read from an array vs drawn in the kernels (Philox)
    probs = torch.empty((B * K1, w.vocab), dtype=torch.float32, device=device)
    _, probs = sv.lm_head(s0["x"], inp["W"], inp["temps"], probs=probs)
    pk = probs.view(B, K1, w.vocab)
    qd = s0["qd"] if k else None
    dr0 = torch.zeros((B, k), dtype=torch.int32, device=device)
    u0 = torch.from_numpy(gen.uniforms(w, step=0)).to(device)
    ws_acc = torch.zeros(sv.accept_workspace_bytes(B, k, w.vocab), dtype=torch.uint8, device=device)
    n_acc = torch.empty((B,), dtype=torch.int32, device=device)
    tok = torch.empty((B, K1), dtype=torch.int32, device=device)
    torch.cuda.synchronize(device)
    a_args = (dr0.data_ptr() if k else None, qd.data_ptr() if k else None, pk.data_ptr())
    a_tail = (n_acc.data_ptr(), tok.data_ptr(), B, k, w.vocab, ws_acc.data_ptr(), ws_acc.numel(),
              sptr)
    ev2 = HipEvents(3)
    ev2.record(0, sptr)
    for it in range(iters):
        rc = lib.spec_accept(*a_args, u0.data_ptr(), *a_tail)
        if rc:
            _lib.check("spec_accept", rc)
    ev2.record(1, sptr)
    for it in range(iters):
        rc = lib.spec_accept_philox(*a_args, 0x5EED, it, None, *a_tail)
        if rc:
            _lib.check("spec_accept_philox", rc)
    ev2.record(2, sptr)
    torch.cuda.synchronize(device)
    kv_us = ev.ms(0, 1) * 1e3 / iters
    dr_us = ev.ms(1, 2) * 1e3 / (iters * max(k, 1))
    acc_us, acc_ph_us = ev2.ms(0, 1) * 1e3 / iters, ev2.ms(1, 2) * 1e3 / iters
    ev.close()
    ev2.close()
    # algorithmic bytes: append reads and writes K1 rows of K and V per layer and sequence
    app_bytes = sum(2 * 2 * B * K1 * L.hkv * L.head_dim * esz for L in w.layers)
    ctx_committed = [int(c) - K1 for c in inp["ctx"]]
    dr_bytes = sum(visible_tokens(c, 1, L.window) * L.hkv * L.head_dim * esz * 2
                   for L in w.layers for c in ctx_committed)
    return {"kv_append_commit_us_per_step": round(kv_us, 2),
            "kv_append_bytes_per_step": app_bytes,
            "drafter_xattn_us_per_draft_step": round(dr_us, 2),
            "drafter_xattn_kv_bytes_per_draft_step": dr_bytes,
            "drafter_xattn_gbs": round(dr_bytes / (dr_us * 1e-6) / 1e9, 1),
            "accept_array_uniforms_us": round(acc_us, 2),
            "accept_philox_uniforms_us": round(acc_ph_us, 2),
            "iterations": iters}


def hbm_ceiling(torch, device, nbytes=2 << 30, reps=10):
    """HBM rates on this box of the library's plain streaming probes (spec_hbm_probe): a read
    of 2 GiB and a copy of 2 GiB (read + write bytes counted), 10 launches each, timed with HIP
    events on the current stream (the verify step's)."""
    from speculative_decoding_decode_amd import _lib
    lib = _lib.load()
    src = torch.ones(nbytes // 4, dtype=torch.float32, device=device)
    dst = torch.empty_like(src)
    sink = torch.empty(4 * lib.spec_hbm_probe_grid(), dtype=torch.int32, device=device)
    sptr = torch.cuda.current_stream(device).cuda_stream
    sptr = ctypes.c_void_p(sptr) if sptr else None

    def run(mode, out):
        rc = lib.spec_hbm_probe(mode, src.data_ptr(), out.data_ptr(), nbytes, sptr)
        if rc:
            _lib.check("spec_hbm_probe", rc)

    for _ in range(2):
        run(0, sink)
        run(1, dst)
    ev = HipEvents(3)
    ev.record(0, sptr)
    for _ in range(reps):
        run(0, sink)
    ev.record(1, sptr)
    for _ in range(reps):
        run(1, dst)
    ev.record(2, sptr)
    torch.cuda.synchronize(device)
    read_gbs = nbytes * reps / (ev.ms(0, 1) * 1e-3) / 1e9
    copy_gbs = 2 * nbytes * reps / (ev.ms(1, 2) * 1e-3) / 1e9
    ev.close()
    del src, dst
    return {"read_gbs": round(read_gbs, 1), "copy_gbs": round(copy_gbs, 1),
            "how": "spec_hbm_probe: 16-byte nontemporal streams over 2 GiB, read and copy "
                   "(read + write bytes), 10 launches each, HIP events"}


def measure(w, steps, warmup, device, two_calls=False):
    """Prepare w's input sets and time `steps` verify steps after `warmup` untimed ones.

    One step = spec_verify_attn per layer, then spec_lm_head_accept (the lm-head and the accept
    step in one call), or with `two_calls` spec_lm_head then spec_accept (the same results)."""
    import torch
    import speculative_decoding_decode_amd as sv
    from speculative_decoding_decode_amd import _lib
    from speculative_decoding_decode_amd.telemetry import accept_stats
    from workloads import gen, noise_sigma

    B, k, K1, V, H = w.batch, w.k, w.k1, w.vocab, w.hidden
    R = B * K1

    log(f"[bench] preparing input sets for {w.name}")
    inp = prepare(w, device, torch, sv, gen, noise_sigma)
    nsets = inp["nsets"]
    lib = _lib.load()
    stream = torch.cuda.current_stream(device)
    sptr = ctypes.c_void_p(stream.cuda_stream) if stream.cuda_stream else None
    nsteps = warmup + max(steps, BRACKET_MAX, 200)   # the timed steps and the passes after them
    U = torch.from_numpy(np.stack([gen.uniforms(w, step=1000 + s) for s in range(nsteps)])).to(device)
    Ud = torch.from_numpy(gen.rng(w, gen.STREAM_DRAFT, 0).random((nsteps, B * k, 1),
                                                                 dtype=np.float32)).to(device)
    drafts = torch.empty((nsteps, B, k), dtype=torch.int32, device=device)
    n_out = torch.empty((nsteps, B), dtype=torch.int32, device=device)
    tok_out = torch.empty((nsteps, B, K1), dtype=torch.int32, device=device)
    attn_out = [torch.empty((B, K1, L.hq, L.head_dim), dtype=torch.float32, device=device)
                for L in w.layers]
    probs = torch.empty((R, V), dtype=torch.float32, device=device)
    # workspaces allocated once, outside the timed region (the calls need no contents in them)
    ws_attn = torch.zeros(max(sv.verify_attn_workspace_bytes(B, K1, L.hq, L.hkv, L.head_dim,
                                                             inp["max_pages"], L.window)
                              for L in w.layers), dtype=torch.uint8, device=device)
    ws_lm = torch.zeros(sv.lm_head_workspace_bytes(R, H, V), dtype=torch.uint8, device=device)
    ws_acc = torch.zeros(sv.accept_workspace_bytes(B, k, V), dtype=torch.uint8, device=device)
    ws_fu = torch.zeros(sv.lm_head_accept_workspace_bytes(B, k, H, V), dtype=torch.uint8,
                        device=device)
    dt = sv.SPEC_BF16 if w.dtype == "bf16" else sv.SPEC_F32

    # argument tuples of the C calls for every input set (pointers only)
    calls = []
    for s in inp["sets"]:
        attn = []
        for li, L in enumerate(w.layers):
            kp, vp = inp["pools"][li]
            attn.append((s["q"][li].data_ptr(), kp.data_ptr(), vp.data_ptr(), s["table"].data_ptr(),
                         s["ctx"].data_ptr(), attn_out[li].data_ptr(), B, K1, L.hq, L.hkv,
                         L.head_dim, w.page_size, inp["P"], inp["max_pages"], L.window,
                         1.0 / math.sqrt(L.head_dim), dt, ws_attn.data_ptr(), ws_attn.numel(),
                         sptr))
        m = (s["x"].data_ptr(), inp["W"].data_ptr(), inp["temps"].data_ptr(), None,
             probs.data_ptr(), R, H, V, dt, ws_lm.data_ptr(), ws_lm.numel(), sptr)
        calls.append((attn, m, s["qd"].data_ptr() if k else None))

    def step(i, ev=None, evi=0):
        attn, m, q_ptr = calls[i % nsets]
        for a in attn:
            rc = lib.spec_verify_attn(*a)
            if rc:
                _lib.check("spec_verify_attn", rc)
        if ev is not None:
            lib.spec_profile_lm_head(ev.ev[evi], ev.ev[evi + 1])
        if not two_calls:
            rc = lib.spec_lm_head_accept(m[0], m[1], m[2], drafts[i].data_ptr() if k else None,
                                         q_ptr, U[i].data_ptr(), 0, 0, None, n_out[i].data_ptr(),
                                         tok_out[i].data_ptr(), B, k, H, V, dt, ws_fu.data_ptr(),
                                         ws_fu.numel(), sptr)
            if rc:
                _lib.check("spec_lm_head_accept", rc)
            return
        rc = lib.spec_lm_head(*m)
        if rc:
            _lib.check("spec_lm_head", rc)
        rc = lib.spec_accept(drafts[i].data_ptr() if k else None, q_ptr, probs.data_ptr(), U[i].data_ptr(),
                             n_out[i].data_ptr(), tok_out[i].data_ptr(), B, k, V,
                             ws_acc.data_ptr(), ws_acc.numel(), sptr)
        if rc:
            _lib.check("spec_accept", rc)

    # the drafter samples its drafts anew every step: d ~ q of that step's input set, drawn by
    # the accept call with k = 0 (plain sampling) before timing; the warm-up steps follow on the
    # stream without a host-side pause, so the GPU is busy from here to the timed region
    for i in range(nsteps if k else 0):
        qs = inp["sets"][i % nsets]["qd"]
        _, tok = sv.accept(None, None, qs.view(B * k, 1, V), Ud[i])
        drafts[i].copy_(tok[:, 0].view(B, k))
    # the HBM ceiling is measured here, right before the warm-up steps: ~11 ms of full-speed
    # streaming that brings the GPU to its steady clocks, so a short run (a few warm-up steps)
    # times the same step as a long one
    ceiling = hbm_ceiling(torch, device)
    log(f"[bench] warmup {warmup} steps ({nsets} input sets)")
    for i in range(warmup):
        step(i)
    torch.cuda.synchronize(device)

    # (1) the timed region: K steps, nothing else on the stream
    K = steps
    ev_tot = HipEvents(2)
    log(f"[bench] timing {K} steps")
    torch.cuda.synchronize(device)
    t0 = time.perf_counter()
    ev_tot.record(0, sptr)
    for j in range(K):
        step(warmup + j)
    ev_tot.record(1, sptr)
    torch.cuda.synchronize(device)
    t1 = time.perf_counter()
    wall = t1 - t0
    gpu_total_ms = ev_tot.ms(0, 1)
    ev_tot.close()
    n_all = n_out[warmup:warmup + K].cpu().numpy()
    tok_all = tok_out[warmup:warmup + K].cpu().numpy()

    # (2) the contraction kernel alone: a separate pass of the same steps with HIP events
    # recorded by the library right before and after that kernel on every step
    NB = max(BRACKET_MIN, min(K, BRACKET_MAX))
    ev_lm = HipEvents(2 * NB)
    for j in range(NB):
        step(warmup + j, ev_lm, 2 * j)
    torch.cuda.synchronize(device)
    lm_ms = np.array([ev_lm.ms(2 * j, 2 * j + 1) for j in range(NB)])
    ev_lm.close()

    # (3) distribution of single-step times: every step between two HIP events, less the
    # median time of an empty event pair (the events' own cost)
    P = min(200, max(steps, 50))
    ev_d = HipEvents(2 * P + 2 * 32)
    for j in range(32):
        ev_d.record(2 * P + 2 * j, sptr)
        ev_d.record(2 * P + 2 * j + 1, sptr)
    for j in range(P):
        ev_d.record(2 * j, sptr)
        step(warmup + j)
        ev_d.record(2 * j + 1, sptr)
    torch.cuda.synchronize(device)
    floor_ms = float(np.median([ev_d.ms(2 * P + 2 * j, 2 * P + 2 * j + 1) for j in range(32)]))
    step_us = np.array([ev_d.ms(2 * j, 2 * j + 1) - floor_ms for j in range(P)]) * 1e3
    ev_d.close()
    pct = {"p10": round(float(np.percentile(step_us, 10)), 2),
           "p50": round(float(np.percentile(step_us, 50)), 2),
           "p90": round(float(np.percentile(step_us, 90)), 2),
           "steps": P, "event_pair_floor_us": round(floor_ms * 1e3, 2)}

    # (4) warm run: the same input set on every step (its KV, queries and drafter rows stay in
    # the caches; the table, far larger than the caches, still streams from HBM)
    WM = max(50, min(K, 500))
    mult = -(-nsteps // nsets)          # steps i < nsteps with i % nsets == 0: set 0's inputs
    ev_w = HipEvents(2)
    ev_w.record(0, sptr)
    for j in range(WM):
        step((j % mult) * nsets)
    ev_w.record(1, sptr)
    torch.cuda.synchronize(device)
    warm_us = ev_w.ms(0, 1) * 1e3 / WM
    ev_w.close()

    assert ((tok_all >= -1) & (tok_all < V)).all()
    emitted = int(np.sum(n_all + 1))
    stats = accept_stats(n_all, k)
    # expected tokens of exactly the timed steps' input sets (closed form of their rows)
    exp_tok = float(sum(inp["expected_tokens"][(warmup + j) % nsets].sum() for j in range(K)))
    value = exp_tok / wall
    value_sampled = emitted / wall
    kv_bytes, table_bytes = algorithmic_bytes(w, inp["ctx"])
    step_bytes = kv_bytes + table_bytes
    ms_per_step = wall * 1e3 / K
    lm_avg_ms = float(lm_ms.mean())
    achieved = table_bytes / (lm_avg_ms * 1e-3) / 1e9
    traffic_bytes = profiled_traffic(w.name)
    traffic = None if traffic_bytes is None else round(traffic_bytes / (lm_avg_ms * 1e-3) / 1e9, 1)
    step_gbs = step_bytes / (ms_per_step * 1e-3) / 1e9
    log(f"[bench] gpu {gpu_total_ms * 1e3 / K:.1f} us/step; lm-head contraction "
        f"{lm_avg_ms * 1e3:.1f} us = {achieved:.0f} GB/s; wall {ms_per_step * 1e3:.1f} us/step; "
        f"warm {warm_us:.1f} us/step; expected tokens/step {exp_tok / K:.4f}, sampled "
        f"{emitted / K:.4f}; acceptance pos {stats.per_position}")

    return dict(inp=inp, lib=lib, sptr=sptr, dt=dt, ws_attn=ws_attn, n_out=n_out, wall=wall,
                value=value, value_sampled=value_sampled, ms_per_step=ms_per_step,
                lm_avg_ms=lm_avg_ms, lm_launches=NB, achieved=achieved, traffic=traffic,
                traffic_bytes=traffic_bytes, step_gbs=step_gbs, step_bytes=step_bytes,
                table_bytes=table_bytes, gpu_total_ms=gpu_total_ms, stats=stats, nsets=nsets,
                step_us_percentiles=pct, warm_us=warm_us, tokens_expected=exp_tok / K,
                tokens_sampled=emitted / K, ceiling=ceiling)


def lm_head_rows(device, reps=30):
    """The lm-head contraction at 1..8 rows over 2560- and 5376-wide bf16 tables of 262144 rows,
    timed inside the call the verify step makes (spec_lm_head_accept for one sequence with k =
    R - 1 drafts: contraction, row statistics, accept): the contraction kernel's time per launch
    (HIP events the library records around it), for the library loaded (SPEC_VERIFY_LIB may name
    a build whose GEMV serves other row counts, so that both kernels can be timed at every row
    count).  Each shape runs 3 untimed and `reps` timed calls."""
    import torch
    import speculative_decoding_decode_amd as sv
    from speculative_decoding_decode_amd import _lib
    lib = _lib.load()
    V = 262144
    out = {}
    for H in (2560, 5376):
        g = torch.Generator(device=device).manual_seed(H)
        W = (torch.randn(V, H, generator=g, device=device) / math.sqrt(H)).to(torch.bfloat16)
        for R in range(1, 9):
            k = R - 1
            x = torch.randn(R, H, generator=g, device=device).to(torch.bfloat16)
            t = torch.ones(R, device=device)
            draft = torch.randint(0, V, (1, k), generator=g, device=device, dtype=torch.int32)
            q = torch.softmax(torch.randn(1, k, V, generator=g, device=device), dim=-1) if k else None
            u = torch.rand(1, R, generator=g, device=device)
            n_acc = torch.empty(1, dtype=torch.int32, device=device)
            tok = torch.empty(1, R, dtype=torch.int32, device=device)
            ws = torch.zeros(sv.lm_head_accept_workspace_bytes(1, k, H, V), dtype=torch.uint8,
                             device=device)
            call = lambda: sv.lm_head_accept(x, W, t, draft, q, uniforms=u, n_accepted=n_acc,
                                             tokens=tok, workspace=ws)
            for _ in range(3):
                call()
            ev = HipEvents(2 * reps)
            for i in range(reps):
                lib.spec_profile_lm_head(ev.ev[2 * i], ev.ev[2 * i + 1])
                call()
            torch.cuda.synchronize(device)
            us = float(np.mean([ev.ms(2 * i, 2 * i + 1) for i in range(reps)]) * 1e3)
            ev.close()
            out[f"{H}x{R}"] = round(us, 2)
            log(f"[bench] lm-head H={H} R={R}: {us:.1f} us ({V * H * 2 / (us * 1e-6) / 1e9:.0f} GB/s)")
        del W
    print(json.dumps({"metric": "lm-head contraction time per launch inside spec_lm_head_accept, "
                                "bf16 table 262144 rows",
                      "unit": "us", "library": _lib.LIB_PATH, "times": out}), flush=True)


def sweep_k(w, kmax, steps, warmup, device):
    """The workload's verify step at k = 0..kmax drafts (plain decoding at k = 0): measured step
    time and tokens per step at every k, the verified tokens per second they give, and the k
    the telemetry picks (highest throughput; where the tokens per step plateau)."""
    from speculative_decoding_decode_amd.telemetry import choose_k, mal_from_positions
    us, mal, pos, lm = {}, {}, {}, {}
    for k in range(kmax + 1):
        wk = dataclasses.replace(w, k=k)
        log(f"[bench] sweep: k = {k}")
        r = measure(wk, steps, warmup, device)
        us[k] = r["ms_per_step"] * 1e3
        lm[k] = r["lm_avg_ms"] * 1e3
        mal[k] = r["stats"].mean_accepted_length
        pos[k] = [round(a, 4) for a in r["stats"].per_position]
        del r
    # tokens per step at every k from the per-position rates of the k = kmax run (one set of
    # draws, so the curve is not perturbed by each run's own sampling noise)
    derived = {k: mal_from_positions(pos[kmax], k) for k in range(kmax + 1)}
    c = choose_k(derived, {k: v * 1e-6 for k, v in us.items()})
    print(json.dumps({
        "metric": f"verify step vs k, {w.description}",
        "unit": "verified tokens/s", "n_gpus": 1, "steps": steps, "warmup": warmup,
        "config": {"workload": w.name, "k": list(range(kmax + 1))},
        "us_per_step": [round(us[k], 2) for k in range(kmax + 1)],
        "lm_head_us_per_launch": [round(lm[k], 2) for k in range(kmax + 1)],
        "tokens_per_step": [round(derived[k], 4) for k in range(kmax + 1)],   # per sequence
        "tokens_per_step_measured_at_k": [round(mal[k], 4) for k in range(kmax + 1)],
        "verified_tokens_per_s": [round(w.batch * c.tokens_per_second[k], 1) for k in range(kmax + 1)],
        "acceptance_per_position_at_kmax": pos[kmax],
        "best_k": c.best_k, "plateau_k": c.plateau_k}), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--two-calls", action="store_true",
                    help="run the lm-head and the accept step as spec_lm_head + spec_accept "
                         "instead of spec_lm_head_accept (same results; for comparison)")
    ap.add_argument("--sweep-k", type=int, default=None, metavar="KMAX",
                    help="time the workload's verify step at k = 0..KMAX drafts and print the "
                         "tokens-per-step curve, throughput per k and the chosen k (one JSON line)")
    ap.add_argument("--lm-head-rows", action="store_true",
                    help="only time the lm-head contraction at 1..8 rows over 2560- and 5376-wide "
                         "tables (one JSON line)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain 1 GiB device copy 10 times (the reference kernel that "
                         "scales rocprofv3 FETCH_SIZE / WRITE_SIZE counters to bytes)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported (the verify step "
              f"runs on a single MI355X).", file=sys.stderr)
        sys.exit(2)

    import torch
    import speculative_decoding_decode_amd as sv
    from speculative_decoding_decode_amd import _lib
    from speculative_decoding_decode_amd.telemetry import accept_stats
    from workloads import WORKLOADS, gen, noise_sigma

    if not torch.cuda.is_available():
        raise RuntimeError("bench.py needs a GPU")
    if args.calibrate_copy:
        src = torch.ones(1 << 28, dtype=torch.float32, device="cuda")     # 1 GiB
        dst = torch.empty_like(src)
        for _ in range(10):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_per_dispatch": src.numel() * 4, "dispatches": 10}))
        return
    if not os.path.exists(_lib.LIB_PATH):
        from speculative_decoding_decode_amd import build
        build.build()
    device = torch.device("cuda", 0)
    torch.cuda.set_device(device)
    w = WORKLOADS[args.workload]
    B, k, K1, V, H = w.batch, w.k, w.k1, w.vocab, w.hidden
    if args.sweep_k is not None:
        sweep_k(w, args.sweep_k, args.steps, args.warmup, device)
        return
    if args.lm_head_rows:
        lm_head_rows(device)
        return
    r = measure(w, args.steps, args.warmup, device, two_calls=args.two_calls)
    inp, lib, sptr, dt, ws_attn, n_out = r["inp"], r["lib"], r["sptr"], r["dt"], r["ws_attn"], r["n_out"]
    value, ms_per_step, lm_avg_ms, achieved = r["value"], r["ms_per_step"], r["lm_avg_ms"], r["achieved"]
    traffic, traffic_bytes, step_gbs = r["traffic"], r["traffic_bytes"], r["step_gbs"]
    step_bytes, table_bytes, gpu_total_ms, stats = r["step_bytes"], r["table_bytes"], r["gpu_total_ms"], r["stats"]
    nsets, pct = r["nsets"], r["step_us_percentiles"]
    K = args.steps
    ceiling = r["ceiling"]

    adjacent = adjacent_calls(w, inp, lib, sv, gen, torch, device, sptr, dt, ws_attn, n_out,
                              args.warmup)

    cpu = None
    if not args.no_cpu_baseline:
        log("[bench] cpu baseline (fp64 oracle)")
        cpu = cpu_baseline(w, gen)

    Ls = w.layers
    result = {
        "metric": METRIC if w.name == DEFAULT_WORKLOAD else
        f"verified tokens/sec and verify-step HBM GB/s (% peak), {w.description}",
        "value": round(value, 2),
        "unit": "verified tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": w.name, "batch": B, "k": k, "verified_positions": K1,
                   "lm_head_accept": "spec_lm_head + spec_accept" if args.two_calls
                   else "spec_lm_head_accept",
                   "ctx": [int(c) for c in inp["ctx"]] if B <= 8 else
                   {"min": int(inp["ctx"].min()), "max": int(inp["ctx"].max()),
                    "mean": float(inp["ctx"].mean())},
                   "attention": [f"{L.kind} hd{L.head_dim}" + (f" window {L.window}" if L.window else "")
                                 + f", {L.hq}q/{L.hkv}kv, 16-token pages" for L in Ls],
                   "lm_head": f"{H} x {V} {w.dtype}", "input_sets": nsets},
        "step_hbm_gbs": round(step_gbs, 1),
        "step_frac_peak": round(step_gbs / HBM_PEAK_GBS, 4),
        "step_algorithmic_bytes": step_bytes,
        "gpu_event_ms_per_step": round(gpu_total_ms / K, 5),
        "step_us_percentiles": pct,
        "tokens_per_step": round(r["tokens_expected"], 4),
        "tokens_per_step_basis": "closed form E[n+1] = 1 + sum_j prod_{i<=j} sum_v min(p_i, q_i) "
                                 "of each timed step's input set; value = B x that / wall time",
        "value_sampled": round(r["value_sampled"], 2),
        "tokens_per_step_sampled": round(r["tokens_sampled"], 4),
        "warm_ms_per_step": round(r["warm_us"] * 1e-3, 5),
        "acceptance_per_position": [round(a, 4) for a in stats.per_position],
        "closed_form_acceptance_per_position": [round(a, 4) for a in inp["alpha_pos"]],
        "roofline": {"kernel": "lm-head vocab-table contraction", "bound": "hbm",
                     "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                     "traffic_bytes_per_launch": traffic_bytes,
                     "bytes_per_launch": table_bytes, "avg_launch_us": round(lm_avg_ms * 1e3, 2),
                     "launches_timed": int(r["lm_launches"]),
                     "frac_of_measured_read": round(achieved / ceiling["read_gbs"], 4)},
        "hbm_ceiling": ceiling,
        "adjacent": adjacent,
        "cpu_baseline": cpu,
    }
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
