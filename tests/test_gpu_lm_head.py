"""GPU parity of spec_lm_head (MFMA contraction + row softmax) against the fp64 oracle."""
import math

import numpy as np
import pytest
import torch

import oracle
import speculative_decoding_decode_amd as sv
from workloads import WORKLOADS, gen
from cases import TOL, REG_TOL, P_TOL, say, dev

pytestmark = pytest.mark.gpu


def run_and_compare(x, w, temps, dtype, rows=None, label=""):
    d = dev()
    say(f"[lm_head] {label}: R={x.shape[0]} H={x.shape[1]} V={w.shape[0]} {dtype}")
    t = torch.as_tensor(np.asarray(temps, np.float32), device=d)
    logits, p = sv.lm_head(x.to(d), w.to(d), t, want_logits=True)
    _, p2 = sv.lm_head(x.to(d), w.to(d), t)            # logits not stored: same p
    torch.cuda.synchronize()
    assert torch.equal(p, p2)
    rows = list(range(x.shape[0])) if rows is None else rows
    z_ref = oracle.logits(x.cpu(), w.cpu(), rows=rows)
    p_ref = oracle.probabilities(z_ref, np.asarray(temps)[rows])
    z = logits.cpu().numpy()[rows].astype(np.float64)
    pg = p.cpu().numpy()[rows].astype(np.float64)
    ez, ep = np.abs(z - z_ref).max(), np.abs(pg - p_ref).max()
    say(f"    max |logit err| = {ez:.3e}   max |p err| = {ep:.3e}")
    assert ez <= TOL[dtype]
    assert ez <= REG_TOL[dtype]
    assert ep <= P_TOL
    np.testing.assert_allclose(pg.sum(axis=1), 1.0, atol=1e-5)
    for i, r in enumerate(rows):
        if not temps[r] > 0:   # greedy: one-hot at an index whose oracle logit is maximal
            j = int(np.argmax(pg[i]))
            assert pg[i, j] == 1.0 and pg[i].sum() == 1.0
            assert z_ref[i, j] >= z_ref[i].max() - TOL[dtype]


def test_tiny_fp32_workload():
    w = WORKLOADS["tiny_fp32_b1_k2"]
    x = gen.hidden_states(w)
    W = gen.lm_head_table(w)
    run_and_compare(x, W, [1.0, 0.0, 0.5], "f32", label="tiny fp32")


@pytest.mark.parametrize("R,H,V,dtype", [(19, 264, 5003, "bf16"), (5, 8, 17, "f32"),
                                          (130, 64, 1000, "bf16"), (1, 512, 4100, "f32"),
                                          (33, 2568, 2048, "bf16"), (20, 200, 777, "f32"),
                                          (97, 136, 700, "bf16"), (40, 64, 100, "bf16"),
                                          (96, 72, 1536, "f32"), (2, 2568, 3000, "bf16"),
                                          (2, 5376, 1500, "bf16"), (4, 2560, 2000, "bf16"),
                                          (1, 2560, 3001, "bf16"), (3, 2560, 4097, "bf16"),
                                          (3, 5376, 2500, "bf16"), (1, 5376, 777, "bf16"),
                                          (2, 8, 100, "bf16"), (3, 24, 65, "f32"),
                                          (1, 8, 1, "bf16"),
                                          # bf16 MFMA with table fragments from HBM: hidden
                                          # widths below one 128-byte chunk, a 256-byte
                                          # super-chunk (5-6 hidden tiles) with a tail
                                          (5, 8, 300, "bf16"), (20, 24, 1000, "bf16"),
                                          (70, 328, 2100, "bf16"), (96, 5376, 1100, "bf16"),
                                          (200, 200, 600, "bf16"),
                                          # the GEMV's most rows and the MFMA path just
                                          # above, at a wide table
                                          (5, 4104, 1000, "bf16"), (6, 4104, 700, "bf16")])
def test_ragged_shapes(R, H, V, dtype):
    torch.manual_seed(R * 7 + V)
    td = torch.float32 if dtype == "f32" else torch.bfloat16
    x = torch.randn(R, H).to(td)
    W = (torch.randn(V, H) / math.sqrt(H)).to(td)
    temps = [(0.0, 0.7, 1.0, 2.0)[r % 4] for r in range(R)]
    run_and_compare(x, W, temps, dtype, label="ragged")


@pytest.mark.parametrize("R", [2, 6, 20])     # GEMV and MFMA paths
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_greedy_ties_take_first_index(R, dtype):
    d = dev()
    x = torch.ones(R, 16, dtype=dtype)
    W = torch.zeros(600, 16, dtype=dtype)
    W[[7, 300, 599]] = 1.0                         # three equal maxima across blocks
    t = torch.zeros(R, device=d)
    _, p = sv.lm_head(x.to(d), W.to(d), t)
    pc = p.cpu()
    assert pc[:, 7].tolist() == [1.0] * R and float(pc.sum()) == float(R)


@pytest.mark.parametrize("R", [2, 3, 4, 5, 6, 20])  # the GEMV (two to five rows), the MFMA path
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("ties", [[45, 13, 2, 3, 130], [50, 33, 17], [1, 0], [255, 64, 128, 192],
                                  [63, 62, 61, 48, 47, 31, 16, 15]])
def test_greedy_ties_within_a_wave(R, dtype, ties):
    # equal maxima on lanes of one 64-row wave in different quads, half rows and rows of 16,
    # and across the waves of one block: the lowest index wins every reduction step
    d = dev()
    x = torch.ones(R, 16, dtype=dtype)
    W = torch.zeros(600, 16, dtype=dtype)
    W[ties] = 1.0
    W[400] = 0.5                                   # a smaller value elsewhere
    t = torch.zeros(R, device=d)
    _, p = sv.lm_head(x.to(d), W.to(d), t)
    pc = p.cpu()
    want = min(ties)
    assert pc[:, want].tolist() == [1.0] * R and float(pc.sum()) == float(R)


@pytest.mark.parametrize("greedy_rows", [[20, 49], [], list(range(50)), [0]])
def test_greedy_rows_in_some_row_tiles(greedy_rows):
    # greedy and tempered rows mixed over the 16-row tiles of the MFMA path: tiles without a
    # greedy row, tiles with one, every row greedy, none greedy
    torch.manual_seed(11)
    R, H, V = 50, 72, 1300
    x = torch.randn(R, H).to(torch.bfloat16)
    W = (torch.randn(V, H) / math.sqrt(H)).to(torch.bfloat16)
    temps = [0.0 if r in greedy_rows else (0.7, 1.0, 2.0)[r % 3] for r in range(R)]
    run_and_compare(x, W, temps, "bf16", label="greedy tiles")


def test_max_rows_per_call():
    # 65535 rows, the most one call takes: 683 passes of the MFMA contraction and the wide
    # finalize chunks (more than 2048 finalize workgroups)
    torch.manual_seed(65535)
    R, H, V = 65535, 16, 300
    x = torch.randn(R, H).to(torch.bfloat16)
    W = (torch.randn(V, H) / math.sqrt(H)).to(torch.bfloat16)
    temps = [0.0 if r % 7 == 0 else (0.7, 1.0, 2.0)[r % 3] for r in range(R)]
    run_and_compare(x, W, temps, "bf16", label="max rows")


@pytest.mark.parametrize("name", ["b1_k2_sliding256_8k", "b1_k4_global512_32k"])
def test_full_size_batch1(name):
    w = WORKLOADS[name]
    d = dev()
    x = gen.hidden_states(w, d)
    W = gen.lm_head_table(w, d)
    temps = gen.row_temperatures(w)
    run_and_compare(x, W, temps, "bf16", label=name)


@pytest.mark.parametrize("name", ["b8_ragged_k5_hybrid", "b32_k2_mixed_16k"])
def test_full_size_batched_sampled_rows(name):
    w = WORKLOADS[name]
    d = dev()
    x = gen.hidden_states(w, d)
    W = gen.lm_head_table(w, d)
    temps = gen.row_temperatures(w)
    rows = sorted(set([0, 1, w.rows // 2, w.rows - 1, 17 % w.rows, 40 % w.rows]))
    run_and_compare(x, W, temps, "bf16", rows=rows, label=name)
