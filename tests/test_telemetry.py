"""The telemetry reproduces the serving guide's printed G4 numbers from synthetic counts
(fixture tests/golden/g4_mtp_table.json, with its citation): 1 + 0.47 + 0.24 = 1.71 tokens per
step at k = 2, and (1.71 - 1) / 2 = 35.5% overall acceptance, inside the 34-36% band."""
import json
import os

import numpy as np

from speculative_decoding_decode_amd.telemetry import (accept_stats, choose_k,
                                                       expected_tokens_per_step,
                                                       mal_from_positions)

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "g4_mtp_table.json")


def test_g4_table_arithmetic():
    g = json.load(open(GOLDEN))
    pos0, pos1 = g["per_position_acceptance_k2"]
    # 100 steps: 53 reject at position 0, 23 accept one draft, 24 accept both
    n = np.array([0] * 53 + [1] * 23 + [2] * 24)
    s = accept_stats(n, 2)
    assert abs(s.per_position[0] - pos0) < 1e-12 and abs(s.per_position[1] - pos1) < 1e-12
    assert abs(s.mean_accepted_length - g["tokens_per_step"]["2"]) < 1e-12
    lo, hi = g["overall_acceptance_band"]
    assert lo <= s.overall_acceptance <= hi
    assert abs(s.overall_acceptance - 0.355) < 1e-12
    assert g["mal_band_k2"][0] <= s.mean_accepted_length <= g["mal_band_k2"][1]
    assert s.alarms == []
    # k = 0 baseline: one token per step
    assert accept_stats(np.zeros(10, int), 0).mean_accepted_length == g["tokens_per_step"]["0"]


def test_alarms():
    drift = accept_stats(np.array([0] * 80 + [1] * 10 + [2] * 10), 2)
    assert any("20%" in a for a in drift.alarms)
    low = accept_stats(np.array([0] * 56 + [1] * 39 + [2] * 5), 2)
    assert any("reduce k" in a for a in low.alarms)
    assert any("25%" in a for a in low.alarms)


def test_iid_closed_form():
    assert abs(expected_tokens_per_step(0.47, 2) - (1 + 0.47 + 0.47 ** 2)) < 1e-15
    assert expected_tokens_per_step(0.0, 5) == 1.0


def test_mal_from_positions_matches_the_g4_table():
    g = json.load(open(GOLDEN))
    pos = g["per_position_acceptance_k2"]
    assert mal_from_positions(pos, 0) == g["tokens_per_step"]["0"]
    assert abs(mal_from_positions(pos, 2) - g["tokens_per_step"]["2"]) < 1e-12
    # the k = 1 run of the table (1.45) sits within 0.02 of 1 + pos0 (1.47): measured separately
    assert abs(mal_from_positions(pos, 1) - g["tokens_per_step"]["1"]) <= 0.02 + 1e-12
    # the same counts, read at k = 1 and k = 2, agree with accept_stats
    n = np.array([0] * 53 + [1] * 23 + [2] * 24)
    assert abs(mal_from_positions(accept_stats(n, 2).per_position, 2)
               - accept_stats(n, 2).mean_accepted_length) < 1e-12


def test_choose_k():
    # geometric acceptance 0.47 per position; step time growing with k
    mal = {k: expected_tokens_per_step(0.47, k) for k in range(6)}
    t = {0: 198e-6, 1: 201e-6, 2: 205e-6, 3: 215e-6, 4: 230e-6, 5: 250e-6}
    c = choose_k(mal, t)
    assert c.best_k == 3 and c.plateau_k == 3                   # 0.47^4 = 0.049 < 0.05
    expect = {k: mal[k] / t[k] for k in t}
    assert all(abs(c.tokens_per_second[k] - expect[k]) < 1e-9 for k in t)
    # flat step time: every extra draft pays, best is the largest k
    assert choose_k(mal, {k: 1.0 for k in mal}).best_k == 5
    # a drafter that is never accepted: plain decoding wins, the curve is flat from k = 0
    c0 = choose_k({k: 1.0 for k in range(4)}, {0: 1.0, 1: 1.1, 2: 1.2, 3: 1.3})
    assert c0.best_k == 0 and c0.plateau_k == 0
    # the G4 table's k = 1, 2 with equal step times: k = 2 (1.71 tokens per step)
    g = json.load(open(GOLDEN))
    tab = {int(k): v for k, v in g["tokens_per_step"].items()}
    assert choose_k(tab, {k: 1.0 for k in tab}).best_k == 2
