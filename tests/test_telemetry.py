"""The telemetry reproduces the serving guide's printed G4 numbers from synthetic counts
(fixture tests/golden/g4_mtp_table.json, with its citation): 1 + 0.47 + 0.24 = 1.71 tokens per
step at k = 2, and (1.71 - 1) / 2 = 35.5% overall acceptance, inside the 34-36% band."""
import json
import os

import numpy as np

from speculative_decoding_decode_amd.telemetry import accept_stats, expected_tokens_per_step

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
