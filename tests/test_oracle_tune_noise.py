"""Pins of oracle.tune_noise, the script that sets the workloads' logit-noise scales (the pages'
acceptance targets: the serving guide's section 2 G4 table, pos0 about 47%, and its section 6
telemetry band, about 35% overall).

* sigma = 0 gives p = q, so every draft is accepted: mean acceptance exactly 1;
* the closed form sum_v min(p, q) it averages agrees with the acceptance frequency of the
  sampling rule itself (draw d ~ q, accept iff u * q(d) < p(d)), estimated by Monte Carlo;
* the bisection returns a scale whose acceptance equals the target, on a small vocabulary, and
  acceptance falls as sigma grows;
* the committed scales reproduce the committed acceptance at the full 262144-entry vocabulary.
"""
import json
import math
import os

import numpy as np

from oracle import tune_noise
from oracle.lm_head import probabilities

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def small_rows(rows=6, vocab=300, seed=5):
    g = np.random.Generator(np.random.Philox(seed))
    return g.standard_normal((rows, vocab)), g.standard_normal((rows, vocab))


def test_zero_noise_accepts_everything():
    base, noise = small_rows()
    assert abs(tune_noise.mean_acceptance(0.0, base, noise) - 1.0) < 1e-12


def test_closed_form_matches_sampled_acceptance():
    base, noise = small_rows(rows=1, vocab=50, seed=9)
    sigma = 1.2
    q = probabilities(base, [1.0])[0]
    p = probabilities(base + sigma * noise, [1.0])[0]
    rng = np.random.default_rng(17)
    n = 400_000
    d = rng.choice(q.size, size=n, p=q / q.sum())
    u = rng.random(n)
    freq = float(np.mean(u * q[d] < p[d]))
    a = tune_noise.mean_acceptance(sigma, base, noise)
    sd = math.sqrt(a * (1 - a) / n)
    assert abs(freq - a) < 4 * sd, (freq, a, sd)


def test_bisection_hits_the_target_and_acceptance_falls():
    base, noise = small_rows()
    grid = [0.2, 0.5, 1.0, 2.0, 4.0]
    acc = [tune_noise.mean_acceptance(s, base, noise) for s in grid]
    assert all(x > y for x, y in zip(acc, acc[1:]))
    for target in (0.47, 0.4747):
        s = tune_noise.bisect(target, base, noise)
        assert abs(tune_noise.mean_acceptance(s, base, noise) - target) < 1e-6


def test_committed_scales_reproduce_their_acceptance():
    with open(os.path.join(ROOT, "workloads", "noise_sigma.json")) as f:
        table = json.load(f)
    e = table["pos0_047"]
    g = np.random.Generator(np.random.Philox(e["seed"]))
    base = g.standard_normal((e["rows"], e["vocab"]))
    noise = g.standard_normal((e["rows"], e["vocab"]))
    for key in ("pos0_047", "overall_035"):
        got = tune_noise.mean_acceptance(table[key]["sigma"], base, noise)
        assert abs(got - table[key]["per_position_acceptance"]) < 1e-5, (key, got)
    # the 35%-overall entry: equal per-position acceptance a with (a + a^2) / 2 = 0.35
    a = table["overall_035"]["per_position_acceptance"]
    assert abs((a + a * a) / 2 - 0.35) < 1e-6
