"""Find the logit-noise scale that gives a stated acceptance rate; writes
workloads/noise_sigma.json.

TEST INFRASTRUCTURE (see oracle/__init__.py): a committed script that calls only this package.

Targets (the serving guide's G4 measurements, [guide] §2 and §6 telemetry table):
  pos0_047     acceptance at the first draft position about 47%;
  overall_035  about 35% overall acceptance at k = 2 (the 34-36% reference band).  With the
               same per-position acceptance a at both positions, overall = (a + a^2) / 2, so
               a = (sqrt(1 + 8 * 0.35) - 1) / 2.
Recipe: drafter logits z_q ~ N(0, 1), target logits z_p = z_q + N(0, sigma^2), temperature 1,
vocabulary 262144; the acceptance of one row is the closed form sum_v min(p, q).  sigma is
bisected on the mean over 64 seeded rows (the same rows at every sigma).

Run:  python -m oracle.tune_noise
"""
from __future__ import annotations

import json
import math
import os
import sys

import numpy as np

from .lm_head import probabilities
from .accept import acceptance_probability

VOCAB = 262144
ROWS = 64
SEED = 20260505


def mean_acceptance(sigma: float, base: np.ndarray, noise: np.ndarray) -> float:
    acc = []
    for r in range(base.shape[0]):
        q = probabilities(base[r:r + 1], [1.0])[0]
        p = probabilities(base[r:r + 1] + sigma * noise[r:r + 1], [1.0])[0]
        acc.append(acceptance_probability(p, q))
    return float(np.mean(acc))


def bisect(target: float, base, noise, lo=0.01, hi=8.0, iters=40) -> float:
    # acceptance falls as sigma grows
    for _ in range(iters):
        mid = 0.5 * (lo + hi)
        if mean_acceptance(mid, base, noise) > target:
            lo = mid
        else:
            hi = mid
    return 0.5 * (lo + hi)


def main(path=None):
    g = np.random.Generator(np.random.Philox(SEED))
    base = g.standard_normal((ROWS, VOCAB))
    noise = g.standard_normal((ROWS, VOCAB))
    a35 = (math.sqrt(1 + 8 * 0.35) - 1) / 2
    out = {}
    for key, target in (("pos0_047", 0.47), ("overall_035", a35)):
        s = bisect(target, base, noise)
        out[key] = {"sigma": round(s, 6), "per_position_acceptance": round(target, 6),
                    "achieved": round(mean_acceptance(s, base, noise), 6),
                    "rows": ROWS, "vocab": VOCAB, "seed": SEED}
    path = path or os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                                "workloads", "noise_sigma.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")
    return out


if __name__ == "__main__":
    print(json.dumps(main(sys.argv[1] if len(sys.argv) > 1 else None), indent=1))
