"""Pins of the oracle's Philox4x32-10 (oracle/philox.py): the published known-answer vectors
(tests/golden/philox4x32_10_kat.json, with its citation), and properties of the uniforms."""
import json
import os

import numpy as np

from oracle import philox

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "philox4x32_10_kat.json")


def test_known_answer_vectors():
    for v in json.load(open(GOLDEN))["vectors"]:
        out = philox.philox4x32_10([int(x, 16) for x in v["counter"]], [int(x, 16) for x in v["key"]])
        assert [f"{w:08x}" for w in out] == v["output"]


def test_uniforms_grid_and_layout():
    u = philox.uniforms(seed=0x1234_5678_9ABC_DEF0, offset=7, B=3, K1=6)
    assert u.dtype == np.float32 and u.shape == (3, 6)
    m = u.astype(np.float64) * 2 ** 24
    assert np.all(m == np.floor(m)) and np.all((u >= 0) & (u < 1))
    # word i mod 4 of block i div 4: position 5 is word 1 of the second counter block
    key = (0x9ABC_DEF0, 0x1234_5678)
    w = philox.philox4x32_10((1, 2, 7, 0), key)
    assert u[2, 5] == np.float32((w[1] >> 8) * 2.0 ** -24)
    # different offsets / sequences give different draws
    assert not np.array_equal(u, philox.uniforms(0x1234_5678_9ABC_DEF0, 8, 3, 6))
    assert len(set(u.reshape(-1).tolist())) == u.size


def test_uniforms_are_uniform():
    u = philox.uniforms(seed=42, offset=0, B=4000, K1=4).reshape(-1).astype(np.float64)
    n = u.size
    assert abs(u.mean() - 0.5) < 4 * np.sqrt(1 / 12 / n)
    hist = np.histogram(u, bins=16, range=(0, 1))[0]
    chi2 = float(((hist - n / 16) ** 2 / (n / 16)).sum())
    assert chi2 < 40.0          # 15 degrees of freedom: p ~ 5e-4
