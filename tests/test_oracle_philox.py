"""Pins for the oracle's Philox4x32-10 and its uniform draws."""
import json
import os

import numpy as np
from scipy import stats

from oracle.philox import draw_counter, philox4x32_10, uniform_draw

HERE = os.path.dirname(os.path.abspath(__file__))


def test_known_answer_vectors():
    with open(os.path.join(HERE, "golden", "philox4x32_10_kat.json")) as f:
        kat = json.load(f)
    for v in kat["vectors"]:
        ctr = [int(w, 16) for w in v["counter"]]
        key = [int(w, 16) for w in v["key"]]
        want = tuple(int(w, 16) for w in v["output"])
        assert philox4x32_10(ctr, key) == want


def test_counter_layout():
    ctr, key = draw_counter(seed=0x1122334455667788, offset=0x0000000500000007, b=3, node=9, purpose=1)
    assert key == (0x55667788, 0x11223344)
    assert ctr == (9, 3, 1 + 2 * 5, 7)


def test_uniform_is_24_bit_and_in_range():
    for node in range(50):
        u = uniform_draw(7, 11, 2, node, 0)
        assert 0.0 <= u < 1.0
        assert float(np.float32(u)) == u  # exact in float32
        assert (u * 2 ** 24) == int(u * 2 ** 24)


def test_draws_depend_on_every_counter_field():
    base = uniform_draw(1, 0, 0, 0, 0)
    others = [uniform_draw(2, 0, 0, 0, 0), uniform_draw(1, 1, 0, 0, 0), uniform_draw(1, 0, 1, 0, 0),
              uniform_draw(1, 0, 0, 1, 0), uniform_draw(1, 0, 0, 0, 1), uniform_draw(1, 1 << 32, 0, 0, 0)]
    assert all(o != base for o in others)


def test_uniformity_chi_square():
    n = 20000
    u = np.array([uniform_draw(12345, k, 0, 0, 0) for k in range(n)])
    counts = np.histogram(u, bins=20, range=(0, 1))[0]
    assert stats.chisquare(counts).pvalue > 1e-3
    # independence of neighbouring counters: lag-1 correlation near 0
    assert abs(np.corrcoef(u[:-1], u[1:])[0, 1]) < 4 / np.sqrt(n)
