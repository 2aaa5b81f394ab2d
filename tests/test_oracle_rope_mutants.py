"""The rotary oracle's pins catch plausible mistakes.

Copies of oracle.rope with one planted mistake (interleaved instead of
half-split pairs, the rotation's sign, the frequency exponent, the position
off by one, cosine and sine swapped) and of oracle.tree_positions (the node
index instead of its depth, the depth off by one) must each fail one of the
pins of tests/test_oracle_rope.py, run here as plain checks; the oracle passes
them all.
"""
import math

import numpy as np
import pytest

import oracle


def rope_pins_hold(rope) -> bool:
    rng = np.random.default_rng(1)
    x = rng.normal(size=(3, 64))
    if not np.allclose(rope(x, np.zeros(3), 10000.0), x, rtol=0, atol=1e-12):
        return False
    a, b = 37.0, 1205.0
    if not np.allclose(rope(rope(x, np.full(3, b), 10000.0), np.full(3, a), 10000.0),
                       rope(x, np.full(3, a + b), 10000.0), rtol=0, atol=1e-9):
        return False
    got = rope(np.array([1.0, 0.0, 0.0, 0.0]), np.array(3.0), 100.0)
    if not np.allclose(got, [math.cos(3.0), 0.0, math.sin(3.0), 0.0], atol=1e-15):
        return False
    got = rope(np.array([0.0, 0.0, 0.0, 1.0]), np.array(3.0), 100.0)
    if not np.allclose(got, [0.0, -math.sin(0.3), 0.0, math.cos(0.3)], atol=1e-15):
        return False
    q, k = np.random.default_rng(2).normal(size=(2, 128))
    for m, n, s in [(5, 2, 77), (100, 4096, 12345)]:
        lhs = rope(q, np.array(m), 10000.0) @ rope(k, np.array(n), 10000.0)
        rhs = rope(q, np.array(m + s), 10000.0) @ rope(k, np.array(n + s), 10000.0)
        if abs(lhs - rhs) > 1e-9 * (1 + abs(lhs)):
            return False
    return True


def positions_pin_holds(tree_positions) -> bool:
    return (tree_positions([[-1, 0, 1, 2, 3]], [2048]).tolist() == [[2048, 2049, 2050, 2051, 2052]] and
            tree_positions([[-1, 0, 0, 1, 1, 2, 3, 4]], [128]).tolist() == [[128, 129, 129, 130, 130, 130, 131, 131]])


def _rope_mutant(*, interleaved=False, sign=1.0, exponent=2.0, shift=0.0, swap=False):
    def rope(x, pos, theta):
        x = np.asarray(x, dtype=np.float64)
        D = x.shape[-1]
        h = D // 2
        j = np.arange(h, dtype=np.float64)
        ang = (np.asarray(pos, dtype=np.float64)[..., None] + shift) * float(theta) ** (-exponent * j / D)
        c, s = np.cos(ang), np.sin(ang)
        if swap:
            c, s = s, c
        if interleaved:
            lo, hi = x[..., 0::2], x[..., 1::2]
            out = np.empty_like(x)
            out[..., 0::2] = lo * c - sign * hi * s
            out[..., 1::2] = hi * c + sign * lo * s
            return out
        lo, hi = x[..., :h], x[..., h:]
        return np.concatenate([lo * c - sign * hi * s, hi * c + sign * lo * s], axis=-1)
    return rope


def _positions_mutant(*, by_index=False, depth_shift=0):
    def tree_positions(parent, prefix_lens):
        parent = np.asarray(parent)
        out = np.zeros(parent.shape, dtype=np.int64)
        for b in range(parent.shape[0]):
            depth = [0] * parent.shape[1]
            for i in range(1, parent.shape[1]):
                depth[i] = depth[parent[b, i]] + 1 + depth_shift
            out[b] = int(prefix_lens[b]) + (np.arange(parent.shape[1]) if by_index else np.asarray(depth))
        return out
    return tree_positions


def test_the_oracle_and_faithful_rewrites_pass():
    assert rope_pins_hold(oracle.rope) and rope_pins_hold(_rope_mutant())
    assert positions_pin_holds(oracle.tree_positions) and positions_pin_holds(_positions_mutant())


@pytest.mark.parametrize("mistake", [dict(interleaved=True), dict(sign=-1.0), dict(exponent=1.0), dict(shift=1.0),
                                     dict(swap=True)],
                         ids=["interleaved_pairs", "sign_flipped", "frequency_exponent", "position_plus_one",
                              "cos_sin_swapped"])
def test_each_planted_rotation_mistake_fails_a_pin(mistake):
    assert not rope_pins_hold(_rope_mutant(**mistake))


@pytest.mark.parametrize("mistake", [dict(by_index=True), dict(depth_shift=1)], ids=["node_index", "depth_plus_one"])
def test_each_planted_position_mistake_fails_a_pin(mistake):
    assert not positions_pin_holds(_positions_mutant(**mistake))
