"""Pins of the rotary-position oracle (oracle/rope.py) against what the
definition and the tree fix, not against a retyped formula:

* position 0 is the identity, and the rotation at position p composes:
  R(a) R(b) = R(a + b);
* a hand-computed case fixes the half-split pairing and the frequencies
  (D = 4: pair (x0, x2) at angle p, pair (x1, x3) at angle p / sqrt(theta));
* every pair keeps its length, and the score <R(m) q, R(n) k> depends only on
  m - n (the relative-position property that defines rotary embeddings);
* tree positions: a chain is at Lb + i, the 8-node tree at Lb + depth;
* the write puts node i's rotated key and its value at logical slot Lb + i
  through the block table and leaves every other slot as it was.
"""
import math

import numpy as np
import pytest

import oracle


def test_position_zero_is_identity_and_rotations_compose():
    rng = np.random.default_rng(1)
    x = rng.normal(size=(3, 64))
    assert np.array_equal(oracle.rope(x, np.zeros(3), 10000.0), x)
    a, b = 37.0, 1205.0
    ab = oracle.rope(oracle.rope(x, np.full(3, b), 10000.0), np.full(3, a), 10000.0)
    np.testing.assert_allclose(ab, oracle.rope(x, np.full(3, a + b), 10000.0), rtol=0, atol=1e-9)


def test_hand_computed_pairing_and_frequencies():
    theta = 100.0  # D = 4: frequencies 1 and theta^(-1/2) = 0.1
    p = 3.0
    x = np.array([1.0, 0.0, 0.0, 0.0])  # only x0: pair (x0, x2)
    got = oracle.rope(x, np.array(p), theta)
    np.testing.assert_allclose(got, [math.cos(3.0), 0.0, math.sin(3.0), 0.0], atol=1e-15)
    y = np.array([0.0, 0.0, 0.0, 1.0])  # only x3: pair (x1, x3) at angle 0.3
    got = oracle.rope(y, np.array(p), theta)
    np.testing.assert_allclose(got, [0.0, -math.sin(0.3), 0.0, math.cos(0.3)], atol=1e-15)


def test_pair_lengths_and_relative_positions():
    rng = np.random.default_rng(2)
    D = 128
    q, k = rng.normal(size=D), rng.normal(size=D)
    for m, n in [(0, 0), (5, 2), (100, 4096), (8191, 3)]:
        rq = oracle.rope(q, np.array(m), 10000.0)
        np.testing.assert_allclose(rq[:64] ** 2 + rq[64:] ** 2, q[:64] ** 2 + q[64:] ** 2, rtol=1e-12)
        for s in (1, 77, 12345):
            a = oracle.rope(q, np.array(m), 10000.0) @ oracle.rope(k, np.array(n), 10000.0)
            b = oracle.rope(q, np.array(m + s), 10000.0) @ oracle.rope(k, np.array(n + s), 10000.0)
            assert abs(a - b) < 1e-9 * (1 + abs(a))
    # and the score does move with m - n
    s0 = oracle.rope(q, np.array(10), 10000.0) @ oracle.rope(k, np.array(0), 10000.0)
    s1 = oracle.rope(q, np.array(11), 10000.0) @ oracle.rope(k, np.array(0), 10000.0)
    assert abs(s0 - s1) > 1e-6


def test_theta_zero_leaves_rows_unrotated():
    x = np.arange(8.0)
    assert np.array_equal(oracle.rope(x, np.array(1000), 0.0), x)


def test_tree_positions():
    assert oracle.tree_positions([[-1, 0, 1, 2, 3]], [2048]).tolist() == [[2048, 2049, 2050, 2051, 2052]]
    assert oracle.tree_positions([[-1, 0, 0, 1, 1, 2, 3, 4]], [128]).tolist() == [[128, 129, 129, 130, 130, 130,
                                                                                   131, 131]]
    with pytest.raises(ValueError):
        oracle.tree_positions([[-1, 2, 0]], [0])


def test_write_lands_at_slot_prefix_plus_node_and_nowhere_else():
    rng = np.random.default_rng(3)
    B, T, Hq, Hkv, D, bs = 2, 5, 4, 2, 8, 4
    lens = [3, 9]
    parent = np.array([[-1, 0, 0, 1, 2], [-1, 0, 1, 1, 3]])
    nblk = 8
    table = np.array([[5, 1, 7, 0], [2, 6, 4, 3]])  # shuffled pages
    kc = rng.normal(size=(nblk, Hkv, bs, D)).astype(np.float32)
    vc = rng.normal(size=(nblk, Hkv, bs, D)).astype(np.float32)
    kn = rng.normal(size=(B, T, Hkv, D)).astype(np.float32)
    vn = rng.normal(size=(B, T, Hkv, D)).astype(np.float32)
    q = rng.normal(size=(B, T, Hq, D)).astype(np.float32)
    qr, kc2, vc2 = oracle.tree_kv_write(kn, vn, q, kc, vc, table, lens, parent, 500.0, block_size=bs)
    pos = oracle.tree_positions(parent, lens)
    written = set()
    for b in range(B):
        for i in range(T):
            t = lens[b] + i
            blk, off = table[b][t // bs], t % bs
            written.add((blk, off))
            np.testing.assert_array_equal(vc2[blk, :, off], vn[b, i].astype(np.float64))
            for g in range(Hkv):  # each head rotated on its own, at the node's tree position
                np.testing.assert_allclose(kc2[blk, g, off], oracle.rope(kn[b, i, g], np.array(pos[b, i]), 500.0),
                                           rtol=0, atol=0)
            for h in range(Hq):
                np.testing.assert_allclose(qr[b, i, h], oracle.rope(q[b, i, h], np.array(pos[b, i]), 500.0),
                                           rtol=0, atol=0)
    for blk in range(nblk):
        for off in range(bs):
            if (blk, off) not in written:
                assert np.array_equal(kc2[blk, :, off], kc[blk, :, off]) and np.array_equal(vc2[blk, :, off],
                                                                                            vc[blk, :, off])
