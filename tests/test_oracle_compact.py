"""Pins for the oracle's selective KV compaction.

* brute force: every possible accepted path of the cfg0 tree (one per end
  node), random paths on random trees, checked slot by slot against a
  from-scratch statement (rows of the path land at prefix + d, nothing else
  changes);
* a chain never moves data;
* attention link: the tree-masked outputs of the accepted nodes before the
  compaction equal chain attention over the compacted cache afterwards.
"""
import numpy as np
import pytest

from oracle import kv_compact, tree_attention, tree_structure
from workloads import make_config, make_workload


def _slot(w, b, t):
    return int(w.block_table[b][t // 16]), t % 16


def _check(w, acc, nacc):
    k2, v2, new_lens = kv_compact(w.k_cache, w.v_cache, w.block_table, w.prefix_lens, acc, nacc)
    expect_k = w.k_cache.copy()
    expect_v = w.v_cache.copy()
    for b in range(w.B):
        L = int(w.prefix_lens[b])
        path = acc[b][:nacc[b] + 1]
        for d, n in enumerate(path):
            sb, ss = _slot(w, b, L + int(n))
            db, ds = _slot(w, b, L + d)
            expect_k[db, :, ds] = w.k_cache[sb, :, ss]
            expect_v[db, :, ds] = w.v_cache[sb, :, ss]
        assert new_lens[b] == L + nacc[b] + 1
    np.testing.assert_array_equal(k2.view(np.uint8), expect_k.view(np.uint8))
    np.testing.assert_array_equal(v2.view(np.uint8), expect_v.view(np.uint8))
    return k2, v2, new_lens


def test_every_path_of_the_tiny_tree():
    w = make_config(0)
    tree = tree_structure(w.parent[0])
    for end in range(w.T):
        path = tree.anc[end]
        acc = np.full((1, w.T), -1, dtype=np.int32)
        acc[0, :len(path)] = path
        _check(w, acc, np.array([len(path) - 1], dtype=np.int32))


def test_in_place_overlap_reads_before_writes():
    # path [0, 2, 5]: d = 1 copies slot L+2 to L+1 while d = 2 overwrites slot L+2
    w = make_config(0)
    acc = np.array([[0, 2, 5, -1, -1, -1, -1, -1]], dtype=np.int32)
    k2, _, _ = _check(w, acc, np.array([2], dtype=np.int32))
    b1, s1 = _slot(w, 0, 128 + 1)
    b2, s2 = _slot(w, 0, 128 + 2)
    o2, os2 = _slot(w, 0, 128 + 2)
    o5, os5 = _slot(w, 0, 128 + 5)
    np.testing.assert_array_equal(k2[b1, :, s1], w.k_cache[o2, :, os2])
    np.testing.assert_array_equal(k2[b2, :, s2], w.k_cache[o5, :, os5])


def test_random_paths_random_trees():
    rng = np.random.default_rng(7)
    w = make_workload(tag=301, B=4, Hq=2, Hkv=2, D=8, dtype="bf16", V=8, prefix=[0, 15, 16, 37],
                      tree="random", T=12, max_depth=6, shuffle_blocks=True)
    acc = np.full((w.B, w.T), -1, dtype=np.int32)
    nacc = np.zeros(w.B, dtype=np.int32)
    for b in range(w.B):
        tree = tree_structure(w.parent[b])
        path = tree.anc[int(rng.integers(w.T))]
        acc[b, :len(path)] = path
        nacc[b] = len(path) - 1
    _check(w, acc, nacc)


def test_chain_is_a_no_op():
    w = make_workload(tag=302, B=2, Hq=2, Hkv=1, D=8, dtype="f32", V=8, prefix=[3, 20],
                      tree="chain", gamma=4)
    acc = np.array([[0, 1, 2, -1, -1], [0, 1, 2, 3, 4]], dtype=np.int32)
    k2, v2, new_lens = kv_compact(w.k_cache, w.v_cache, w.block_table, w.prefix_lens, acc,
                                  np.array([2, 4], dtype=np.int32))
    np.testing.assert_array_equal(k2.view(np.uint8), w.k_cache.view(np.uint8))
    np.testing.assert_array_equal(v2.view(np.uint8), w.v_cache.view(np.uint8))
    assert new_lens.tolist() == [3 + 3, 20 + 5]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_compacted_cache_gives_chain_attention_of_accepted_nodes(dtype):
    rng = np.random.default_rng(8)
    w = make_workload(tag=303, B=3, Hq=4, Hkv=2, D=16, dtype=dtype, V=8, prefix=[5, 16, 30],
                      tree="random", T=10, max_depth=5, shuffle_blocks=True)
    before = tree_attention(w.q, w.k_cache, w.v_cache, w.block_table, w.prefix_lens, w.parent,
                            w.scale, dtype=dtype)
    acc = np.full((w.B, w.T), -1, dtype=np.int32)
    nacc = np.zeros(w.B, dtype=np.int32)
    for b in range(w.B):
        tree = tree_structure(w.parent[b])
        leaves = [i for i in range(w.T) if not tree.children[i]]
        path = tree.anc[leaves[int(rng.integers(len(leaves)))]]
        acc[b, :len(path)] = path
        nacc[b] = len(path) - 1
    k2, v2, _ = kv_compact(w.k_cache, w.v_cache, w.block_table, w.prefix_lens, acc, nacc)
    for b in range(w.B):
        n = int(nacc[b]) + 1
        path = acc[b, :n]
        chain = np.array([[-1] + list(range(n - 1))], dtype=np.int32)
        after = tree_attention(w.q[b:b + 1, path], k2, v2, w.block_table[b:b + 1],
                               w.prefix_lens[b:b + 1], chain, w.scale, dtype=dtype)
        np.testing.assert_allclose(after[0], before[b, path], rtol=1e-13, atol=1e-14)
