"""The synthetic workloads have the shapes, trees and layouts the configurations state."""
import numpy as np
import pytest

from workloads import make_config, make_workload


def _check_tree(parent, T, max_depth):
    assert parent.shape[-1] == T and parent[0] == -1
    depth = [0]
    for i in range(1, T):
        assert 0 <= parent[i] < i
        depth.append(depth[parent[i]] + 1)
    assert max(depth) <= max_depth
    return max(depth)


@pytest.mark.parametrize("cfg", [0, 1, 3])
def test_small_configs(cfg):
    w = make_config(cfg)
    want = {0: (1, 8, 2, 2, 64, 1000, 3), 1: (1, 5, 40, 40, 128, 32000, 4),
            3: (1, 256, 64, 8, 128, 32000, 10)}[cfg]
    assert (w.B, w.T, w.Hq, w.Hkv, w.D, w.V) == want[:6]
    assert _check_tree(w.parent[0], w.T, want[6]) == want[6]
    assert w.target_logits.shape == (w.B, w.T, w.V) == w.draft_probs.shape
    np.testing.assert_allclose(w.draft_probs.astype(np.float64).sum(-1), 1.0, atol=1e-5)
    assert (w.draft_tokens[:, 1:] >= 0).all() and (w.draft_tokens < w.V).all()
    assert w.block_table.shape[1] == -(-(int(w.prefix_lens.max()) + w.T) // 16)


def test_tiny_tree_and_poisoned_tail():
    w = make_config(0)
    assert w.parent[0].tolist() == [-1, 0, 0, 1, 1, 2, 3, 4]
    assert w.k_cache.shape == (9, 2, 16, 64)
    # positions 136..143 of the last page are unused: NaN
    assert np.isnan(w.k_cache[8, :, 8:]).all() and not np.isnan(w.k_cache[8, :, :8]).any()


def test_sequoia_tree_siblings_distinct():
    w = make_config(3)
    par = w.parent[0]
    for u in range(w.T):
        kids = np.nonzero(par == u)[0]
        toks = w.draft_tokens[0][kids]
        assert len(set(toks.tolist())) == len(toks)


def test_determinism_and_seed_sensitivity():
    a = make_workload(tag=9, B=2, Hq=2, Hkv=1, D=8, dtype="bf16", V=12, prefix=(3, 40), tree="random",
                      T=6, max_depth=3, shuffle_blocks=True, seed=4)
    b = make_workload(tag=9, B=2, Hq=2, Hkv=1, D=8, dtype="bf16", V=12, prefix=(3, 40), tree="random",
                      T=6, max_depth=3, shuffle_blocks=True, seed=4)
    c = make_workload(tag=9, B=2, Hq=2, Hkv=1, D=8, dtype="bf16", V=12, prefix=(3, 40), tree="random",
                      T=6, max_depth=3, shuffle_blocks=True, seed=5)
    for name in ("q", "k_cache", "block_table", "prefix_lens", "parent", "draft_tokens", "target_logits"):
        assert np.array_equal(getattr(a, name), getattr(b, name))
    assert not np.array_equal(a.target_logits, c.target_logits)


@pytest.mark.slow
def test_eagle_and_batched_configs():
    w = make_config(2)
    assert (w.B, w.T, w.Hq, w.Hkv, w.V) == (8, 64, 32, 8, 128256)
    for b in range(w.B):
        assert _check_tree(w.parent[b], 64, 6) == 6
    w = make_config(4)
    assert (w.B, w.T, w.Hq, w.Hkv) == (64, 16, 32, 8)
    assert 512 <= w.prefix_lens.min() and w.prefix_lens.max() <= 16384
    for b in range(w.B):
        _check_tree(w.parent[b], 16, 5)
    used = np.concatenate([w.block_table[b, :-(-(int(w.prefix_lens[b]) + 16) // 16)] for b in range(w.B)])
    assert len(np.unique(used)) == len(used)  # no two sequences share a page
    assert not (np.diff(used) == 1).all()  # the table is shuffled
