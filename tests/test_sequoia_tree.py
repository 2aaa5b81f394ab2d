"""The library's Sequoia tree builder (spec_sequoia_tree, host code behind the
C ABI) against the oracle's dynamic program: the same tree (parent array) and
the same expected token count, bit for bit, for monotone and non-monotone
acceptance vectors, sizes up to 48 and every depth bound; at the
Sequoia-scale size (256 nodes, depth 10) the value is checked against the
greedy optimum of a non-increasing vector; bad arguments are refused.  No GPU
is used."""
import math

import numpy as np
import pytest

import tree_verify_attention_masked_amd as stv
from oracle.sequoia import expected_tokens, sequoia_tree
from test_oracle_sequoia import greedy_top_n
from workloads import make_config


def _vectors(seed):
    rng = np.random.default_rng(seed)
    out = [list(np.sort(rng.uniform(0, 0.95, size=int(rng.integers(1, 9))))[::-1]) for _ in range(3)]
    out += [list(rng.uniform(0, 1, size=int(rng.integers(1, 9)))) for _ in range(3)]
    out += [[0.7], [], [1.0, 1.0], [0.0, 0.5, 0.0, 0.25]]
    return out


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_library_tree_equals_oracle(seed):
    rng = np.random.default_rng(100 + seed)
    for accept in _vectors(seed):
        for n in sorted({1, 2, 3, 5, 8, 13, int(rng.integers(14, 49))}):
            for d in sorted({1, 2, 3, int(rng.integers(1, 12)), n - 1}):
                if n > 1 and d < 1:
                    continue
                want_v, want_p = sequoia_tree(accept, n, d)
                got_p, got_v = stv.spec_sequoia_tree(accept, n, d)
                assert got_p.tolist() == want_p, (accept, n, d)
                assert got_v == want_v, (accept, n, d, got_v, want_v)


def test_sequoia_scale_tree_is_optimal():
    # the Sequoia-scale shape: 256 nodes, depth <= 10, rank profile a_r = 0.8 / r (non-increasing)
    accept = [0.8 / r for r in range(1, 65)]
    parent, value = stv.spec_sequoia_tree(accept, 256, 10)
    assert math.isclose(value, greedy_top_n(accept, 256, 10), rel_tol=1e-12)
    assert math.isclose(expected_tokens(parent.tolist(), accept), value, rel_tol=1e-12)
    d = [0] * 256
    for i in range(1, 256):
        assert 0 <= parent[i] < i
        d[i] = d[parent[i]] + 1
    assert max(d) <= 10


def test_library_refuses_bad_arguments():
    for accept, n, d in (([0.5], 0, 3), ([1.5], 4, 2), ([float("nan")], 4, 2), ([0.5], 4, 0), ([0.5], 5000, 4),
                         ([0.5] * 4095, 4096, 4095)):
        with pytest.raises(stv.SpecError):
            stv.spec_sequoia_tree(accept, n, d)
    assert stv.spec_sequoia_tree([0.5], 1, 0)[0].tolist() == [-1]


@pytest.mark.parametrize("T", [16, 256, 512])
def test_sequoia_scale_trees_are_optimal_for_their_acceptance_vector(T):
    """The Sequoia-scale workload keeps the T best nodes by path score under a
    non-increasing acceptance-by-rank vector; the library's dynamic program must
    find no better tree of that size and depth (the two agree to rounding)."""
    w = make_config(3, T=T, prefix=64, max_depth=10, with_kv=False)
    a = w.info["accept_profile"]
    _, best = stv.spec_sequoia_tree(a, T, 10)
    assert math.isclose(expected_tokens(list(w.parent[0]), a), best, rel_tol=1e-12)
