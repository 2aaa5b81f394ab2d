"""Pins for the oracle's Sequoia tree construction (oracle/sequoia.py).

* the objective F(T) on a hand-worked tree;
* brute force: every ordered tree of up to 8 nodes under a depth bound is
  enumerated and scored, for monotone and non-monotone acceptance vectors; the
  dynamic program's value is the best score, and its tree has that score, the
  asked size and a depth within the bound;
* closed forms: depth 1 gives the star 1 + p_1 + ... + p_(n-1); a single
  acceptance entry gives the chain 1 + p + ... + p^d;
* for a non-increasing vector the optimum is the n nodes of highest path
  score (greedy, a different algorithm);
* planted mistakes (p indexed by depth instead of rank, the depth bound
  ignored, ranks shifted by one, the root's token not counted) each fail a pin.
"""
import itertools
import math

import numpy as np
import pytest

from oracle.sequoia import expected_tokens, sequoia_tree


def ordered_trees(n):
    """Every ordered tree of n nodes, as nested tuples of children."""
    if n == 1:
        return [()]
    return [kids for kids in ordered_forests(n - 1)]


def ordered_forests(m):
    if m == 0:
        return [()]
    out = []
    for a in range(1, m + 1):
        for t in ordered_trees(a):
            for rest in ordered_forests(m - a):
                out.append((t,) + rest)
    return out


def tree_depth(t):
    return 0 if not t else 1 + max(tree_depth(c) for c in t)


def score(t, accept):
    """F of a nested-tuple tree: 1 for the node plus p_rank * F(child) over its children."""
    return 1.0 + sum((accept[k] if k < len(accept) else 0.0) * score(c, accept) for k, c in enumerate(t))


def depth_of(parent):
    d = [0] * len(parent)
    for i in range(1, len(parent)):
        d[i] = d[parent[i]] + 1
    return max(d)


def greedy_top_n(accept, n, max_depth):
    """Sum of the n largest path scores among nodes of depth <= max_depth (best first from the root)."""
    import heapq
    K = len(accept)
    heap = [(-1.0, 0, 0)]  # (-score, depth, next child rank to open)
    total, taken = 0.0, 0
    while heap and taken < n:
        s, d, _ = heapq.heappop(heap)
        total += -s
        taken += 1
        if d < max_depth:
            for k in range(K):  # every child: the heap keeps them in score order
                heapq.heappush(heap, (s * accept[k], d + 1, 0))
    return total if taken == n else None


# ----------------------------------------------------------------------------

def test_objective_hand_worked():
    # root; 1 and 2 its first and second children; 3 the first child of 1
    assert math.isclose(expected_tokens([-1, 0, 0, 1], [0.5, 0.3]), 1 + 0.5 + 0.3 + 0.5 * 0.5)
    # ranks beyond the vector add nothing
    assert math.isclose(expected_tokens([-1, 0, 0, 0], [0.5, 0.3]), 1.8)
    assert expected_tokens([-1], [0.9]) == 1.0


def _vectors():
    rng = np.random.default_rng(0)
    vs = [[0.8, 0.5, 0.3], [0.3, 0.8, 0.1], [0.9], [0.5, 0.5, 0.5, 0.5], [0.0, 0.7], [1.0, 0.0, 1.0]]
    for _ in range(6):
        vs.append(list(rng.uniform(0, 1, size=int(rng.integers(1, 5)))))
    return vs


def dp_pins(build, objective) -> bool:
    for accept in _vectors():
        for n in range(1, 9):
            trees = ordered_trees(n)
            for d in range(0 if n == 1 else 1, 8):
                best = max(score(t, accept) for t in trees if tree_depth(t) <= d)
                value, parent = build(accept, n, d)
                if not math.isclose(value, best, rel_tol=1e-12, abs_tol=1e-12):
                    return False
                if len(parent) != n or depth_of(parent) > d or any(not 0 <= parent[i] < i for i in range(1, n)):
                    return False
                if not math.isclose(objective(parent, accept), best, rel_tol=1e-12):
                    return False
    return True


def closed_form_pins(build) -> bool:
    for accept in ([0.9, 0.6, 0.5, 0.2, 0.1], [0.2, 0.7, 0.4]):
        for n in range(2, 7):
            if not math.isclose(build(accept, n, 1)[0], 1 + sum(accept[: n - 1]), rel_tol=1e-12):
                return False
    for p in (0.3, 0.9):
        for n, d in ((6, 5), (6, 2), (10, 3), (4, 9)):
            want = sum(p ** j for j in range(min(d, n - 1) + 1))
            if not math.isclose(build([p], n, d)[0], want, rel_tol=1e-12):
                return False
    return True


def test_dp_against_brute_force_over_every_small_tree():
    assert dp_pins(sequoia_tree, expected_tokens)


def test_dp_closed_forms():
    assert closed_form_pins(sequoia_tree)


@pytest.mark.parametrize("n,d", [(16, 5), (40, 6), (64, 10)])
def test_dp_equals_greedy_for_non_increasing_vectors(n, d):
    rng = np.random.default_rng(n)
    accept = sorted(rng.uniform(0, 0.9, size=8), reverse=True)
    value, parent = sequoia_tree(accept, n, d)
    assert math.isclose(value, greedy_top_n(accept, n, d), rel_tol=1e-12)
    assert math.isclose(expected_tokens(parent, accept), value, rel_tol=1e-12)


def test_dp_rejects_infeasible_and_invalid_inputs():
    with pytest.raises(ValueError):
        sequoia_tree([0.5], 3, 0)
    with pytest.raises(ValueError):
        sequoia_tree([1.5], 3, 2)
    with pytest.raises(ValueError):
        sequoia_tree([0.5], 0, 2)
    assert sequoia_tree([0.5], 1, 0) == (1.0, [-1])


# ----------------------------------------------------------------------------
# planted mistakes
# ----------------------------------------------------------------------------

def _objective_by_depth(parent, accept):  # p indexed by the node's depth instead of its rank
    d = [0] * len(parent)
    f = [1.0] * len(parent)
    for i in range(1, len(parent)):
        d[i] = d[parent[i]] + 1
        f[i] = f[parent[i]] * (accept[d[i] - 1] if d[i] <= len(accept) else 0.0)
    return sum(f)


def _dp_without_root(accept, n, d):  # the target's own token not counted
    v, parent = sequoia_tree(accept, n, d)
    return v - 1.0, parent


def _dp_ignoring_depth(accept, n, d):
    return sequoia_tree(accept, n, n - 1)


def _dp_ranks_shifted(accept, n, d):  # the first child weighted by p_2
    return sequoia_tree(list(accept[1:]) + [0.0], n, d)


@pytest.mark.parametrize("name,ok", [
    ("objective by depth", lambda: dp_pins(sequoia_tree, _objective_by_depth)),
    ("root not counted", lambda: closed_form_pins(_dp_without_root)),
    ("depth bound ignored", lambda: dp_pins(_dp_ignoring_depth, expected_tokens)),
    ("ranks shifted by one", lambda: closed_form_pins(_dp_ranks_shifted)),
])
def test_planted_mistake_fails_a_pin(name, ok):
    assert not ok(), f"the pins do not catch: {name}"
