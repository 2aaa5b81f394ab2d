"""Sequoia tree construction by dynamic programming (oracle side) -- TEST
INFRASTRUCTURE ONLY, like the rest of this package.

The Sequoia summary ("Sequoia: Scalable and Robust Speculative Decoding",
"Scalable Speculative Decoding" and "Dynamic Programming") says that the tree
of speculated tokens is built by dynamic programming to balance exploration
(width) against exploitation (depth), and (its "More on figures") that the
tree size is then chosen against the target's forward time at each input
length.  It gives neither the objective nor the recurrence; both are taken
from the published Sequoia paper (Chen et al. 2024), outside the pages:

* positional acceptance: the k-th child (in the order the verifier tries
  siblings) of an accepted node is the one accepted with probability p_k,
  whatever the node or its depth;
* so node v is accepted with probability f(v) = product of p_rank over the
  edges from the root to v (the root: 1), and a verification step generates
  F(T) = sum over v of f(v) tokens in expectation (the accepted drafts plus
  the one token the target always adds);
* c(n, d) = the largest F over trees of exactly n nodes and depth <= d (depth
  in edges): c(1, d) = 1; c(n, 0) is infeasible for n > 1; for d >= 1,
  c(n, d) = 1 + g(n - 1, 1, d - 1), where g(m, k, e) is the best way to hand
  m nodes to children of ranks k, k+1, ..., each child getting a subtree of
  depth <= e: g(0, k, e) = 0 and
      g(m, k, e) = max over a = 1..m of  p_k c(a, e) + g(m - a, k + 1, e).

Readings where the paper leaves a choice: p_k = 0 for ranks beyond the given
vector (a child there adds nothing); among equal values the smallest subtree
for the lower rank wins (a = 1, 2, ... tried in turn, strict improvement); the
tree is returned as a parent array numbered breadth first, siblings in rank
order, so a node's children are tried by the verifier in index order.
"""
from __future__ import annotations

import sys
from collections import deque
from functools import lru_cache


def sibling_ranks(parent):
    """1-based position of every node among its parent's children, in index order (root: 0)."""
    seen = {}
    rank = [0] * len(parent)
    for i in range(1, len(parent)):
        seen[parent[i]] = seen.get(parent[i], 0) + 1
        rank[i] = seen[parent[i]]
    return rank


def expected_tokens(parent, accept):
    """F(T): sum over the nodes of the product of p_rank along the path from the root."""
    rank = sibling_ranks(parent)
    p = lambda k: float(accept[k - 1]) if k <= len(accept) else 0.0
    f = [1.0] * len(parent)
    total = 1.0
    for i in range(1, len(parent)):
        f[i] = f[parent[i]] * p(rank[i])
        total += f[i]
    return total


def sequoia_tree(accept, n, max_depth):
    """(c(n, max_depth), parent array of an optimal tree); ValueError if no tree fits."""
    accept = [float(x) for x in accept]
    K = len(accept)
    if n < 1 or max_depth < 0 or any(not 0.0 <= x <= 1.0 for x in accept):
        raise ValueError("need n >= 1, max_depth >= 0 and every p in [0, 1]")
    if n > 1 and max_depth == 0:
        raise ValueError("a tree of more than one node needs depth >= 1")
    sys.setrecursionlimit(max(10000, 50 * n))
    p = lambda k: accept[k - 1] if k <= K else 0.0
    NONE = None  # infeasible

    @lru_cache(maxsize=None)
    def c(m, d):
        if m == 1:
            return 1.0
        if d == 0:
            return NONE
        rest = g(m - 1, 1, d - 1)
        return NONE if rest is NONE else 1.0 + rest[0]

    @lru_cache(maxsize=None)
    def g(m, k, e):
        """(best value, size of rank k's subtree) for m nodes under ranks k, k+1, ..."""
        if m == 0:
            return (0.0, 0)
        if k > K:  # every later child adds 0: m leaves
            return (0.0, 1)
        best = NONE
        for a in range(1, m + 1):
            sub = c(a, e)
            tail = g(m - a, k + 1, e)
            if sub is NONE or tail is NONE:
                continue
            prod = p(k) * sub
            v = prod + tail[0]
            if best is NONE or v > best[0]:
                best = (v, a)
        return best

    value = c(n, max_depth)
    if value is NONE:
        raise ValueError("no tree of that size fits the depth")

    # rebuild: the children of a node of subtree size m and remaining depth d
    def children_sizes(m, d):
        sizes, left, k = [], m - 1, 1
        while left > 0:
            a = g(left, k, d - 1)[1]
            sizes.append(a)
            left -= a
            k += 1
        return sizes

    parent = [-1]
    queue = deque([(0, n, max_depth)])
    while queue:  # breadth first: children numbered in rank order after everything above them
        u, m, d = queue.popleft()
        for a in (children_sizes(m, d) if m > 1 else []):
            parent.append(u)
            queue.append((len(parent) - 1, a, d - 1))
    return value, parent
