"""Draft-tree structure (oracle side).

The draft tree arrives flattened as a parent array: node 0 is the root (the
last committed token, whose row gives the distribution its children were
drafted from), parent[0] = -1 and 0 <= parent[i] < i for every other node, so
the flattening is topological.  The tree_mask of the EAGLE report ("Report:
Support nextn speculative decoding", the tree_mask / tree_structure example
and step 3 of the implementation summary) is the ancestor-or-self relation
computed here: node i may attend to tree node j iff j is i or an ancestor of i.
"""
from __future__ import annotations

from dataclasses import dataclass


@dataclass
class Tree:
    parent: list
    depth: list
    anc: list  # anc[i]: sorted list of ancestor-or-self node indices of i
    children: list  # children[u]: child node indices of u, increasing

    @property
    def T(self) -> int:
        return len(self.parent)


def tree_structure(parent) -> Tree:
    parent = [int(p) for p in parent]
    T = len(parent)
    if T < 1 or parent[0] != -1:
        raise ValueError("parent[0] must be -1")
    for i in range(1, T):
        if not (0 <= parent[i] < i):
            raise ValueError(f"parent[{i}] = {parent[i]} is not in [0, {i})")
    depth = [0] * T
    anc = [[0]]
    children = [[] for _ in range(T)]
    for i in range(1, T):
        p = parent[i]
        depth[i] = depth[p] + 1
        anc.append(sorted(anc[p] + [i]))
        children[p].append(i)
    return Tree(parent=parent, depth=depth, anc=anc, children=children)
