"""Pins for the oracle's top-k / top-p truncation.

* a hand-worked row (probabilities 0.5, 0.3, 0.15, 0.05): kept sets for top-k,
  top-p, both (top-k first, then top-p renormalised on the top-k set), a
  temperature that changes the nucleus, and temperature 0;
* brute force on tiny rows: the nucleus has the size of the smallest subset of
  tokens whose mass reaches top_p, and is the most probable subset of that size;
* top-k against NumPy's argsort for distinct logits, ties kept whole, -inf not
  counted, the switches that turn a rule off;
* exact enumeration: speculative rejection over a small tree, with the target
  rows truncated, emits tokens that follow the truncated target exactly;
* top_k = 1 at a positive temperature gives greedy verification's result.
"""
import itertools
import math

import numpy as np
import pytest

from oracle import PhiloxDraws, reject_sequence, softmax64, tree_reject, truncate_logits, truncate_row
from test_oracle_reject import (_draft_assignments, _max_deviation_from_target, _model, _token_paths,
                                _walk_outcomes)

PROBS = np.array([0.5, 0.3, 0.15, 0.05])
ROW = np.log(PROBS).astype(np.float32)


def kept(row, tau, k, p):
    out, _ = truncate_row(row, tau, k, p)
    return np.flatnonzero(np.isfinite(out)).tolist()


@pytest.mark.parametrize("tau,k,p,want", [
    (1.0, 0, 0.75, [0, 1]),           # 0.5 < 0.75 <= 0.8
    (1.0, 0, 0.85, [0, 1, 2]),        # 0.8 < 0.85 <= 0.95
    (1.0, 0, 0.97, [0, 1, 2, 3]),
    (1.0, 0, 0.4, [0]),
    (1.0, 2, 1.0, [0, 1]),
    (1.0, 3, 0.82, [0, 1]),           # on the top-3 set: 0.5/0.95 = 0.526, 0.8/0.95 = 0.842 >= 0.82
    (1.0, 0, 0.82, [0, 1, 2]),        # without top-k: 0.8 < 0.82
    (1.0, 0, 0.7, [0, 1]),
    (2.0, 0, 0.7, [0, 1, 2]),         # tau 2: p ~ sqrt(PROBS) = .379 .293 .207 .120; .672 < .7
    (0.0, 0, 0.3, [0]),               # temperature 0: the maximum only
    (0.0, 2, 1.0, [0, 1]),
])
def test_hand_worked_row(tau, k, p, want):
    assert kept(ROW, tau, k, p) == want


def test_margin_is_distance_to_the_two_cumulative_masses():
    _, m = truncate_row(ROW, 1.0, 0, 0.75)
    assert abs(m - 0.05) < 1e-6          # min(0.75 - 0.5, 0.8 - 0.75)
    _, m = truncate_row(ROW, 1.0, 0, 0.52)
    assert abs(m - 0.02) < 1e-6
    assert truncate_row(ROW, 1.0, 3, 1.0)[1] == math.inf


@pytest.mark.parametrize("seed", range(12))
def test_nucleus_is_the_smallest_subset_reaching_top_p(seed):
    rng = np.random.default_rng(seed)
    V = int(rng.integers(3, 9))
    row = (1.5 * rng.standard_normal(V)).astype(np.float32)
    tau = float(rng.choice([0.5, 1.0, 1.7]))
    top_p = float(np.float32(rng.uniform(0.05, 0.99)))
    p = softmax64(row, tau)
    best_size, best_mass = None, -1.0
    for size in range(1, V + 1):
        masses = [p[list(s)].sum() for s in itertools.combinations(range(V), size)]
        if max(masses) >= top_p:
            best_size, best_mass = size, max(masses)
            break
    ks = kept(row, tau, 0, top_p)
    assert len(ks) == best_size
    assert abs(p[ks].sum() - best_mass) < 1e-12


@pytest.mark.parametrize("seed", range(6))
def test_top_k_is_the_k_largest(seed):
    rng = np.random.default_rng(100 + seed)
    V = 50
    row = rng.standard_normal(V).astype(np.float32)
    for k in (1, 2, 7, 49):
        assert kept(row, 1.0, k, 1.0) == sorted(np.argsort(-row.astype(np.float64))[:k].tolist())


def test_ties_kept_whole_and_minus_inf_not_counted():
    assert kept(np.array([3, 3, 3, 1, 0], np.float32), 1.0, 2, 1.0) == [0, 1, 2]
    assert kept(np.array([2, 2, 0, 0], np.float32), 1.0, 0, 0.3) == [0, 1]
    assert kept(np.array([-np.inf, 5, 4, 3], np.float32), 1.0, 2, 1.0) == [1, 2]
    assert kept(np.array([-np.inf, 5, 4, 3], np.float32), 1.0, 3, 1.0) == [1, 2, 3]
    assert kept(np.full(6, 0.25, np.float32), 1.0, 0, 0.5) == list(range(6))
    assert kept(np.full(4, -np.inf, np.float32), 1.0, 2, 0.5) == []
    assert kept(np.full(4, -np.inf, np.float32), 0.0, 2, 0.5) == []


def test_switches_off_leave_the_row_alone():
    rng = np.random.default_rng(7)
    row = rng.standard_normal(20).astype(np.float32)
    for k, p in ((0, 1.0), (20, 1.0), (25, 1.0), (-3, 1.0)):
        out, _ = truncate_row(row, 0.8, k, p)
        assert np.array_equal(out, row)
    with pytest.raises(ValueError):
        truncate_row(np.array([1.0, np.nan], np.float32), 1.0, 1, 1.0)


def test_truncate_logits_rows_independent():
    rng = np.random.default_rng(9)
    lg = rng.standard_normal((2, 3, 40)).astype(np.float32)
    out, margins = truncate_logits(lg, 1.0, 10, 0.8)
    assert margins.shape == (2, 3)
    for b in range(2):
        for u in range(3):
            assert np.array_equal(out[b, u], truncate_row(lg[b, u], 1.0, 10, 0.8)[0])
            assert np.isfinite(out[b, u]).sum() <= 10


@pytest.mark.parametrize("parent,V,k,p", [([-1, 0, 0, 0], 4, 3, 1.0), ([-1, 0, 0, 0], 4, 0, 0.7),
                                          ([-1, 0, 1], 4, 2, 0.9), ([-1, 0, 0, 1], 3, 0, 0.6)])
@pytest.mark.parametrize("wo", [False, True])
def test_enumeration_follows_truncated_target(parent, V, k, p, wo):
    tau = 1.0
    depth = max(len(_token_paths(parent, np.zeros(len(parent), np.int32))[i]) for i in range(len(parent)))
    logits, draft = _model(V, depth, seed=5 * V + k, tau=tau)
    trunc = {h: truncate_row(row, tau, k, p)[0] for h, row in logits.items()}
    dist = {}
    mode = "without_replacement" if wo else "iid"
    for tokens, pr in _draft_assignments(parent, lambda h: draft[h].astype(np.float64), mode, V):
        tp = _token_paths(parent, tokens)
        lg = np.stack([trunc[h] for h in tp])
        qq = np.stack([draft[h] for h in tp])

        def run(src, lg=lg, qq=qq, tokens=tokens):
            return reject_sequence(lg, qq, tokens, parent, tau, wo, src)

        for (path, emitted), w in _walk_outcomes(run):
            seq = tuple(int(tokens[n]) for n in path[1:]) + (int(emitted),)
            dist[seq] = dist.get(seq, 0.0) + pr * w
    assert abs(sum(dist.values()) - 1.0) < 1e-12
    assert _max_deviation_from_target(dist, trunc, tau, V) < 1e-12
    # and not the untruncated target
    assert _max_deviation_from_target(dist, logits, tau, V) > 1e-3
    # no emitted token is ever outside its history's kept set
    for seq in dist:
        for i in range(len(seq)):
            assert np.isfinite(trunc[seq[:i]][seq[i]]) or dist[seq] == 0.0


@pytest.mark.parametrize("wo", [False, True])
def test_top_k_one_gives_greedy(wo):
    rng = np.random.default_rng(21)
    B, T, V = 6, 12, 30
    parent = np.array([[-1] + [int(rng.integers(0, i)) for i in range(1, T)] for _ in range(B)], np.int32)
    logits = rng.standard_normal((B, T, V)).astype(np.float32)
    am = logits.argmax(-1)
    tokens = np.zeros((B, T), np.int32)
    for b in range(B):
        for i in range(1, T):
            tokens[b, i] = am[b, parent[b, i]] if rng.random() < 0.6 else rng.integers(V)
    q = rng.dirichlet(np.ones(V), size=(B, T)).astype(np.float32)
    greedy = tree_reject(logits, q, tokens, parent, 0.0, wo, 3, 0)
    trunc, _ = truncate_logits(logits, 1.0, 1, 1.0)
    sampled = tree_reject(trunc, q, tokens, parent, 1.0, wo, 3, 0)
    assert np.array_equal(greedy["accepted_nodes"], sampled["accepted_nodes"])
    assert np.array_equal(greedy["out_tokens"], sampled["out_tokens"])
    assert greedy["num_accepted"].sum() > 0
