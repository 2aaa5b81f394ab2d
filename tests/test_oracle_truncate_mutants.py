"""The truncation oracle's pins catch plausible mistakes.

Each mutant below is a copy of oracle.truncate_row with one planted mistake
(an off-by-one k, ties split, the temperature ignored, top-p not renormalised
on the top-k set, the two rules swapped, the nucleus one token short, the k
smallest kept).  The pins of tests/test_oracle_truncate.py, run here as plain
checks, must pass for the oracle and fail for every mutant.
"""
import itertools

import numpy as np
import pytest

from oracle import softmax64, truncate_row

PROBS = np.array([0.5, 0.3, 0.15, 0.05])
ROW = np.log(PROBS).astype(np.float32)
HAND = [(1.0, 0, 0.75, [0, 1]), (1.0, 0, 0.85, [0, 1, 2]), (1.0, 0, 0.97, [0, 1, 2, 3]), (1.0, 0, 0.4, [0]),
        (1.0, 2, 1.0, [0, 1]), (1.0, 3, 0.82, [0, 1]), (1.0, 0, 0.82, [0, 1, 2]), (1.0, 0, 0.7, [0, 1]),
        (2.0, 0, 0.7, [0, 1, 2]), (0.0, 0, 0.3, [0]), (0.0, 2, 1.0, [0, 1])]
TIES = [(np.array([3, 3, 3, 1, 0], np.float32), 1.0, 2, 1.0, [0, 1, 2]),
        (np.array([2, 2, 0, 0], np.float32), 1.0, 0, 0.3, [0, 1]),
        (np.array([-np.inf, 5, 4, 3], np.float32), 1.0, 2, 1.0, [1, 2])]


def _kept(fn, row, tau, k, p):
    out = fn(row, tau, k, p)[0]
    return np.flatnonzero(np.isfinite(out)).tolist()


def pins_hold(fn) -> bool:
    for tau, k, p, want in HAND:
        if _kept(fn, ROW, tau, k, p) != want:
            return False
    for row, tau, k, p, want in TIES:
        if _kept(fn, row, tau, k, p) != want:
            return False
    for seed in range(12):  # brute-force nucleus
        rng = np.random.default_rng(seed)
        V = int(rng.integers(3, 9))
        row = (1.5 * rng.standard_normal(V)).astype(np.float32)
        tau = float(rng.choice([0.5, 1.0, 1.7]))
        top_p = float(np.float32(rng.uniform(0.05, 0.99)))
        p = softmax64(row, tau)
        size = next(n for n in range(1, V + 1)
                    if max(p[list(s)].sum() for s in itertools.combinations(range(V), n)) >= top_p)
        if len(_kept(fn, row, tau, 0, top_p)) != size:
            return False
    for seed in range(6):  # top-k against argsort
        row = np.random.default_rng(100 + seed).standard_normal(50).astype(np.float32)
        for k in (1, 2, 7, 49):
            if _kept(fn, row, 1.0, k, 1.0) != sorted(np.argsort(-row.astype(np.float64))[:k].tolist()):
                return False
    return True


def _mutant(*, k_shift=0, split_ties=False, ignore_tau=False, no_renorm=False, swap=False, short=False,
            smallest=False):
    """truncate_row with one planted mistake (written out again, plainly)."""
    def top_k(vals, keep, k):
        n = int(keep.sum())
        k = k + k_shift
        if k <= 0 or k >= n:
            return keep.copy()
        order = np.argsort(vals if smallest else -vals, kind="stable")
        order = [i for i in order if keep[i]]
        if split_ties:
            out = np.zeros_like(keep)
            out[order[:k]] = True
            return out
        t = vals[order[k - 1]]
        return keep & ((vals <= t) if smallest else (vals >= t))

    def top_p(vals, keep, tau, p):
        if p >= 1.0 or not keep.any():
            return keep.copy()
        tau = 1.0 if ignore_tau else tau
        if tau == 0.0:
            return keep & (vals == vals[keep].max())
        prob = np.zeros(vals.size)
        if no_renorm:
            prob = softmax64(vals, tau) * keep
        else:
            prob[keep] = softmax64(vals[keep], tau)
        distinct = np.unique(vals[keep])[::-1]
        at = np.cumsum([prob[keep & (vals == v)].sum() for v in distinct])
        j = int(np.flatnonzero(at >= p)[0]) if (at >= p).any() else distinct.size - 1
        if short and j > 0:
            j -= 1
        return keep & (vals >= distinct[j])

    def fn(row, tau, k, p):
        row = np.asarray(row, np.float32)
        vals = row.astype(np.float64)
        keep = np.isfinite(vals)
        tau, p = float(np.float32(tau)), float(np.float32(p))
        if swap:
            keep = top_k(vals, top_p(vals, keep, tau, p), int(k))
        else:
            keep = top_p(vals, top_k(vals, keep, int(k)), tau, p)
        out = row.copy()
        out[~keep] = -np.inf
        return out, 0.0
    return fn


def test_the_oracle_and_a_faithful_rewrite_pass():
    assert pins_hold(truncate_row)
    assert pins_hold(_mutant())


@pytest.mark.parametrize("mistake", [dict(k_shift=1), dict(k_shift=-1), dict(split_ties=True), dict(ignore_tau=True),
                                     dict(no_renorm=True), dict(swap=True), dict(short=True), dict(smallest=True)],
                         ids=["k_plus_one", "k_minus_one", "ties_split", "temperature_ignored", "not_renormalised",
                              "rules_swapped", "nucleus_one_short", "smallest_kept"])
def test_each_planted_mistake_fails_a_pin(mistake):
    assert not pins_hold(_mutant(**mistake))
