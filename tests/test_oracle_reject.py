"""Pins for the oracle's tree rejection sampler.

* greedy: the SGLang doc's worked example, its three outcomes and the closed
  form "longest matching prefix + one target token" on chains;
* the accept test equals probability min(1, p/q) exactly over the 24-bit grid
  of uniforms, and the inverse CDF reproduces the weights exactly over a grid;
* exact enumeration on tiny vocabularies: over every draft-token tuple and
  every random branch, the emitted tokens follow the target distribution
  (next token given the emitted history ~ the target row of that history), for
  (with-replacement verifier, i.i.d. drafts) and (without-replacement verifier,
  without-replacement drafts); the two mismatched pairings are shown to fail;
* chi-square and acceptance-rate tests of the real Philox-driven walk;
* residual invariants and the temperature -> 0+ limit (greedy).
"""
import json
import os

import numpy as np
import pytest
from scipy import stats

from oracle import (accept_draw, inverse_cdf, reject_sequence, residual_update, softmax64,
                    tree_reject, without_replacement_update, PhiloxDraws)
from oracle.tree import tree_structure

HERE = os.path.dirname(os.path.abspath(__file__))


# ----------------------------------------------------------------------------
# greedy verification
# ----------------------------------------------------------------------------

def _rows_with_argmax(argmaxes, V, rng, gap=1.0):
    rows = rng.standard_normal((len(argmaxes), V)).astype(np.float32)
    for u, a in enumerate(argmaxes):
        rows[u, a] = rows[u].max() + gap
    return rows


def test_worked_example_prefix_match():
    with open(os.path.join(HERE, "golden", "sglang_worked_example.json")) as f:
        ex = json.load(f)
    vocab = ex["vocab"]
    ix = {w: i for i, w in enumerate(vocab)}
    V = len(vocab)
    T = len(ex["draft"]) + 1
    parent = np.array([[-1] + list(range(T - 1))], dtype=np.int32)
    tokens = np.array([[ix["<ctx>"]] + [ix[w] for w in ex["draft"]]], dtype=np.int32)
    target = [ix[w] for w in ex["target_greedy"]] + [ix["<other>"]]
    logits = _rows_with_argmax(target, V, np.random.default_rng(0))[None]
    q = np.full((1, T, V), 1.0 / V, dtype=np.float32)
    res = tree_reject(logits, q, tokens, parent, 0.0, False, seed=0, offset=0)
    want = ex["expected"]
    L = want["num_accepted"]
    assert res["num_accepted"][0] == L
    assert res["accepted_nodes"][0, :L + 1].tolist() == want["accepted_nodes"]
    assert [vocab[t] for t in res["out_tokens"][0, :L + 1]] == want["emitted"]
    assert (res["out_tokens"][0, L + 1:] == -1).all() and (res["accepted_nodes"][0, L + 1:] == -1).all()


@pytest.mark.parametrize("case", ["full", "none", "prefix"])
def test_greedy_three_outcomes(case):
    rng = np.random.default_rng(1)
    V, gamma = 50, 6
    argmax = rng.integers(0, V, size=gamma + 1)
    logits = _rows_with_argmax(argmax, V, rng)
    drafts = argmax[:gamma].copy()
    if case == "none":
        drafts[0] = (argmax[0] + 1) % V
    elif case == "prefix":
        drafts[3] = (argmax[3] + 1) % V
    tokens = np.concatenate([[0], drafts]).astype(np.int32)
    parent = [-1] + list(range(gamma))
    path, emitted = reject_sequence(logits, np.full((gamma + 1, V), 1 / V), tokens, parent, 0.0,
                                    False, None)
    L = len(path) - 1
    want_L = {"full": gamma, "none": 0, "prefix": 3}[case]
    assert L == want_L
    assert emitted == argmax[L]  # the target always adds exactly one token


def test_greedy_chain_closed_form():
    rng = np.random.default_rng(2)
    V = 6
    for trial in range(200):
        gamma = int(rng.integers(1, 7))
        logits = rng.standard_normal((gamma + 1, V)).astype(np.float32)
        am = logits.argmax(axis=1)
        drafts = np.where(rng.random(gamma) < 0.6, am[:gamma], rng.integers(0, V, gamma))
        tokens = np.concatenate([[0], drafts]).astype(np.int32)
        path, emitted = reject_sequence(logits, np.full((gamma + 1, V), 1 / V), tokens,
                                        [-1] + list(range(gamma)), 0.0, False, None)
        k = 0
        while k < gamma and drafts[k] == am[k]:
            k += 1
        assert path == list(range(k + 1)) and emitted == am[k]


def test_greedy_takes_first_matching_sibling_and_ties_to_lowest_index():
    V = 10
    parent = [-1, 0, 0, 0, 2, 2]
    tokens = np.array([0, 5, 7, 7, 3, 3], dtype=np.int32)
    logits = np.zeros((6, V), dtype=np.float32)
    logits[0, 7] = 2.0
    logits[2, 3] = 1.0
    logits[2, 8] = 1.0  # tie between tokens 3 and 8: the lower index (3) is the argmax
    logits[4, 1] = 4.0
    path, emitted = reject_sequence(logits, np.full((6, V), 0.1), tokens, parent, 0.0, False, None)
    assert path == [0, 2, 4] and emitted == 1


# ----------------------------------------------------------------------------
# the two random decisions, exactly
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("p_x,q_x", [(0.1, 0.3), (0.3, 0.1), (0.25, 0.25), (0.0, 0.2), (0.2, 0.0),
                                     (1e-7, 0.9), (0.123456789, 0.987654321)])
def test_accept_probability_is_min_one_p_over_q_on_the_24_bit_grid(p_x, q_x):
    r = np.arange(1 << 24, dtype=np.float64) * 2.0 ** -24
    frac = np.count_nonzero(accept_draw(r, p_x, q_x)) / 2.0 ** 24
    want = 1.0 if (q_x == 0 and p_x > 0) else (0.0 if q_x == 0 else min(1.0, p_x / q_x))
    assert abs(frac - want) <= 2.0 ** -24


def test_inverse_cdf_reproduces_weights_on_a_grid():
    w = np.array([0.2, 0.0, 0.35, 0.05, 0.4, 0.0])
    n = 1 << 16
    counts = np.bincount([inverse_cdf(w, k / n) for k in range(n)], minlength=w.size)
    np.testing.assert_allclose(counts / n, w / w.sum(), atol=2.0 / n)
    assert counts[1] == 0 and counts[5] == 0
    # unnormalised weights: the scan's own total is used
    assert inverse_cdf(w * 7.0, 0.21) == inverse_cdf(w, 0.21) == 2


def test_residual_and_without_replacement_invariants():
    rng = np.random.default_rng(3)
    for _ in range(50):
        p = rng.dirichlet(np.ones(9))
        q = rng.dirichlet(np.ones(9))
        r = residual_update(p, q)
        assert abs(r.sum() - 1) < 1e-12
        assert (r[p <= q] == 0).all() and (r[p > q] > 0).all()
        x = int(rng.integers(9))
        q2 = without_replacement_update(q, x)
        assert q2[x] == 0 and abs(q2.sum() - 1) < 1e-12
        np.testing.assert_allclose(q2[np.arange(9) != x], q[np.arange(9) != x] / (1 - q[x]))
    p = np.array([0.5, 0.5])
    assert (residual_update(p, p) == p).all()  # zero residual mass leaves p unchanged


# ----------------------------------------------------------------------------
# exact enumeration
# ----------------------------------------------------------------------------

class _Need(Exception):
    def __init__(self, alts):
        super().__init__()
        self.alts = alts


class _Scripted:
    """Decision source that replays a script and asks for the branches past its end.

    Accept weight = min(1, p/q): the probability that r*q < p for r ~ U[0, 1)."""

    def __init__(self, script):
        self.script = script
        self.i = 0
        self.path_len = 0

    def _next(self, alts):
        if self.i < len(self.script):
            self.i += 1
            return self.script[self.i - 1]
        raise _Need(alts)

    def accept(self, b, node, p_x, q_x):
        a = (1.0 if p_x > 0 else 0.0) if q_x == 0 else min(1.0, p_x / q_x)
        return self._next([(True, a), (False, 1.0 - a)])

    def sample(self, b, node, weights):
        w = np.asarray(weights, dtype=np.float64)
        w = w / w.sum()
        return self._next([(x, float(w[x])) for x in range(w.size)])


def _walk_outcomes(run):
    out = []

    def rec(script, weight):
        try:
            res = run(_Scripted(script))
        except _Need as need:
            for choice, w in need.alts:
                if w > 0:
                    rec(script + [choice], weight * w)
            return
        out.append((res, weight))

    rec([], 1.0)
    return out


def _token_paths(parent, tokens):
    paths = [()]
    for i in range(1, len(parent)):
        paths.append(paths[parent[i]] + (int(tokens[i]),))
    return paths


def _draft_assignments(parent, q_of, mode, V):
    """Every token assignment of the non-root nodes with its drafting probability."""
    tree = tree_structure(parent)
    T = len(parent)
    results = []

    def rec(u, tokens, prob):
        if u == T:
            results.append((tokens.copy(), prob))
            return
        kids = tree.children[u]
        if not kids:
            rec(u + 1, tokens, prob)
            return
        q = q_of(_token_paths(parent, tokens)[u])

        def group(k, avail_q, pr):
            if k == len(kids):
                rec(u + 1, tokens, pr)
                return
            tot = avail_q.sum() if mode == "without_replacement" else 1.0
            for x in range(V):
                if avail_q[x] <= 0:
                    continue
                tokens[kids[k]] = x
                nq = avail_q.copy()
                if mode == "without_replacement":
                    nq[x] = 0.0
                group(k + 1, nq, pr * avail_q[x] / tot)
            tokens[kids[k]] = 0

        group(0, q.copy(), prob)

    rec(0, np.zeros(T, dtype=np.int32), 1.0)
    return results


def _model(V, depth, seed, tau):
    """Rows indexed by token path, so that equal histories have equal distributions."""
    rng = np.random.default_rng(seed)
    logits, draft = {}, {}
    paths = [()]
    for _ in range(depth + 1):
        nxt = []
        for h in paths:
            logits[h] = (2 * rng.standard_normal(V)).astype(np.float32)
            d = logits[h] + rng.standard_normal(V)
            e = np.exp(d - d.max())
            # multiples of 2^-20 summing to exactly 1: an exact distribution in float32
            k = np.maximum(np.floor(e / e.sum() * 2 ** 20), 1)
            k[np.argmax(k)] += 2 ** 20 - k.sum()
            draft[h] = (k * 2.0 ** -20).astype(np.float32)
            nxt += [h + (x,) for x in range(V)]
        paths = nxt
    return logits, draft


def _emitted_distribution(parent, V, tau, verifier_wo, draft_mode, seed):
    depth = max(tree_structure(parent).depth)
    logits, draft = _model(V, depth, seed, tau)
    dist = {}
    for tokens, pr in _draft_assignments(parent, lambda h: draft[h].astype(np.float64), draft_mode, V):
        tp = _token_paths(parent, tokens)
        lg = np.stack([logits[h] for h in tp])
        qq = np.stack([draft[h] for h in tp])

        def run(src, lg=lg, qq=qq, tokens=tokens):
            return reject_sequence(lg, qq, tokens, parent, tau, verifier_wo, src)

        for (path, emitted), w in _walk_outcomes(run):
            seq = tuple(int(tokens[n]) for n in path[1:]) + (int(emitted),)
            dist[seq] = dist.get(seq, 0.0) + pr * w
    return dist, logits


def _max_deviation_from_target(dist, logits, tau, V):
    """max over histories h and tokens y of |A(h+y) - p_h(y) * sum_y' A(h+y')|,
    A(h) = probability that the emitted sequence starts with h."""
    A = {}
    for seq, w in dist.items():
        for k in range(len(seq) + 1):
            A[seq[:k]] = A.get(seq[:k], 0.0) + w
    dev = abs(A[()] - 1.0)
    for h in list(A):
        tot = sum(A.get(h + (y,), 0.0) for y in range(V))
        if tot == 0.0:
            continue
        p = softmax64(logits[h], tau)
        for y in range(V):
            dev = max(dev, abs(A.get(h + (y,), 0.0) - p[y] * tot))
    return dev


SHAPES = {
    "three_siblings": [-1, 0, 0, 0],
    "two_by_two": [-1, 0, 0, 1, 1, 2, 2],
    "chain3": [-1, 0, 1, 2],
}


@pytest.mark.parametrize("shape,V", [("three_siblings", 4), ("two_by_two", 3), ("chain3", 3),
                                     ("three_siblings", 3)])
@pytest.mark.parametrize("tau", [1.0, 0.6])
@pytest.mark.parametrize("variant", ["with_replacement", "without_replacement"])
def test_exact_enumeration_recovers_target_distribution(shape, V, tau, variant):
    wo = variant == "without_replacement"
    dist, logits = _emitted_distribution(SHAPES[shape], V, tau, wo,
                                         "without_replacement" if wo else "iid", seed=V * 7 + len(shape))
    assert abs(sum(dist.values()) - 1.0) < 1e-12
    assert _max_deviation_from_target(dist, logits, tau, V) < 1e-12


@pytest.mark.parametrize("verifier_wo,draft_mode", [(False, "without_replacement"), (True, "iid")])
def test_exact_enumeration_detects_mismatched_pairing(verifier_wo, draft_mode):
    dist, logits = _emitted_distribution(SHAPES["three_siblings"], 4, 1.0, verifier_wo, draft_mode, seed=11)
    assert _max_deviation_from_target(dist, logits, 1.0, 4) > 1e-3


# ----------------------------------------------------------------------------
# the real Philox-driven walk, statistically
# ----------------------------------------------------------------------------

def _philox_trials(parent, V, tau, wo, n, seed):
    depth = max(tree_structure(parent).depth)
    logits, draft = _model(V, depth, seed, tau)
    rng = np.random.default_rng(seed + 1)
    firsts = np.zeros(V, dtype=np.int64)
    accepted_first = 0
    tree = tree_structure(parent)
    for trial in range(n):
        tokens = np.zeros(len(parent), dtype=np.int32)
        for u in range(len(parent)):
            kids = tree.children[u]
            if not kids:
                continue
            q = draft[_token_paths(parent, tokens)[u]].astype(np.float64)
            q = q / q.sum()
            if wo:
                xs = []
                qq = q.copy()
                for _ in kids:
                    x = int(rng.choice(V, p=qq / qq.sum()))
                    xs.append(x)
                    qq[x] = 0
            else:
                xs = rng.choice(V, size=len(kids), p=q).tolist()
            tokens[kids] = xs
        tp = _token_paths(parent, tokens)
        lg = np.stack([logits[h] for h in tp])
        qq = np.stack([draft[h] for h in tp])
        path, emitted = reject_sequence(lg, qq, tokens, parent, tau, wo, PhiloxDraws(seed, trial))
        first = int(tokens[path[1]]) if len(path) > 1 else int(emitted)
        firsts[first] += 1
        accepted_first += len(path) > 1
    return firsts, accepted_first, logits, draft


@pytest.mark.parametrize("wo", [False, True])
def test_chi_square_first_token_follows_target(wo):
    n = 20000
    V, tau = 6, 1.0
    firsts, _, logits, _ = _philox_trials([-1, 0, 0, 0, 1, 2], V, tau, wo, n, seed=21)
    p = softmax64(logits[()], tau)
    assert stats.chisquare(firsts, n * p).pvalue > 1e-3


def test_single_child_acceptance_rate_is_sum_of_min():
    n = 20000
    V, tau = 5, 1.0
    _, acc, logits, draft = _philox_trials([-1, 0], V, tau, False, n, seed=33)
    p = softmax64(logits[()], tau)
    q = draft[()].astype(np.float64) / draft[()].astype(np.float64).sum()
    beta = np.minimum(p, q).sum()
    assert abs(acc / n - beta) < 4 * np.sqrt(beta * (1 - beta) / n)


def test_temperature_to_zero_gives_greedy():
    rng = np.random.default_rng(4)
    V = 12
    for trial in range(40):
        T = 9
        parent = [-1] + [int(rng.integers(0, i)) for i in range(1, T)]
        logits = rng.standard_normal((T, V)).astype(np.float32)
        am = logits.argmax(1)
        logits[np.arange(T), am] += 3.0
        tokens = np.array([0] + [am[parent[i]] if rng.random() < 0.5 else int(rng.integers(V))
                                 for i in range(1, T)], dtype=np.int32)
        q = rng.dirichlet(np.ones(V), size=T).astype(np.float32)
        g = reject_sequence(logits, q, tokens, parent, 0.0, False, None)
        for wo in (False, True):
            s = reject_sequence(logits, q, tokens, parent, 0.02, wo, PhiloxDraws(trial, 0))
            assert s == g


def test_tree_reject_output_format_and_flags():
    from workloads import make_config
    w = make_config(0)
    res = tree_reject(w.target_logits, w.draft_probs, w.draft_tokens, w.parent, w.temperature,
                      w.without_replacement, w.seed, w.offset)
    L = int(res["num_accepted"][0])
    acc = res["accepted_nodes"][0]
    assert acc[0] == 0 and (np.diff(acc[:L + 1]) > 0).all() and (acc[L + 1:] == -1).all()
    tree = tree_structure(w.parent[0])
    for d in range(1, L + 1):
        assert tree.parent[acc[d]] == acc[d - 1]
    assert res["out_tokens"][0, :L].tolist() == [int(w.draft_tokens[0][n]) for n in acc[1:L + 1]]
    assert 0 <= res["out_tokens"][0, L] < w.V
    assert res["flag_path_len"][0] == -1  # no draw of this seed sits within 1e-6 of a threshold


def test_final_draw_candidates_bracket_the_draw():
    from oracle.reject import final_draw_candidates
    w = np.array([0.25, 0.0, 0.25, 0.5])
    assert final_draw_candidates(w, 0.5 + 1e-7).tolist() == [2, 3]  # at the boundary between 2 and 3
    assert final_draw_candidates(w, 0.7).tolist() == [3]
    assert final_draw_candidates(w, 0.25 - 5e-7).tolist() == [0, 2]  # token 1 has no weight
