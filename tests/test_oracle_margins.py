"""Pins for the oracle's draw margins, which decide which GPU disagreements are excused.

A draw is flagged when its uniform lies within 1e-6 of the value at which the
decision would change.  For the accept test r * q(x) < p(x) ("Speculative
Decoding" notes, "Draft Token Validation") that value is r = p(x)/q(x); for the
final draw by inverse CDF it is either edge of the chosen token's interval of
the normalised CDF.  Both margins, the flag probabilities that set the GPU
tests' caps on flagged sequences, and the candidate set of a flagged final draw
are checked on hand-worked cases, by brute force over a grid of uniforms, and
end to end through tree_reject on an input built to land a draw within 1e-6 of
its threshold.  Copies with planted mistakes (margin taken as |r q - p|, the
ratio inverted, the CDF not normalised, the lower edge one token off, only the
upper edge, zero-weight tokens kept as candidates, the flag probability without
its cap) must each fail one of the pins.
"""
import math

import numpy as np
import pytest

from oracle import (FLAG_MARGIN, accept_flag_probability, accept_margin, final_draw_candidates,
                    final_flag_probability, final_margin, inverse_cdf, tree_reject, uniform_draw)
from oracle.philox import PURPOSE_FINAL

W4 = np.array([1.0, 2.0, 3.0, 4.0])  # normalised CDF 0.1, 0.3, 0.6, 1.0


# ----------------------------------------------------------------------------
# the pins, each a function of the implementations under test, so that the
# planted mistakes below can be run through the same checks
# ----------------------------------------------------------------------------

def accept_margin_pins(am) -> bool:
    # hand-worked: |r - p/q|
    cases = [(0.3, 0.1, 0.2, 0.2),        # ratio 0.5
             (0.9, 0.3, 0.1, 2.1),        # ratio 3: accepted for every r, far from the threshold
             (0.25, 0.25, 0.25, 0.75),    # ratio 1
             (0.0, 0.0, 0.5, 0.0),        # p = 0, r = 0: exactly on the threshold (rejected)
             (0.7, 0.35, 0.5, 0.0)]       # r = p/q exactly
    for r, p, q, want in cases:
        if not math.isclose(am(r, p, q), want, rel_tol=1e-12, abs_tol=1e-15):
            return False
    return am(0.5, 0.2, 0.0) == math.inf  # q = 0: the decision does not depend on r


def final_margin_pins(fm) -> bool:
    # weights 1, 2, 3, 4: intervals [0, .1), [.1, .3), [.3, .6), [.6, 1)
    cases = [(W4, 0.35, 2, 0.05), (W4, 0.05, 0, 0.05), (W4, 0.99, 3, 0.01), (W4, 0.3, 2, 0.0),
             (W4 * 7.0, 0.35, 2, 0.05),                      # scale-free
             (np.array([0.0, 2.0, 0.0, 2.0]), 0.75, 3, 0.25),  # zero-weight tokens own no interval
             (np.array([5.0]), 0.2, 0, 0.2)]
    for w, u, x, want in cases:
        if inverse_cdf(w, u) != x or not math.isclose(fm(w, u, x), want, rel_tol=1e-12, abs_tol=1e-15):
            return False
    return True


def candidate_pins(cand) -> bool:
    m = FLAG_MARGIN
    checks = [(W4, 0.3 + 0.5 * m, [1, 2]), (W4, 0.3 - 0.5 * m, [1, 2]), (W4, 0.45, [2]),
              (W4, 0.5 * m, [0]), (W4, 1.0 - 0.5 * m, [3]),
              # a zero-weight token between two others is never a candidate
              (np.array([1.0, 0.0, 1.0]), 0.5, [0, 2])]
    return all(list(cand(w, u)) == want for w, u, want in checks)


def _grid_fraction(pred, n=1 << 18):
    u = (np.arange(n) + 0.5) / n
    return float(np.mean([pred(x) for x in u]))


def flag_probability_pins(fp_final, fp_accept, fm, am) -> bool:
    # brute force over a grid of uniforms at a margin wide enough for the grid to resolve
    m = 1e-2
    for w in (W4, np.array([0.004, 1.0, 0.003, 2.0, 0.0, 0.5]), np.array([1.0])):
        want = _grid_fraction(lambda u: fm(w, u, inverse_cdf(w, u)) < m, n=1 << 16)
        if abs(fp_final(w, m) - want) > 2e-4:
            return False
    for p, q in ((0.1, 0.2), (0.3, 0.1), (0.2, 0.205), (0.0, 0.4), (0.004, 0.8)):
        r = (np.arange(1 << 16) + 0.5) / (1 << 16)
        want = float(np.mean([am(x, p, q) < m for x in r]))
        if abs(fp_accept(p, q, m) - want) > 2e-4:
            return False
    # closed form at the real margin: a token of mass above 2m contributes 2m, a lighter one its mass
    w = np.array([0.5, 0.5 - 3e-6, 1e-6, 2e-6])
    return math.isclose(fp_final(w), 2 * FLAG_MARGIN * 2 + 1e-6 + 2e-6, rel_tol=1e-9)


# ----------------------------------------------------------------------------
# the oracle passes every pin
# ----------------------------------------------------------------------------

def test_accept_margin_hand_worked():
    assert accept_margin_pins(accept_margin)


def test_final_margin_hand_worked():
    assert final_margin_pins(final_margin)


def test_final_candidates_hand_worked():
    assert candidate_pins(final_draw_candidates)


def test_flag_probabilities_against_brute_force():
    assert flag_probability_pins(final_flag_probability, accept_flag_probability, final_margin, accept_margin)


def test_flag_end_to_end_final_draw():
    # a root-only tree (the root is a leaf): one bonus draw from softmax of two
    # logits, with p(0) set 5e-7 above the uniform the draw uses, so the draw is
    # taken within 1e-6 of the edge between the two tokens and must be flagged
    seed, offset = 7, 3
    u = uniform_draw(seed, offset, 0, 0, PURPOSE_FINAL)
    p0 = u + 5e-7
    a = np.float32(math.log(p0 / (1.0 - p0)))
    logits = np.array([[[a, 0.0]]], dtype=np.float32)
    q = np.full((1, 1, 2), 0.5, dtype=np.float32)
    res = tree_reject(logits, q, np.zeros((1, 1), np.int32), np.array([[-1]], np.int32), 1.0, False, seed, offset)
    assert res["flag_path_len"][0] == 1 and res["flag_kind"][0] == "final"
    assert sorted(res["final_candidates"][0].tolist()) == [0, 1]
    assert res["margins"][0] < FLAG_MARGIN
    assert math.isclose(res["flag_prob"][0], 2 * FLAG_MARGIN * 2, rel_tol=1e-9)
    # moved 1e-3 away the same draw is not flagged, and its flag probability is unchanged
    a2 = np.float32(math.log((u + 1e-3) / (1.0 - u - 1e-3)))
    res2 = tree_reject(np.array([[[a2, 0.0]]], np.float32), q, np.zeros((1, 1), np.int32),
                       np.array([[-1]], np.int32), 1.0, False, seed, offset)
    assert res2["flag_path_len"][0] == -1 and res2["out_tokens"][0, 0] == 0


def test_flag_end_to_end_accept_test():
    # one child whose accept ratio p(x)/q(x) sits 2e-7 above its uniform: flagged
    # at path length 1 (the root's decision), with the accept record's margin
    seed, offset = 12, 0  # r = 0.818: q(0) = p(0)/ratio stays a probability
    r = uniform_draw(seed, offset, 0, 1, 0)
    assert r > 0.5
    V = 2
    ratio = r + 2e-7
    # p(0) = 1/2 from equal logits, q(0) = p(0)/ratio
    logits = np.zeros((1, 2, V), dtype=np.float32)
    q = np.zeros((1, 2, V), dtype=np.float32)
    q[0, 0, 0] = np.float32(0.5 / ratio)
    q[0, 0, 1] = np.float32(1.0 - q[0, 0, 0])
    q[0, 1] = 0.5
    tok = np.array([[0, 0]], np.int32)
    res = tree_reject(logits, q, tok, np.array([[-1, 0]], np.int32), 1.0, False, seed, offset)
    want = abs(r - 0.5 / float(q[0, 0, 0]))
    assert res["flag_kind"][0] == "accept" and res["flag_path_len"][0] == 1
    assert math.isclose(res["margins"][0], want, rel_tol=1e-12) and want < FLAG_MARGIN


# ----------------------------------------------------------------------------
# planted mistakes: each copy fails at least one pin
# ----------------------------------------------------------------------------

def _am_product(r, p, q):  # |r q - p| instead of |r - p/q|
    return math.inf if q <= 0 else abs(r * q - p)


def _am_inverted(r, p, q):  # |r - q/p|
    return math.inf if q <= 0 else (abs(r - q / p) if p > 0 else math.inf)


def _fm_unnormalised(w, u, x):  # CDF edges not divided by the total
    c = np.cumsum(np.asarray(w, dtype=np.float64))
    lo = c[x - 1] if x > 0 else 0.0
    return min(u - lo, c[x] - u)


def _fm_lower_edge_off_by_one(w, u, x):
    c = np.cumsum(np.asarray(w, dtype=np.float64))
    lo = c[x - 2] / c[-1] if x > 1 else 0.0
    return min(u - lo, c[x] / c[-1] - u)


def _fm_upper_only(w, u, x):
    c = np.cumsum(np.asarray(w, dtype=np.float64))
    return c[x] / c[-1] - u


def _cand_keeps_zero_weight(w, u, margin=None):
    m = FLAG_MARGIN if margin is None else margin
    w = np.asarray(w, dtype=np.float64)
    c = np.cumsum(w) / w.sum()
    lo = np.concatenate([[0.0], c[:-1]])
    return np.nonzero((lo <= u + m) & (c >= u - m))[0]


def _fp_uncapped(w, margin=None):  # every token counted at 2m, however light
    m = FLAG_MARGIN if margin is None else margin
    return float(2.0 * m * np.count_nonzero(np.asarray(w) > 0))


def _fp_accept_one_sided(p, q, margin=None):  # only r below the threshold counted
    m = FLAG_MARGIN if margin is None else margin
    if q <= 0:
        return 0.0
    ratio = p / q
    return max(0.0, min(1.0, ratio) - max(0.0, ratio - m))


@pytest.mark.parametrize("name,ok", [
    ("accept margin |rq - p|", lambda: accept_margin_pins(_am_product)),
    ("accept margin |r - q/p|", lambda: accept_margin_pins(_am_inverted)),
    ("final margin, CDF not normalised", lambda: final_margin_pins(_fm_unnormalised)),
    ("final margin, lower edge one token off", lambda: final_margin_pins(_fm_lower_edge_off_by_one)),
    ("final margin, upper edge only", lambda: final_margin_pins(_fm_upper_only)),
    ("candidates keep zero-weight tokens", lambda: candidate_pins(_cand_keeps_zero_weight)),
    ("flag probability without the cap at the token's mass",
     lambda: flag_probability_pins(_fp_uncapped, accept_flag_probability, final_margin, accept_margin)),
    ("accept flag probability one-sided",
     lambda: flag_probability_pins(final_flag_probability, _fp_accept_one_sided, final_margin, accept_margin)),
])
def test_planted_mistake_fails_a_pin(name, ok):
    assert not ok(), f"the pins do not catch: {name}"


# ----------------------------------------------------------------------------
# the cap the GPU tests put on flagged sequences
# ----------------------------------------------------------------------------

def test_flag_cap_is_the_binomial_upper_quantile():
    from scipy import stats

    from helpers import flag_cap

    for n, p in ((12, 0.05), (128, 0.05), (500, 0.3), (40, 1e-6)):
        k = flag_cap([p] * n)
        assert stats.binom.sf(k, n, p) <= 1e-6
        assert k == 0 or stats.binom.sf(k - 1, n, p) > 1e-6
    assert flag_cap([]) == 0 and flag_cap([0.0, 0.0]) == 0 and flag_cap([1.0, 1.0]) == 2


def test_flag_rate_of_the_batched_serving_workload_follows_its_probabilities():
    # 64 sequences at V = 32000, four offsets: the flagged count must lie inside
    # the central 1 - 2e-6 range of its Poisson-binomial distribution
    from helpers import flag_cap
    from workloads import make_config

    w = make_config(4, with_kv=False)
    flagged, probs = 0, []
    for off in range(4):
        r = tree_reject(w.target_logits, w.draft_probs, w.draft_tokens, w.parent, w.temperature,
                        w.without_replacement, w.seed, off)
        flagged += int((r["flag_path_len"] >= 0).sum())
        probs.extend(r["flag_prob"].tolist())
    lo = len(probs) - flag_cap([1.0 - p for p in probs])  # lower quantile: n minus the cap of the complements
    assert lo <= flagged <= flag_cap(probs), (flagged, sum(probs))
    assert 0.02 < np.mean(probs) < 0.08  # about sum_x min(p(x), 2e-6) per final draw at V = 32000
