"""Tree rejection sampling (oracle side), fp64.

Per sequence the verifier walks the draft tree from the root.  Rule for one
drafted token x at the current node ("Speculative Decoding" notes, section
"Draft Token Validation"): with p the target and q the draft distribution,
accept when p(x) >= q(x); otherwise accept when a uniform r falls below
p(x)/q(x).  Both cases are the single test r*q(x) < p(x) for r in [0, 1).
On rejection the target is replaced by the residual max(0, p - q),
renormalised, and the next token is drawn from it; when every drafted token is
accepted, the bonus token is drawn from the distribution after the last one.

Trees: the children of the current node are tried in turn (increasing node
index).  A rejected child turns p into the residual before the next sibling is
tested.  With replacement (siblings drafted i.i.d. from q) q is kept; the
Sequoia variant ("Sequoia: Scalable and Robust Speculative Decoding" summary,
"Robust Sampling": sampling without replacement so bad tokens are not re-tried)
zeroes the rejected token in q and renormalises q.  An accepted child becomes
the current node; a node whose children are all rejected (or a leaf) ends the
walk with one draw from the current p.  Greedy verification (temperature 0)
accepts the first child whose token is the target's argmax and otherwise emits
that argmax (the SGLang "SpeculativeDecoding" doc, "Target Verification": full
match, no match, prefix match).

Readings taken where the pages are silent: p = softmax(logits / temperature);
q is used exactly as given (not renormalised); a residual with zero total mass
leaves p unchanged; the final draw is the inverse CDF in vocabulary order with
the scan's own total; ties of the argmax go to the lowest index.
"""
from __future__ import annotations

import math

import numpy as np

from .philox import PURPOSE_ACCEPT, PURPOSE_FINAL, uniform_draw
from .tree import tree_structure

FLAG_MARGIN = 1e-6  # draws closer than this to a decision threshold are flagged


def softmax64(logits_row, temperature) -> np.ndarray:
    """p = softmax(logits / temperature), max-subtracted, in fp64."""
    z = np.asarray(logits_row, dtype=np.float64) / float(temperature)
    z = z - z.max()
    e = np.exp(z)
    return e / e.sum()


def accept_draw(r, p_x, q_x):
    """Accept test for a uniform r in [0, 1): accept iff r * q(x) < p(x)."""
    return r * q_x < p_x


def residual_update(p: np.ndarray, q: np.ndarray) -> np.ndarray:
    """p <- max(p - q, 0) / sum(max(p - q, 0)); unchanged if that sum is 0."""
    w = np.maximum(p - q, 0.0)
    s = w.sum()
    return w / s if s > 0 else p


def without_replacement_update(q: np.ndarray, x: int) -> np.ndarray:
    """Remove a rejected token from the draft distribution and renormalise."""
    q = q.copy()
    q_old = q[x]
    q[x] = 0.0
    if q_old < 1.0:
        q = q / (1.0 - q_old)
    return q


def inverse_cdf(weights: np.ndarray, u: float) -> int:
    """Smallest x with C[x] > u * C[V-1], C the running sum in index order."""
    c = np.cumsum(np.asarray(weights, dtype=np.float64))
    x = int(np.searchsorted(c, u * c[-1], side="right"))
    if x >= c.shape[0]:
        raise ValueError("inverse CDF over an all-zero weight vector")
    return x


def accept_margin(r, p_x, q_x):
    """Distance of the uniform r from the accept threshold p(x)/q(x) of the
    test r * q(x) < p(x); infinite when q(x) = 0 (the decision then does not
    depend on r)."""
    if q_x <= 0:
        return math.inf
    return abs(float(r) - float(p_x) / float(q_x))


def final_margin(weights, u, x):
    """Distance of the uniform u from the nearer edge of the chosen token's
    interval [C[x-1], C[x]) / C[V-1] of the normalised CDF (C[-1] = 0)."""
    c = np.cumsum(np.asarray(weights, dtype=np.float64))
    lo = c[x - 1] / c[-1] if x > 0 else 0.0
    return min(u - lo, c[x] / c[-1] - u)


def accept_flag_probability(p_x, q_x, margin=None):
    """Probability over a uniform r in [0, 1) that accept_margin(r, p_x, q_x) < margin:
    the length of (ratio - margin, ratio + margin) inside [0, 1)."""
    margin = FLAG_MARGIN if margin is None else margin
    if q_x <= 0:
        return 0.0
    ratio = float(p_x) / float(q_x)
    return max(0.0, min(1.0, ratio + margin) - max(0.0, ratio - margin))


def final_flag_probability(weights, margin=None):
    """Probability over a uniform u in [0, 1) that the final draw from `weights`
    is flagged: u falls within `margin` of an edge of the interval of the token
    it selects.  Token x's interval has length w(x)/W; the part of it within
    `margin` of either edge has length min(w(x)/W, 2 margin)."""
    margin = FLAG_MARGIN if margin is None else margin
    w = np.asarray(weights, dtype=np.float64)
    return float(np.minimum(w / w.sum(), 2.0 * margin).sum())


def final_draw_candidates(weights, u, margin=None):
    """Tokens whose normalised CDF interval [C[x-1], C[x]) / C[V-1] lies within
    `margin` of u (nonzero weight only): the tokens a draw flagged at that
    margin may legitimately return."""
    margin = FLAG_MARGIN if margin is None else margin
    w = np.asarray(weights, dtype=np.float64)
    c = np.cumsum(w) / w.sum()
    lo = np.concatenate([[0.0], c[:-1]])
    return np.nonzero((w > 0) & (lo < u + margin) & (c > u - margin))[0]


class PhiloxDraws:
    """The real source of randomness: Philox4x32-10 uniforms, with margins recorded."""

    def __init__(self, seed: int, offset: int):
        self.seed = int(seed)
        self.offset = int(offset)
        self.records = []  # (kind, b, node, margin, path_len, flag probability of the draw)
        self.path_len = 0
        self.final_candidates = None  # set when the final draw is flagged

    def accept(self, b, node, p_x, q_x) -> bool:
        r = uniform_draw(self.seed, self.offset, b, node, PURPOSE_ACCEPT)
        self.records.append(("accept", b, node, accept_margin(r, p_x, q_x), self.path_len,
                             accept_flag_probability(p_x, q_x)))
        return bool(accept_draw(r, p_x, q_x))

    def sample(self, b, node, weights) -> int:
        u = uniform_draw(self.seed, self.offset, b, node, PURPOSE_FINAL)
        x = inverse_cdf(weights, u)
        m = final_margin(weights, u, x)
        self.records.append(("final", b, node, m, self.path_len, final_flag_probability(weights)))
        if m < FLAG_MARGIN:
            self.final_candidates = final_draw_candidates(weights, u)
        return x


def reject_sequence(logits_b, q_b, tokens_b, parent_b, temperature, without_replacement,
                    draws, b=0):
    """Walk one sequence's tree.  Returns (path, emitted_token).

    path[0] = 0 (root) followed by the accepted nodes; the emitted token is the
    residual / bonus draw (or the greedy argmax)."""
    tree = tree_structure(parent_b)
    V = logits_b.shape[-1]
    for c in range(1, tree.T):
        if not 0 <= int(tokens_b[c]) < V:
            raise ValueError(f"draft token of node {c} out of range")
    path = [0]
    u = 0
    if float(temperature) == 0.0:
        while True:
            t = int(np.argmax(logits_b[u]))
            nxt = next((c for c in tree.children[u] if int(tokens_b[c]) == t), None)
            if nxt is None:
                return path, t
            path.append(nxt)
            u = nxt
    while True:
        p = softmax64(logits_b[u], temperature)
        q = np.asarray(q_b[u], dtype=np.float64).copy()
        accepted = None
        if draws is not None:
            draws.path_len = len(path)
        for c in tree.children[u]:
            x = int(tokens_b[c])
            if draws.accept(b, c, p[x], q[x]):
                accepted = c
                break
            p = residual_update(p, q)
            if without_replacement:
                q = without_replacement_update(q, x)
        if accepted is None:
            return path, draws.sample(b, u, p)
        path.append(accepted)
        u = accepted


def tree_reject(target_logits, draft_probs, draft_tokens, parent, temperature,
                without_replacement, seed, offset):
    """All sequences.  The temperature is taken as the float32 value a caller passes.

    Returns a dict with accepted_nodes [B, T] and out_tokens [B, T] (unused
    entries -1), num_accepted [B] (= L, the number of accepted draft nodes),
    and `flag_path_len` [B]: -1 if no draw of the sequence came within
    FLAG_MARGIN of its threshold, else the path length when the first such
    draw was taken (outputs beyond that point are not decided robustly);
    `flag_kind` [B]: "" / "accept" / "final" for that first flagged draw, and
    `final_candidates`: {b: tokens a flagged final draw may return};
    `flag_prob` [B]: the probability, over the uniforms of the draws the walk
    took, that at least one of them is flagged (1 - prod(1 - p_draw)); the
    number of flagged sequences in a batch is a sum of independent Bernoulli
    variables with these means."""
    B, T, V = target_logits.shape
    tau = float(np.float32(temperature))
    acc = np.full((B, T), -1, dtype=np.int32)
    out = np.full((B, T), -1, dtype=np.int32)
    nacc = np.zeros(B, dtype=np.int32)
    flag = np.full(B, -1, dtype=np.int32)
    kind_of = [""] * B
    cands = {}
    margins = []
    fprob = np.zeros(B, dtype=np.float64)
    for b in range(B):
        draws = PhiloxDraws(seed, offset)
        path, emitted = reject_sequence(target_logits[b], draft_probs[b], draft_tokens[b],
                                        parent[b], tau, without_replacement, draws, b)
        L = len(path) - 1
        acc[b, :L + 1] = path
        out[b, :L] = [int(draft_tokens[b][n]) for n in path[1:]]
        out[b, L] = emitted
        nacc[b] = L
        keep = 1.0
        for kind, _, node, m, plen, pf in draws.records:
            margins.append(m)
            keep *= 1.0 - pf
            if m < FLAG_MARGIN and flag[b] < 0:
                flag[b] = plen
                kind_of[b] = kind
        fprob[b] = 1.0 - keep
        if kind_of[b] == "final":
            cands[b] = draws.final_candidates
    return {"accepted_nodes": acc, "out_tokens": out, "num_accepted": nacc,
            "flag_path_len": flag, "flag_kind": kind_of, "final_candidates": cands,
            "margins": np.array(margins), "flag_prob": fprob}
