"""Top-k / top-p truncation of the target distribution before the acceptance
tests (oracle side), fp64 -- TEST INFRASTRUCTURE ONLY.

The Sequoia summary ("Sequoia: Scalable and Robust Speculative Decoding",
the robustness table over the top-p hyperparameter and the empirical
validation section) verifies drafts against a target sampled with nucleus
(top-p) truncation, but gives no definition.  The definitions taken here come
from outside the pages:

* top-k (Fan et al., "Hierarchical Neural Story Generation", 2018): keep the
  k largest logits;
* top-p (Holtzman et al., "The Curious Case of Neural Text Degeneration",
  2020): keep the smallest set of most probable tokens whose probability
  under p = softmax(logits / temperature) reaches top_p.

Readings taken where the definitions leave a choice:
* a threshold rule, so that equal logits are never split: the kept set is
  {x : logit(x) >= t}, with t the k-th largest logit for top-k and, for top-p,
  the largest logit value v for which the mass of {logit >= v} reaches top_p;
* both given: top-k first, then top-p over the distribution renormalised on
  the top-k set;
* temperature 0: the nucleus is the set of tokens tied at the maximum (the
  limit of softmax(logits / tau) as tau -> 0); top-k is applied as for tau > 0;
* logits equal to -inf are already outside every kept set and do not count
  toward k; top_k <= 0 or >= the number of finite logits, and top_p >= 1,
  switch the respective rule off;
* only the target's logits are truncated; q is the distribution the drafts
  were actually drawn from and is used as given (a draft sampled with its own
  truncation passes the truncated q);
* dropped logits become -inf, so p of a dropped token is 0 in every later
  step of the sampler (acceptance tests, residuals, final draw).

Speculative rejection sampling then returns tokens distributed as the
truncated target, as it does for any target distribution.
"""
from __future__ import annotations

import math

import numpy as np

from .reject import softmax64


def _keep_top_k(vals: np.ndarray, finite: np.ndarray, top_k: int) -> np.ndarray:
    """Mask of {x : v(x) >= k-th largest finite v}."""
    n = int(finite.sum())
    if top_k <= 0 or top_k >= n:
        return finite.copy()
    desc = np.sort(vals[finite])[::-1]
    t = desc[top_k - 1]
    return finite & (vals >= t)


def _keep_top_p(vals: np.ndarray, kept: np.ndarray, temperature: float, top_p: float):
    """Mask of the nucleus within `kept`, and the decision's margin: the
    distance of top_p from the two cumulative masses around the threshold
    (mass of the values above t, and of the values >= t)."""
    if top_p >= 1.0 or not kept.any():
        return kept.copy(), math.inf
    if temperature == 0.0:
        return kept & (vals == vals[kept].max()), math.inf
    pk = softmax64(vals[kept], temperature)                 # renormalised on the kept set
    distinct, group = np.unique(vals[kept], return_inverse=True)
    distinct = distinct[::-1]                               # distinct values, descending
    group_mass = np.bincount(group, weights=pk, minlength=distinct.size)[::-1]
    at = np.cumsum(group_mass)                              # mass of the values >= distinct[j]
    reached = np.flatnonzero(at >= top_p)
    if reached.size == 0:  # the masses summed short of top_p by rounding: keep everything
        return kept.copy(), 0.0
    j = int(reached[0])
    above = float(at[j - 1]) if j > 0 else 0.0              # mass of the values > distinct[j]
    return kept & (vals >= distinct[j]), min(top_p - above, float(at[j]) - top_p)


def truncate_row(logits_row, temperature, top_k, top_p):
    """One row.  Returns (logits with dropped entries set to -inf, as float32;
    margin of the top-p decision, inf when no mass comparison was made)."""
    row = np.asarray(logits_row, dtype=np.float32)
    vals = row.astype(np.float64)
    finite = np.isfinite(vals)
    if np.isnan(vals).any() or np.isposinf(vals).any():
        raise ValueError("NaN or +inf logit")
    keep = _keep_top_k(vals, finite, int(top_k))
    keep, margin = _keep_top_p(vals, keep, float(np.float32(temperature)), float(np.float32(top_p)))
    out = row.copy()
    out[~keep] = -np.inf
    return out, margin


def truncate_logits(target_logits, temperature, top_k, top_p):
    """All rows of [B, T, V] logits.  Returns (truncated float32 logits,
    margins [B, T])."""
    lg = np.asarray(target_logits, dtype=np.float32)
    out = np.empty_like(lg)
    margins = np.empty(lg.shape[:-1], dtype=np.float64)
    for idx in np.ndindex(*lg.shape[:-1]):
        out[idx], margins[idx] = truncate_row(lg[idx], temperature, top_k, top_p)
    return out, margins
