"""Shared test helpers: move a synthetic workload to the GPU, call the library,
compare with the oracle under the stated tolerances."""
from __future__ import annotations

import numpy as np
import torch

import oracle
import tree_verify_attention_masked_amd as stv

# Attention outputs vs the fp64 oracle, per element.  The stated bar:
#   bf16 |gpu - oracle| <= 2e-2 + 1e-2 |oracle|,  fp32 <= 1e-5 + 1e-5 |oracle|.
BF16_ATOL, BF16_RTOL = 2e-2, 1e-2
F32_ATOL, F32_RTOL = 1e-5, 1e-5
# bf16 outputs must also meet a bound derived from the arithmetic, because the
# stated bar is of the order of the outputs themselves once a row averages over
# thousands of keys:
#   |gpu - oracle| <= BF16_U2 * (attn(|V|) + |oracle|) + BF16_FLOOR
# The inputs are exact bf16 values; scores are products of bf16 values summed in
# fp32 (relative error ~1e-5, negligible).  Two roundings to bf16 (unit roundoff
# u = 2^-9) remain: the probabilities that enter the P.V product, each off by at
# most u relative, move the output by at most u * sum_k p_k |v_k| / l =
# u * attn(|V|) (attention with every value replaced by its magnitude, computed
# by the oracle); the output itself is rounded once more, u * |out|.  The bound
# takes twice each term (2u = 2^-8) to leave room for the fp32 accumulations and
# the approximate exp2.  A row sum or a max off by a factor, a key dropped or
# counted twice, or a mask slip all exceed it by orders of magnitude.
BF16_U2 = 2.0 ** -8
BF16_FLOOR = 1e-5


def dev(a, device="cuda"):
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


def dev_kv(w, a, device="cuda"):
    """bf16 bit patterns -> torch.bfloat16 (bit exact); float32 stays float32."""
    t = torch.from_numpy(np.ascontiguousarray(a))
    if w.dtype == "bf16":
        t = t.view(torch.int16).view(torch.bfloat16)
    return t.to(device)


def host_kv(w, t):
    """Inverse of dev_kv: torch tensor -> numpy array in the workload's storage type."""
    t = t.detach().cpu()
    if w.dtype == "bf16":
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


class DevWorkload:
    def __init__(self, w, device="cuda"):
        self.w = w
        self.q = dev_kv(w, w.q, device)
        self.k = None if w.k_cache is None else dev_kv(w, w.k_cache, device)
        self.v = None if w.v_cache is None else dev_kv(w, w.v_cache, device)
        self.block_table = dev(w.block_table, device)
        self.prefix_lens = dev(w.prefix_lens, device)
        self.parent = dev(w.parent, device)
        self.tokens = dev(w.draft_tokens, device)
        self.logits = dev(w.target_logits, device)
        self.probs = dev(w.draft_probs, device)
        self.status = torch.zeros(w.B, dtype=torch.int32, device=device)

    def attn(self):
        return stv.spec_tree_attn(self.q, self.k, self.v, self.block_table, self.prefix_lens, self.parent,
                                  scale=self.w.scale, status=self.status)

    def reject(self, temperature=None, without_replacement=None, seed=None, offset=None):
        w = self.w
        return stv.spec_tree_reject(self.logits, self.probs, self.tokens, self.parent,
                                    w.temperature if temperature is None else temperature,
                                    w.without_replacement if without_replacement is None else without_replacement,
                                    w.seed if seed is None else seed, w.offset if offset is None else offset,
                                    status=self.status)

    def compact(self, acc, nacc):
        return stv.spec_kv_compact(self.k, self.v, self.block_table, self.prefix_lens, acc, nacc,
                                   status=self.status)


def abs_values(w, v_cache):
    """The value cache with every element replaced by its magnitude (bf16: sign
    bit cleared), for the attn(|V|) term of the bf16 bound."""
    if w.dtype == "bf16":
        return np.asarray(v_cache, dtype=np.uint16) & np.uint16(0x7FFF)
    return np.abs(v_cache)


def oracle_attn(w, rows=None):
    """(oracle output, oracle attn(|V|)) for the whole workload or for a list of
    (b, node, head) rows."""
    va = abs_values(w, w.v_cache)
    if rows is None:
        f = lambda v: oracle.tree_attention(w.q, w.k_cache, v, w.block_table, w.prefix_lens, w.parent, w.scale,
                                            dtype=w.dtype)
    else:
        f = lambda v: oracle.tree_attention_rows(w.q, w.k_cache, v, w.block_table, w.prefix_lens, w.parent,
                                                 w.scale, rows, dtype=w.dtype)
    return f(w.v_cache), f(va)


def assert_attn_close(got, ref, dtype, what="", ref_abs=None):
    got = np.asarray(got, dtype=np.float64)
    err = np.abs(got - ref)
    atol, rtol = (BF16_ATOL, BF16_RTOL) if dtype == "bf16" else (F32_ATOL, F32_RTOL)
    bad = ~(err <= atol + rtol * np.abs(ref))
    if bad.any():
        idx = np.argwhere(bad)[:5].tolist()
        raise AssertionError(f"{what}: {int(bad.sum())} of {bad.size} outside the stated tolerance; "
                             f"max abs err {err.max():.3e}; first {idx}")
    if dtype == "bf16":
        assert ref_abs is not None, "the bf16 rounding bound needs attn(|V|) from the oracle"
        bad = ~(err <= BF16_U2 * (np.asarray(ref_abs) + np.abs(ref)) + BF16_FLOOR)
        what = f"{what} (bf16 rounding bound)"
    if bad.any():
        idx = np.argwhere(bad)[:5].tolist()
        raise AssertionError(f"{what}: {int(bad.sum())} of {bad.size} outside tolerance; "
                             f"max abs err {err.max():.3e}; first {idx}")
    return float(err.max())


def attn_to_f64(w, out):
    t = out.detach().float().cpu().numpy()
    return t.astype(np.float64)


def compare_reject(got, ref, stats=None):
    """Bit-exact comparison of the walk outputs with the oracle's.

    A sequence none of whose draws the oracle flags (within 1e-6 of its
    threshold) must match exactly.  If the first flagged draw is the final
    one, the path, L and accepted tokens must still match exactly and the
    emitted token must be one of the tokens whose CDF interval lies within
    1e-6 of the uniform.  If an accept test is flagged, the path decided
    before it must match.  Returns the number of flagged sequences."""
    acc, toks, nacc = (t.cpu().numpy() for t in got)
    flagged = 0
    for b in range(acc.shape[0]):
        fl = int(ref["flag_path_len"][b])
        kind = ref["flag_kind"][b] if "flag_kind" in ref else ""
        if fl >= 0:
            flagged += 1
            assert (acc[b, :fl] == ref["accepted_nodes"][b, :fl]).all(), f"seq {b}: path differs before a flagged draw"
            if kind == "final":
                L = int(ref["num_accepted"][b])
                assert nacc[b] == L and (acc[b] == ref["accepted_nodes"][b]).all(), f"seq {b}: path"
                assert (toks[b, :L] == ref["out_tokens"][b, :L]).all(), f"seq {b}: accepted tokens"
                assert toks[b, L] in set(int(x) for x in ref["final_candidates"][b]), \
                    f"seq {b}: emitted {toks[b, L]} not among {ref['final_candidates'][b]}"
                if stats is not None:
                    stats["final_flag_same"] = stats.get("final_flag_same", 0) + int(toks[b, L] == ref["out_tokens"][b, L])
            continue
        assert nacc[b] == ref["num_accepted"][b], f"seq {b}: L {nacc[b]} vs {ref['num_accepted'][b]}"
        assert (acc[b] == ref["accepted_nodes"][b]).all(), f"seq {b}: accepted {acc[b]} vs {ref['accepted_nodes'][b]}"
        assert (toks[b] == ref["out_tokens"][b]).all(), f"seq {b}: tokens {toks[b]} vs {ref['out_tokens'][b]}"
    return flagged


def flag_cap(probs, alpha=1e-6) -> int:
    """Upper bound on the number of flagged sequences: the smallest k with
    P(X > k) <= alpha for X a sum of independent Bernoulli variables with the
    given means (the oracle's per-sequence flag probabilities, `flag_prob`),
    from the exact Poisson-binomial distribution (convolution of the terms)."""
    dist = np.array([1.0])
    for p in np.asarray(probs, dtype=np.float64).ravel():
        nxt = np.zeros(dist.size + 1)
        nxt[:-1] += dist * (1.0 - p)
        nxt[1:] += dist * p
        dist = nxt
    tail = 1.0 - np.cumsum(dist)  # tail[k] = P(X > k)
    return int(np.argmax(tail <= alpha))


def oracle_reject(w, temperature=None, without_replacement=None, seed=None, offset=None):
    return oracle.tree_reject(w.target_logits, w.draft_probs, w.draft_tokens, w.parent,
                              w.temperature if temperature is None else temperature,
                              w.without_replacement if without_replacement is None else without_replacement,
                              w.seed if seed is None else seed, w.offset if offset is None else offset)
