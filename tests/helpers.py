"""Shared test helpers: move a synthetic workload to the GPU, call the library,
compare with the oracle under the stated tolerances."""
from __future__ import annotations

import numpy as np
import torch

import oracle
import tree_verify_attention_masked_amd as stv

BF16_ATOL, BF16_RTOL = 2e-2, 1e-2  # bf16 attention outputs vs the fp64 oracle
F32_ATOL, F32_RTOL = 1e-5, 1e-5  # fp32 attention outputs vs the fp64 oracle


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


def assert_attn_close(got, ref, dtype, what=""):
    got = np.asarray(got, dtype=np.float64)
    atol, rtol = (BF16_ATOL, BF16_RTOL) if dtype == "bf16" else (F32_ATOL, F32_RTOL)
    err = np.abs(got - ref)
    bad = err > atol + rtol * np.abs(ref)
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


def oracle_reject(w, temperature=None, without_replacement=None, seed=None, offset=None):
    return oracle.tree_reject(w.target_logits, w.draft_probs, w.draft_tokens, w.parent,
                              w.temperature if temperature is None else temperature,
                              w.without_replacement if without_replacement is None else without_replacement,
                              w.seed if seed is None else seed, w.offset if offset is None else offset)
