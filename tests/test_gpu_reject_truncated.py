"""spec_tree_reject_truncated on the GPU against the oracle: the oracle's
top-k / top-p truncation of every target row (oracle/truncate.py), then the
oracle sampler (oracle/reject.py), through the C ABI.

The walk outputs must match bit for bit, with draws the oracle flags (within
1e-6 of their threshold) treated as in compare_reject.  A sequence holding a
row whose top-p decision lies within 1e-9 of a cumulative mass is skipped and
counted (both sides sum fp64 masses, in different orders).  Cases: the chain,
batched-serving, EAGLE-style and Sequoia-scale workloads; rows with ties, with
-inf entries, all equal; rows whose top values sit in one member's slice (the
second exchange, with K-lists); vocabularies smaller than K; a 300-node tree;
slices too long for LDS; the fused compaction; workspace reuse.  Some cases
redraw the draft tokens from the oracle-truncated target, so that most are
accepted and the walks go deep.
"""
import numpy as np
import pytest
import torch

import oracle
import tree_verify_attention_masked_amd as stv
from helpers import compare_reject, flag_cap, host_kv
from workloads import make_config, make_workload

pytestmark = pytest.mark.gpu

MARGIN = 1e-9


def _redraft(w, k, p, seed):
    """Draft tokens drawn from the oracle-truncated target rows (siblings
    distinct when the workload samples without replacement)."""
    trunc, _ = oracle.truncate_logits(w.target_logits, w.temperature, k, p)
    rng = np.random.default_rng(seed)
    toks = w.draft_tokens.copy()
    for b in range(w.B):
        taken = {}
        for c in range(1, w.T):
            u = int(w.parent[b, c])
            row = trunc[b, u].astype(np.float64)
            pr = oracle.softmax64(row, w.temperature)
            used = taken.setdefault(u, set())
            if w.without_replacement and used:
                pr = pr.copy()
                pr[list(used)] = 0.0
                if pr.sum() <= 0.0:
                    continue
                pr /= pr.sum()
            x = int(rng.choice(pr.size, p=pr))
            toks[b, c] = x
            used.add(x)
    return toks


def _run(w, k, p, tokens=None, workspace=None, status=None, kv=None):
    dev = "cuda"
    logits = torch.from_numpy(w.target_logits).to(dev)
    probs = torch.from_numpy(w.draft_probs).to(dev)
    toks = torch.from_numpy(w.draft_tokens if tokens is None else tokens).to(dev)
    parent = torch.from_numpy(w.parent).to(dev)
    if status is None:
        status = torch.zeros(w.B, dtype=torch.int32, device=dev)
    kw = {}
    if kv is not None:
        kw = dict(k_cache=kv[0], v_cache=kv[1], block_table=kv[2], prefix_lens=kv[3])
    acc, out, nacc, new_lens = stv.spec_tree_reject_truncated(
        logits, probs, toks, parent, w.temperature, k, p, w.without_replacement, w.seed, w.offset,
        status=status, workspace=workspace, **kw)
    torch.cuda.synchronize()
    return (acc, out, nacc), new_lens, status


def _expected(w, k, p, tokens=None):
    trunc, margins = oracle.truncate_logits(w.target_logits, w.temperature, k, p)
    ref = oracle.tree_reject(trunc, w.draft_probs, w.draft_tokens if tokens is None else tokens, w.parent,
                             w.temperature, w.without_replacement, w.seed, w.offset)
    near = (margins < MARGIN).any(axis=1)
    for b in np.flatnonzero(near):  # a truncation not decided robustly: nothing to compare
        ref["flag_path_len"][b] = 0
        ref["flag_kind"][b] = "accept"
    return ref, int(near.sum())


def _check(w, k, p, tokens=None, **kw):
    got, new_lens, status = _run(w, k, p, tokens=tokens, **kw)
    assert int(status.abs().sum()) == 0, f"device status {status.tolist()}"
    ref, near = _expected(w, k, p, tokens)
    assert near <= max(1, w.B // 20), f"{near} sequences with a truncation within {MARGIN} of a top-p mass"
    flagged = compare_reject(got, ref)
    assert flagged - near <= flag_cap(ref["flag_prob"]), f"{flagged} flagged sequences"
    return got, ref, new_lens


WORKLOADS = [
    # config, top_k, top_p, redraw the drafts from the truncated target
    (1, 50, 0.9, True),
    (1, 20, 1.0, False),
    (1, 64, 0.3, True),
    (4, 50, 0.9, True),
    (4, 64, 0.5, False),
    (2, 40, 0.95, True),
    (3, 50, 0.8, True),
    (3, 16, 1.0, False),
]


@pytest.mark.parametrize("case", WORKLOADS, ids=[f"cfg{c[0]}-k{c[1]}-p{c[2]}{'-redraft' if c[3] else ''}"
                                                  for c in WORKLOADS])
def test_workloads(case):
    cfg, k, p, redraft = case
    w = make_config(cfg, with_kv=False)
    print(f"truncated sampler: config {cfg} k={k} p={p} redraft={redraft}", flush=True)
    toks = _redraft(w, k, p, seed=cfg) if redraft else None
    got, ref, _ = _check(w, k, p, tokens=toks)
    if redraft:  # the drafts come from the truncated target: the walks must go past the root
        assert ref["num_accepted"].max() >= 2


def test_greedy_is_unchanged():
    w = make_config(2, with_kv=False, temperature=0.0)
    got, _, _ = _run(w, 30, 0.9)
    plain = stv.spec_tree_reject(torch.from_numpy(w.target_logits).cuda(), None,
                                 torch.from_numpy(w.draft_tokens).cuda(), torch.from_numpy(w.parent).cuda(),
                                 0.0, False, w.seed, w.offset)
    for g, r in zip(got, plain):
        assert torch.equal(g, r)


def _rows(kind, w, rng):
    x = w.target_logits
    if kind == "ties":  # seven distinct values: hundreds of a slice's logits at or above any threshold
        x[:] = np.round(rng.standard_normal(x.shape)).astype(np.float32)
    elif kind == "ties_narrow":  # five values: a slice of 8000 holds over a thousand at its top-k threshold
        x[:] = np.round(0.5 * rng.standard_normal(x.shape)).astype(np.float32)
    elif kind == "coarse_ties":
        x[:] = np.round(x * 2) / 2
    elif kind == "equal":
        x[:] = np.float32(0.75)
    elif kind == "minus_inf":
        x[rng.random(x.shape) < 0.6] = -np.inf
    elif kind == "clustered":  # each row's largest values in the first member's slice
        top = 6.0 + rng.random(x.shape[:-1] + (60,)).astype(np.float32)
        x[..., :60] = top
    elif kind == "clustered_far":  # ... and in the last member's slice
        x[..., -70:] = 6.0 + rng.random(x.shape[:-1] + (70,)).astype(np.float32)


SYNTH = [
    # kind, B, T, V, tau, k, p, tree
    ("ties", 2, 5, 32000, 1.0, 50, 0.9, "chain"),
    ("ties", 8, 4, 32000, 1.0, 50, 0.9, "random"),
    ("ties_narrow", 64, 4, 32000, 1.0, 50, 0.9, "random"),
    ("coarse_ties", 3, 16, 32000, 1.0, 30, 0.8, "random"),
    ("equal", 2, 5, 3000, 1.0, 10, 0.5, "chain"),
    ("equal", 1, 16, 32000, 1.0, 64, 1.0, "random"),
    ("minus_inf", 2, 5, 32000, 1.0, 64, 0.85, "chain"),
    ("minus_inf", 4, 16, 5000, 0.8, 40, 0.9, "random"),
    ("clustered", 1, 5, 32000, 1.0, 50, 0.9, "chain"),
    ("clustered", 2, 16, 32000, 1.0, 60, 1.0, "random"),
    ("clustered_far", 1, 16, 128256, 0.7, 64, 0.95, "random"),
    ("normal", 3, 7, 37, 1.0, 5, 0.7, "random"),
    ("normal", 2, 6, 50, 1.0, 64, 0.9, "random"),
    ("normal", 2, 4, 1, 1.0, 1, 0.5, "random"),
    ("normal", 1, 300, 32000, 0.6, 50, 0.9, "random"),
    ("normal", 64, 4, 40000, 1.0, 50, 0.9, "random"),   # slices of 10000 logits: read from global memory
    ("normal", 1, 5, 32000, 1.0, 1, 1.0, "chain"),      # top-1: only the argmax survives
]


@pytest.mark.parametrize("case", SYNTH, ids=[f"{c[0]}-B{c[1]}-T{c[2]}-V{c[3]}-k{c[5]}-p{c[6]}" for c in SYNTH])
def test_synthetic_rows(case):
    kind, B, T, V, tau, k, p, tree = case
    seed = SYNTH.index(case)
    if tree == "chain":
        kw = dict(tree="chain", gamma=T - 1)
    else:
        kw = dict(tree="random", T=T, max_depth=max(1, min(T - 1, 8)))
    w = make_workload(tag=900 + seed, B=B, V=V, temperature=tau, with_kv=False, **kw)
    _rows(kind, w, np.random.default_rng(seed))
    print(f"truncated sampler: {case}", flush=True)
    toks = _redraft(w, k, p, seed) if kind != "equal" else None
    _check(w, k, p, tokens=toks)


def test_fused_compaction():
    w = make_workload(tag=950, B=6, Hq=8, Hkv=2, D=128, dtype="bf16", V=32000, prefix=(100, 900), tree="random",
                      T=16, max_depth=5, shuffle_blocks=True)
    toks = _redraft(w, 50, 0.9, seed=950)
    dev = "cuda"
    k = torch.from_numpy(w.k_cache.view(np.int16)).to(dev).view(torch.bfloat16)
    v = torch.from_numpy(w.v_cache.view(np.int16)).to(dev).view(torch.bfloat16)
    bt = torch.from_numpy(w.block_table).to(dev)
    lens = torch.from_numpy(w.prefix_lens).to(dev)
    got, ref, new_lens = _check(w, 50, 0.9, tokens=toks, kv=(k, v, bt, lens))
    acc, _, nacc = (t.cpu().numpy() for t in got)
    k_ref, v_ref, lens_ref = oracle.kv_compact(w.k_cache, w.v_cache, w.block_table, w.prefix_lens, acc, nacc)
    assert np.array_equal(host_kv(w, k).view(np.uint8), k_ref.view(np.uint8))
    assert np.array_equal(host_kv(w, v).view(np.uint8), v_ref.view(np.uint8))
    assert np.array_equal(new_lens.cpu().numpy(), lens_ref)


def test_workspace_reuse_across_shapes():
    """One zero-filled workspace for three calls of different shapes (the epoch tags keep each call's lists
    apart), the plain sampler in between."""
    ws_bytes = max(stv.spec_tree_reject_truncated_workspace_size(4, 16, 32000, 64),
                   stv.spec_tree_reject_truncated_workspace_size(1, 5, 32000, 50))
    ws = torch.zeros(ws_bytes, dtype=torch.uint8, device="cuda")
    w1 = make_workload(tag=960, B=4, V=32000, tree="random", T=16, max_depth=5, with_kv=False)
    w2 = make_workload(tag=961, B=1, V=32000, tree="chain", gamma=4, with_kv=False)
    _check(w1, 64, 0.9, tokens=_redraft(w1, 64, 0.9, 960), workspace=ws)
    stv.spec_tree_reject(torch.from_numpy(w2.target_logits).cuda(), torch.from_numpy(w2.draft_probs).cuda(),
                         torch.from_numpy(w2.draft_tokens).cuda(), torch.from_numpy(w2.parent).cuda(),
                         1.0, False, 0, 0, workspace=ws)
    _check(w2, 50, 0.9, tokens=_redraft(w2, 50, 0.9, 961), workspace=ws)
    _check(w1, 10, 1.0, workspace=ws)


def test_arguments_and_device_errors():
    w = make_workload(tag=970, B=3, V=5000, tree="random", T=8, max_depth=3, with_kv=False)
    for k, p in ((0, 0.9), (65, 0.9)):
        with pytest.raises(stv.SpecError, match="UNSUPPORTED"):
            _run(w, k, p)
    for p in (0.0, float("nan")):
        with pytest.raises(stv.SpecError, match="INVALID_ARG"):
            _run(w, 10, p)
    w.target_logits[1, 0, 17] = np.nan
    got, _, status = _run(w, 10, 0.9)
    st = status.cpu().numpy()
    nonfinite = {v: k for k, v in stv.DEV_ERRORS.items()}["nonfinite"]
    assert st[0] == 0 and st[2] == 0 and st[1] & nonfinite
    acc, out, nacc = (t.cpu().numpy() for t in got)
    assert nacc[1] == 0 and (acc[1, 1:] == -1).all() and (out[1] == -1).all()
