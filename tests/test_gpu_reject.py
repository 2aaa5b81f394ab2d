"""GPU parity of spec_tree_reject against the oracle (C ABI).

Accepted nodes, emitted tokens and L must be bit-identical to the oracle
(same Philox stream) for every sequence, except from a draw the oracle flags
as lying within 1e-6 of its decision threshold; such sequences only have to
agree on the path decided before that draw, and are counted.
"""
import numpy as np
import pytest
import torch

import tree_verify_attention_masked_amd as stv
from helpers import DevWorkload, compare_reject, flag_cap, oracle_reject
from workloads import make_config, make_workload

pytestmark = pytest.mark.gpu


def _many_offsets(w, offsets, temperature=None, wr=None):
    """GPU against oracle on every offset.  The number of sequences the oracle
    flags (a draw within 1e-6 of its threshold: those are compared only up to
    that draw) must stay below the 1e-6 upper quantile of its own distribution,
    a sum of Bernoulli variables with the oracle's per-sequence flag
    probabilities, so a flagging mistake that excuses more cannot pass."""
    d = DevWorkload(w)
    flagged = 0
    probs = []
    for off in offsets:
        got = d.reject(temperature=temperature, without_replacement=wr, offset=off)
        torch.cuda.synchronize()
        ref = oracle_reject(w, temperature=temperature, without_replacement=wr, offset=off)
        flagged += compare_reject(got, ref)
        probs.extend(ref["flag_prob"].tolist())
    assert int(d.status.abs().sum()) == 0
    cap = flag_cap(probs)
    print(f"[reject] flagged {flagged} of {len(probs)} (expected {sum(probs):.3f}, cap {cap})", flush=True)
    assert flagged <= cap
    return flagged


# at most 3 children per node, so that drafting without replacement works at V = 3
TINY_TREE = [-1, 0, 0, 0, 1, 1, 1, 2, 2, 3, 4, 4]


@pytest.mark.parametrize("V", [3, 5, 8])
@pytest.mark.parametrize("wr", [False, True])
def test_tiny_vocab_many_draws(V, wr):
    # tiny vocabularies make rejections, sibling residuals and duplicate tokens frequent
    w = make_workload(tag=500 + V, B=3, Hq=2, Hkv=2, D=64, dtype="f32", V=V, prefix=[4, 4, 4], tree="fixed",
                      parent=TINY_TREE, draft_mode="without_replacement" if wr else "iid",
                      temperature=0.8, without_replacement=wr, with_kv=True)
    print(f"[reject] tiny V={V} wr={wr}", flush=True)
    _many_offsets(w, range(60))


def test_greedy_tiny():
    w = make_workload(tag=520, B=4, Hq=2, Hkv=2, D=64, dtype="f32", V=4, prefix=[4] * 4, tree="random", T=10,
                      max_depth=4, temperature=0.0)
    _many_offsets(w, [0])


# Large vocabularies: a final draw is flagged with probability sum_x min(p(x), 2e-6)
# (about 5 % at V = 32000 with logits ~ N(0, 2^2)); flagged sequences are still
# checked up to the flagged draw (see compare_reject), and their count is capped
# by the oracle's own flag probabilities (see _many_offsets).
@pytest.mark.parametrize("cfg", [0, 1, 3])
def test_config_parity(cfg):
    w = make_config(cfg)
    print(f"[reject] config {cfg} {w.name}", flush=True)
    _many_offsets(w, range(12))


def test_config2_greedy_and_sampled():
    w = make_config(2)
    print("[reject] config 2 greedy + 0.7", flush=True)
    assert _many_offsets(w, [0], temperature=0.0) == 0
    _many_offsets(w, range(3))


def test_config4_parity():
    w = make_config(4, with_kv=False)
    print("[reject] config 4", flush=True)
    _many_offsets(w, range(2))


def test_worked_example_on_gpu():
    # the SGLang doc's prefix match: drafts "and it's so hot", target "and it's very warm"
    V = 8
    w = make_workload(tag=530, B=1, Hq=2, Hkv=2, D=64, dtype="f32", V=V, prefix=[3], tree="chain", gamma=4,
                      temperature=0.0)
    w.draft_tokens[0] = [0, 1, 2, 3, 4]
    logits = np.random.default_rng(0).standard_normal((1, 5, V)).astype(np.float32)
    for u, t in enumerate([1, 2, 5, 6, 7]):
        logits[0, u, t] = logits[0, u].max() + 1
    w.target_logits = logits
    d = DevWorkload(w)
    acc, toks, nacc = (t.cpu().numpy() for t in d.reject())
    assert nacc[0] == 2 and acc[0].tolist() == [0, 1, 2, -1, -1] and toks[0].tolist() == [1, 2, 5, -1, -1]


def test_device_errors_reported():
    w = make_workload(tag=540, B=3, Hq=2, Hkv=2, D=64, dtype="f32", V=16, prefix=[4] * 3, tree="random", T=6,
                      max_depth=3, temperature=1.0)
    d = DevWorkload(w)
    d.parent[0, 2] = 4
    d.tokens[1, 3] = 99
    d.logits[2, 0, 5] = float("nan")
    acc, toks, nacc = d.reject()
    st = d.status.cpu().numpy()
    assert st[0] & 1 and st[1] & 8 and st[2] & 16
    assert (nacc.cpu().numpy() == 0).all() and (toks.cpu().numpy() == -1).all()


def test_statistics_single_child_acceptance_rate():
    # P(accept) of one child equals sum_x min(p(x), q(x)); draws indexed by offset
    V, n = 6, 4000
    w = make_workload(tag=550, B=1, Hq=2, Hkv=2, D=64, dtype="f32", V=V, prefix=[2], tree="chain", gamma=1,
                      temperature=1.0)
    d = DevWorkload(w)
    rng = np.random.default_rng(3)
    q = w.draft_probs[0, 0].astype(np.float64)
    p = np.exp(w.target_logits[0, 0].astype(np.float64) - w.target_logits[0, 0].max())
    p /= p.sum()
    beta = np.minimum(p, q / q.sum()).sum()
    acc = 0
    toks = rng.choice(V, size=n, p=q / q.sum())
    for off in range(n):
        d.tokens[0, 1] = int(toks[off])
        _, _, nacc = d.reject(offset=off)
        acc += int(nacc.item())
    assert abs(acc / n - beta) < 4 * np.sqrt(beta * (1 - beta) / n)


# Trees of more than 256 nodes (the sampler kernel with 512-node arrays, two
# nodes per thread, a smaller eager space): a 512-node random tree at a small
# vocabulary (frequent rejections, sibling residuals), a 300-node Sequoia-profile
# tree drafted and verified without replacement, and a batch whose slices are
# too long for that eager space but fit the current-row buffer (64 sequences, 4
# members each, 8000-entry slices: no eager rows, every visited row staged).
def test_tree_of_512_nodes():
    w = make_workload(tag=560, B=2, Hq=2, Hkv=2, D=64, dtype="f32", V=50, prefix=[4, 4], tree="random", T=512,
                      max_depth=9, temperature=0.9, with_kv=False)
    print(f"[reject] T=512 depth {w.info['depth']}", flush=True)
    _many_offsets(w, range(20))


def test_tree_of_300_nodes_without_replacement():
    w = make_workload(tag=561, B=2, Hq=2, Hkv=2, D=64, dtype="f32", V=100, prefix=[4, 4], tree="sequoia", T=300,
                      max_depth=12, draft_mode="without_replacement", temperature=0.6, without_replacement=True,
                      with_kv=False)
    print(f"[reject] T=300 sequoia widths {w.info['width_profile']}", flush=True)
    _many_offsets(w, range(20))


def test_large_tree_without_eager_rows():
    w = make_workload(tag=562, B=64, Hq=2, Hkv=2, D=64, dtype="f32", V=32000, prefix=[4] * 64, tree="random",
                      T=257, max_depth=4, temperature=1.0, with_kv=False)
    assert stv.spec_tree_reject_plan(64, 257, 32000, 1 << 20) == (4, 8000)
    print("[reject] B=64 T=257 V=32000", flush=True)
    _many_offsets(w, range(2))


# Eager row counts other than 1, 2, 4 and 8 (the rows whose statistics are taken
# before the walk): a tree of more than 256 nodes keeps min(8, 7680 / slice
# stride) of them, so 300-node trees over one sequence (32 members) at V = 70000,
# 38400 and 32000 keep 3, 6 and 7.
EAGER = [
    ("e3_t300", dict(B=1, V=70000, prefix=[4], tree="random", T=300, max_depth=8, temperature=0.9), 6),
    ("e6_t300", dict(B=1, V=38400, prefix=[4], tree="random", T=300, max_depth=8, temperature=1.0), 6),
    ("e7_sequoia_t300", dict(B=1, V=32000, prefix=[4], tree="sequoia", T=300, max_depth=10, temperature=0.6,
                             draft_mode="without_replacement", without_replacement=True), 6),
]


@pytest.mark.parametrize("name,kw,n_off", EAGER, ids=[e[0] for e in EAGER])
def test_eager_row_counts(name, kw, n_off):
    w = make_workload(tag=570 + [e[0] for e in EAGER].index(name), Hq=2, Hkv=2, D=64, dtype="f32", with_kv=False,
                      **kw)
    print(f"[reject] {name} B={w.B} T={w.T} V={w.V}", flush=True)
    _many_offsets(w, range(n_off))
