"""spec_tree_truncate on the GPU against the oracle (oracle/truncate.py),
through the C ABI.

Per row the output must equal the oracle's bit for bit (same kept logits,
-inf elsewhere), except where the oracle's top-p decision lies within 1e-6 of
a cumulative mass (the kernel's masses carry about 1e-7 relative error): such
rows may keep one group of equal logits more or fewer, must still follow the
threshold rule, and are counted.  Then the whole verify step on a truncated
target: the sampler on the GPU-truncated logits against the oracle sampler on
the oracle-truncated logits.  Inputs: seeded synthetic rows (normal logits,
quantised logits with many ties, rows with -inf entries, a huge outlier) and
the chain and batched-serving workloads.
"""
import numpy as np
import pytest
import torch

import oracle
import tree_verify_attention_masked_amd as stv
from helpers import compare_reject
from workloads import make_config

pytestmark = pytest.mark.gpu

MARGIN = 1e-6


def _rows(kind, B, T, V, seed):
    rng = np.random.default_rng(seed)
    x = (2.5 * rng.standard_normal((B, T, V))).astype(np.float32)
    if kind == "ties":
        x = (np.round(x * 2) / 2).astype(np.float32)
    elif kind == "minus_inf":
        x[rng.random((B, T, V)) < 0.3] = -np.inf
    elif kind == "outlier":
        x[:, :, V // 3] = 1e30
        x[:, :, V // 2] = -1e30
    elif kind == "flat":
        x = (0.01 * rng.standard_normal((B, T, V))).astype(np.float32)
    elif kind == "equal":
        x[:] = 0.75
    return x


def _threshold_rule(row_in, row_out):
    """The output keeps exactly {x >= t} for t = its smallest kept logit."""
    kept = np.isfinite(row_out)
    if not kept.any():
        return np.isneginf(row_in).all()
    t = row_out[kept].min()
    return np.array_equal(kept, row_in >= t) and np.array_equal(row_out[kept], row_in[kept])


def check_rows(x, got, tau, k, p):
    ref, margins = oracle.truncate_logits(x, tau, k, p)
    flagged = 0
    for idx in np.ndindex(*x.shape[:-1]):
        if margins[idx] >= MARGIN:
            assert np.array_equal(got[idx], ref[idx]), f"row {idx}: kept set differs"
            continue
        flagged += 1
        assert _threshold_rule(x[idx], got[idx]), f"row {idx}: not a threshold rule"
        vals = np.unique(x[idx][np.isfinite(x[idx])])[::-1]
        t_ref = ref[idx][np.isfinite(ref[idx])].min()
        t_got = got[idx][np.isfinite(got[idx])].min()
        j = int(np.flatnonzero(vals == t_ref)[0])
        assert t_got in vals[max(0, j - 1):j + 2], f"row {idx}: threshold more than one group off"
    return flagged


CASES = [
    # kind, B, T, V, tau, top_k, top_p
    ("normal", 2, 5, 32000, 1.0, 50, 1.0),
    ("normal", 2, 5, 32000, 1.0, 0, 0.9),
    ("normal", 2, 5, 32000, 0.6, 100, 0.8),
    ("normal", 1, 4, 32000, 1.0, 0, 0.05),
    ("normal", 1, 3, 32768, 1.0, 7, 0.95),        # the longest row staged in LDS
    ("normal", 1, 3, 32769, 1.0, 7, 0.95),        # the shortest row read from global memory
    ("normal", 1, 3, 128256, 0.7, 20, 0.9),
    ("normal", 1, 3, 128256, 1.0, 0, 0.6),
    ("normal", 3, 7, 37, 1.0, 5, 0.7),
    ("normal", 2, 2, 1, 1.0, 1, 0.5),
    ("normal", 2, 3, 1000, 0.0, 10, 0.5),          # temperature 0: the maximum (ties) only
    ("normal", 2, 3, 1000, 0.0, 10, 1.0),
    ("ties", 2, 5, 32000, 1.0, 300, 1.0),
    ("ties", 2, 5, 32000, 1.0, 0, 0.7),
    ("ties", 1, 3, 128256, 1.0, 3000, 0.9),
    ("minus_inf", 2, 4, 32000, 1.0, 64, 0.85),
    ("minus_inf", 1, 2, 50000, 1.0, 0, 0.3),
    ("outlier", 2, 3, 32000, 1.0, 40, 1.0),
    ("outlier", 1, 3, 40000, 1.0, 2, 1.0),
    ("flat", 2, 4, 32000, 1.0, 0, 0.9),
    ("flat", 1, 3, 32000, 1.0, 1000, 0.5),
    ("equal", 1, 2, 3000, 1.0, 10, 0.5),
    ("normal", 2, 3, 32000, 1.0, 0, 1.0),          # both rules off
    ("normal", 2, 3, 32000, 1.0, 32000, 1.0),
]


@pytest.mark.parametrize("in_place", [True, False])
@pytest.mark.parametrize("case", CASES, ids=[f"{c[0]}-V{c[3]}-t{c[4]}-k{c[5]}-p{c[6]}" for c in CASES])
def test_rows_match_oracle(case, in_place):
    kind, B, T, V, tau, k, p = case
    x = _rows(kind, B, T, V, seed=CASES.index(case))
    print(f"truncate {case} in_place={in_place}", flush=True)
    xd = torch.from_numpy(x).cuda()
    status = torch.zeros(B, dtype=torch.int32, device="cuda")
    if in_place:
        out = stv.spec_tree_truncate(xd, tau, k, p, status=status)
    else:
        dst = torch.full_like(xd, 7.0)
        out = stv.spec_tree_truncate(xd, tau, k, p, out=dst, status=status)
        assert np.array_equal(xd.cpu().numpy(), x)  # the input is left alone
    got = out.cpu().numpy()
    assert int(status.abs().sum()) == 0
    flagged = check_rows(x, got, tau, k, p)
    assert flagged <= max(1, B * T // 10), f"{flagged} rows near a top-p boundary"


def test_nonfinite_row_reported_and_left_alone():
    B, T, V = 3, 2, 5000
    x = _rows("normal", B, T, V, seed=3)
    x[1, 1, 17] = np.nan
    x[2, 0, 4] = np.inf
    xd = torch.from_numpy(x).cuda()
    status = torch.zeros(B, dtype=torch.int32, device="cuda")
    stv.spec_tree_truncate(xd, 1.0, 30, 0.9, status=status)
    got = xd.cpu().numpy()
    st = status.cpu().numpy()
    nonfinite = {v: k for k, v in stv.DEV_ERRORS.items()}["nonfinite"]
    assert st[0] == 0 and st[1] == nonfinite == st[2]
    np.testing.assert_array_equal(got[1, 1], x[1, 1])
    np.testing.assert_array_equal(got[2, 0], x[2, 0])
    good = [(0, 0), (0, 1), (1, 0), (2, 1)]
    ref, _ = oracle.truncate_logits(x[[i for i, _ in good], [j for _, j in good]][:, None], 1.0, 30, 0.9)
    for n, (i, j) in enumerate(good):
        assert np.array_equal(got[i, j], ref[n, 0])


@pytest.mark.parametrize("cfg,k,p,wr", [(1, 40, 0.9, False), (4, 0, 0.8, False), (4, 50, 0.95, True),
                                        (2, 50, 0.9, False), (3, 0, 0.8, True), (3, 100, 0.95, True)])
def test_verify_step_on_truncated_target(cfg, k, p, wr):
    w = make_config(cfg, with_kv=False)
    print(f"truncate+reject config {cfg} k={k} p={p} wr={wr}", flush=True)
    logits = torch.from_numpy(w.target_logits).cuda()
    probs = torch.from_numpy(w.draft_probs).cuda()
    tokens = torch.from_numpy(w.draft_tokens).cuda()
    parent = torch.from_numpy(w.parent).cuda()
    status = torch.zeros(w.B, dtype=torch.int32, device="cuda")
    stv.spec_tree_truncate(logits, w.temperature, k, p, status=status)
    got = stv.spec_tree_reject(logits, probs, tokens, parent, w.temperature, wr, w.seed, w.offset, status=status)
    torch.cuda.synchronize()
    assert int(status.abs().sum()) == 0
    trunc, margins = oracle.truncate_logits(w.target_logits, w.temperature, k, p)
    gl = logits.cpu().numpy()
    near = margins < MARGIN
    assert near.sum() <= max(1, near.size // 20)
    for b in range(w.B):
        if near[b].any():
            continue
        assert np.array_equal(gl[b], trunc[b]), f"seq {b}: truncated logits differ"
    ref = oracle.tree_reject(trunc, w.draft_probs, w.draft_tokens, w.parent, w.temperature, wr, w.seed, w.offset)
    for b in np.flatnonzero(near.any(axis=1)):  # inputs not decided robustly: nothing to compare
        ref["flag_path_len"][b] = 0
        ref["flag_kind"][b] = "accept"
    compare_reject(got, ref)


def test_empty_batch_and_longest_row():
    empty = torch.zeros((0, 3, 100), dtype=torch.float32, device="cuda")
    assert stv.spec_tree_truncate(empty, 1.0, 5, 0.9).shape == (0, 3, 100)
    V = 1 << 24  # the longest row the call takes, read from global memory in each pass
    x = _rows("normal", 1, 1, V, seed=77)
    print(f"truncate V={V}", flush=True)
    xd = torch.from_numpy(x).cuda()
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    for k, p in ((1000, 0.9), (0, 0.5)):
        got = stv.spec_tree_truncate(xd, 1.0, k, p, out=torch.empty_like(xd), status=status).cpu().numpy()
        assert int(status.abs().sum()) == 0
        assert check_rows(x, got, 1.0, k, p) <= 1
