"""Repeated calls sharing one workspace (the way a serving loop or a captured
graph calls the library): the workspace is zero-filled once.  Attention must
leave its split-arrival counters back at zero (a counter left behind would stop
the next call's merge, so its output would never be written; the output is
poisoned with NaN before each call so that a skipped write cannot pass on stale
data).  The sampler's exchange slots carry a per-call tag taken from the
epoch in the workspace header: slots written by earlier calls must never be
taken for this call's, including across the epoch's wrap-around."""
import numpy as np
import pytest
import torch

import tree_verify_attention_masked_amd as stv
from helpers import DevWorkload, assert_attn_close, attn_to_f64, compare_reject, oracle_attn, oracle_reject
from workloads import make_config, make_workload

pytestmark = pytest.mark.gpu

ATTN_CASES = [
    # streaming kernel with several splits per (b, g)
    ("stream_splits", dict(B=2, Hq=4, Hkv=4, prefix=[3000, 700], tree="chain", gamma=4)),
    # 64-row tiles, ragged batch: sequences with 1 .. many splits
    ("tile64_ragged", dict(B=3, Hq=8, Hkv=2, prefix=[3, 9000, 700], tree="random", T=16, max_depth=5,
                           shuffle_blocks=True)),
    # 128-row tiles, several row tiles and splits
    ("tile128_splits", dict(B=1, Hq=16, Hkv=2, prefix=[5000], tree="random", T=24, max_depth=6)),
]


@pytest.mark.parametrize("name,kw", ATTN_CASES, ids=[c[0] for c in ATTN_CASES])
def test_attention_reuses_one_workspace(name, kw):
    w = make_workload(name=name, tag=600 + [c[0] for c in ATTN_CASES].index(name), V=8, D=128, dtype="bf16", **kw)
    print(f"[reuse] {name} B={w.B} T={w.T} Hq={w.Hq} Hkv={w.Hkv} lens={w.prefix_lens.tolist()}", flush=True)
    d = DevWorkload(w)
    ws_bytes = stv.spec_tree_attn_workspace_size(w.B, w.T, w.Hq, w.Hkv, w.D, w.block_table.shape[1], stv.SPEC_BF16)
    assert ws_bytes > 0, "these shapes use split partials"
    ws = torch.zeros(ws_bytes, dtype=torch.uint8, device="cuda")
    ref, ref_abs = oracle_attn(w)
    first = None
    for call in range(3):
        out = torch.full_like(d.q, float("nan"))
        stv.spec_tree_attn(d.q, d.k, d.v, d.block_table, d.prefix_lens, d.parent, scale=w.scale, out=out,
                           status=d.status, workspace=ws)
        torch.cuda.synchronize()
        got = attn_to_f64(w, out)
        assert_attn_close(got, ref, w.dtype, f"{name} call {call}", ref_abs)
        if first is None:
            first = got
        else:
            assert np.array_equal(got, first), f"{name}: call {call} differs from call 0"
    assert int(d.status.abs().sum()) == 0


@pytest.mark.parametrize("cfg", [1, 4])
def test_sampler_reuses_one_workspace(cfg):
    w = make_config(cfg, with_kv=False)
    print(f"[reuse] sampler config {cfg} {w.name}", flush=True)
    d = DevWorkload(w)
    lib = stv.load_library()
    ws = torch.zeros(int(lib.spec_tree_reject_workspace_size(w.B, w.T, w.V)), dtype=torch.uint8, device="cuda")
    for offset in (0, 1, 2):
        acc = torch.full((w.B, w.T), -7, dtype=torch.int32, device="cuda")
        toks = torch.full((w.B, w.T), -7, dtype=torch.int32, device="cuda")
        nacc = torch.full((w.B,), -7, dtype=torch.int32, device="cuda")
        stv.spec_tree_reject(d.logits, d.probs, d.tokens, d.parent, w.temperature, w.without_replacement, w.seed,
                             offset, accepted_nodes=acc, out_tokens=toks, num_accepted=nacc, status=d.status,
                             workspace=ws)
        torch.cuda.synchronize()
        assert int(d.status.abs().sum()) == 0
        ref = oracle_reject(w, offset=offset)
        compare_reject((acc, toks, nacc), ref)


HEADER_WORDS = 64  # int32 words of the sampler's workspace header: [0] exit counter of the grid, [1] epoch


@pytest.mark.parametrize("cfg", [1, 0])
def test_sampler_epoch_wraps(cfg):
    """Start the epoch three calls before it wraps (white-box: the header words of
    the workspace) and check every call against the oracle: the call whose next
    tag would be 0 restarts the epoch at 0 after clearing every slot, so the
    stale slots of the first two calls (tags 2^32 - 2 and 2^32 - 1) and of all
    earlier calls cannot pass for the later calls' (tags 1, 2)."""
    w = make_config(cfg, with_kv=False)
    print(f"[reuse] epoch wrap, sampler config {cfg} {w.name}", flush=True)
    d = DevWorkload(w)
    lib = stv.load_library()
    ws = torch.zeros(int(lib.spec_tree_reject_workspace_size(w.B, w.T, w.V)), dtype=torch.uint8, device="cuda")
    words = ws[: HEADER_WORDS * 4].view(torch.int32)
    # slots of an earlier cycle: run once from a fresh epoch on other logits, so
    # every slot that walk used holds tag 1 and records that differ from the later
    # calls' (a slot taken for the wrong call changes their decisions), then move
    # the epoch to 2^32 - 3
    stv.spec_tree_reject(d.logits * 0.5, d.probs, d.tokens, d.parent, w.temperature, w.without_replacement, w.seed,
                         0, status=d.status, workspace=ws)
    torch.cuda.synchronize()
    assert int(words[1]) == 1
    words[1] = -3  # 0xFFFFFFFD
    for call, offset in enumerate((5, 6, 7, 8)):
        acc = torch.full((w.B, w.T), -7, dtype=torch.int32, device="cuda")
        toks = torch.full((w.B, w.T), -7, dtype=torch.int32, device="cuda")
        nacc = torch.full((w.B,), -7, dtype=torch.int32, device="cuda")
        stv.spec_tree_reject(d.logits, d.probs, d.tokens, d.parent, w.temperature, w.without_replacement, w.seed,
                             offset, accepted_nodes=acc, out_tokens=toks, num_accepted=nacc, status=d.status,
                             workspace=ws)
        torch.cuda.synchronize()
        assert int(d.status.abs().sum()) == 0, f"call {call}: device status {d.status.tolist()}"
        compare_reject((acc, toks, nacc), oracle_reject(w, offset=offset))
        expect = [-2, 0, 1, 2][call]  # 0xFFFFFFFE, then the wrap to 0, then 1, 2
        assert int(words[1]) == expect, f"call {call}: epoch {int(words[1])}"
        assert int(words[0]) == 0, "the exit counter must be back at zero"
