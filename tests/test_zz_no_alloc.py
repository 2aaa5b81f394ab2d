"""The allocation-free entry point (spec_tree_reject_compact_noalloc, the
sampler's workspace in a static device array of the library) against the
entry point it varies (spec_tree_reject_compact with a caller's workspace),
through the C ABI: accepted paths, emitted tokens, lengths, new lengths and the
whole compacted KV cache bit for bit (the same Philox stream, so the same
walk), on consecutive calls of different shapes -- the second smaller than the
first, then the first again -- plus a shape whose workspace exceeds the array,
which must be refused before anything is launched."""
import numpy as np
import pytest
import torch

import tree_verify_attention_masked_amd as stv
from helpers import DevWorkload, compare_reject, oracle_reject
from workloads import make_workload

pytestmark = pytest.mark.gpu

SHAPES = [
    # (tag, B, T, Hkv, Hq, V, prefix range, tree, depth, tau, without replacement)
    (700, 16, 16, 8, 32, 32000, (512, 2048), "random", 5, 1.0, False),
    (701, 3, 8, 2, 8, 5000, (20, 300), "random", 3, 0.7, True),
    (702, 16, 16, 8, 32, 32000, (512, 2048), "random", 5, 0.0, False),
]


def _workload(tag, B, T, Hkv, Hq, V, prefix, tree, depth, tau, wr):
    return make_workload(tag=tag, B=B, Hq=Hq, Hkv=Hkv, D=128, dtype="bf16", V=V, prefix=prefix, tree=tree, T=T,
                         max_depth=depth, temperature=tau, without_replacement=wr,
                         draft_mode="without_replacement" if wr else "iid", shuffle_blocks=True)


def _outputs(B, T, dev="cuda"):
    z = lambda *s: torch.full(s, -7, dtype=torch.int32, device=dev)  # poisoned: every entry must be written
    return z(B, T), z(B, T), z(B), z(B)


def test_noalloc_matches_the_workspace_entry_point():
    for call, shape in enumerate(SHAPES):
        w = _workload(*shape)
        print(f"[noalloc] call {call}: B={w.B} T={w.T} V={w.V} tau={w.temperature} wr={w.without_replacement}",
              flush=True)
        a, b = DevWorkload(w), DevWorkload(w)  # two copies of the caches: each entry point compacts its own
        ref = stv.spec_tree_reject_compact(a.logits, a.probs, a.tokens, a.parent, w.temperature, a.k, a.v,
                                           a.block_table, a.prefix_lens, w.without_replacement, w.seed, call,
                                           status=a.status)
        got = stv.spec_tree_reject_compact_noalloc(b.logits, b.probs, b.tokens, b.parent, w.temperature, b.k, b.v,
                                                   b.block_table, b.prefix_lens, *_outputs(w.B, w.T),
                                                   without_replacement=w.without_replacement, seed=w.seed,
                                                   offset=call, status=b.status)
        torch.cuda.synchronize()
        assert int(a.status.abs().sum()) == 0 and int(b.status.abs().sum()) == 0
        for x, y, name in zip(ref, got, ("accepted_nodes", "out_tokens", "num_accepted", "new_lens")):
            assert torch.equal(x, y), f"call {call}: {name} differs"
        assert torch.equal(a.k.view(torch.int16), b.k.view(torch.int16)), f"call {call}: K cache differs"
        assert torch.equal(a.v.view(torch.int16), b.v.view(torch.int16)), f"call {call}: V cache differs"
        # and both against the oracle's walk (flagged draws excepted, as in the other sampler tests)
        compare_reject(got[:3], oracle_reject(w, offset=call))


def test_noalloc_refuses_a_workspace_larger_than_its_array():
    B, T, V = 1000, 256, 16  # one member per sequence: 1000 x (8 + 2T + 2) slots of 32 bytes, past 8 MiB
    assert stv.load_library().spec_tree_reject_workspace_size(B, T, V) > (8 << 20)
    dev = "cuda"
    logits = torch.zeros((B, T, V), dtype=torch.float32, device=dev)
    tok = torch.zeros((B, T), dtype=torch.int32, device=dev)
    parent = torch.arange(-1, T - 1, dtype=torch.int32, device=dev).repeat(B, 1)
    k = torch.zeros((20, 1, 16, 128), dtype=torch.bfloat16, device=dev)
    bt = torch.zeros((B, 20), dtype=torch.int32, device=dev)
    lens = torch.zeros((B,), dtype=torch.int32, device=dev)
    outs = _outputs(B, T)
    with pytest.raises(stv.SpecError) as e:
        stv.spec_tree_reject_compact_noalloc(logits, logits, tok, parent, 1.0, k, k, bt, lens, *outs)
    assert e.value.code == stv.binding.SPEC_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert (outs[2] == -7).all(), "nothing may have been launched"
