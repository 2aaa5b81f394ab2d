"""GPU parity of the sampler's team shapes against the oracle (C ABI).

* slices too long for LDS (more than 8192 logits per team member): the
  members read their slices from global memory; sampling with and without
  replacement and greedy, at B = 64, V = 40000 and B = 16, V = 140000;
* one member per sequence (a batch larger than the device holds teams for),
  with slices in LDS and in global memory;
* the team plan the library launches fits the device's resident grid;
* one workspace, zero-filled once, reused across batch sizes and tree sizes.
Every call is compared with the oracle as in test_gpu_reject.py.
"""
import numpy as np
import pytest
import torch

import tree_verify_attention_masked_amd as stv
from helpers import DevWorkload, compare_reject, flag_cap, oracle_reject
from workloads import make_workload

pytestmark = pytest.mark.gpu


def _check(w, offsets, temperature=None, wr=None, workspace=None, d=None):
    d = d or DevWorkload(w)
    flagged, probs = 0, []
    for off in offsets:
        got = stv.spec_tree_reject(d.logits, d.probs, d.tokens, d.parent,
                                   w.temperature if temperature is None else temperature,
                                   w.without_replacement if wr is None else wr, w.seed, off, status=d.status,
                                   workspace=workspace)
        torch.cuda.synchronize()
        ref = oracle_reject(w, temperature=temperature, without_replacement=wr, offset=off)
        flagged += compare_reject(got, ref)
        probs.extend(ref["flag_prob"].tolist())
    assert int(d.status.abs().sum()) == 0, d.status.tolist()
    assert flagged <= flag_cap(probs)
    return flagged


def test_resident_capacity_and_plan():
    cap = stv.spec_tree_reject_max_resident()
    print(f"[teams] resident sampler workgroups: {cap}", flush=True)
    assert cap >= 256  # one workgroup per CU on a 256-CU MI355X
    for B, T, V in ((1, 5, 32000), (64, 16, 32000), (1, 256, 32000), (8, 64, 128256), (300, 4, 1000)):
        team, _ = stv.spec_tree_reject_plan(B, T, V, cap)
        assert team == 1 or B * team <= cap


@pytest.mark.parametrize("B,V,T,depth", [(64, 40000, 16, 5), (16, 140000, 12, 4)])
@pytest.mark.parametrize("mode", ["iid", "without_replacement", "greedy"])
def test_global_memory_slices(B, V, T, depth, mode):
    cap = stv.spec_tree_reject_max_resident()
    team, sl = stv.spec_tree_reject_plan(B, T, V, cap)
    assert sl > 8192, "these shapes must take the global-memory slice path"
    wr = mode == "without_replacement"
    tau = 0.0 if mode == "greedy" else 0.9
    w = make_workload(tag=600 + B, B=B, Hq=2, Hkv=2, D=64, dtype="f32", V=V, prefix=[4] * B, tree="random", T=T,
                      max_depth=depth, draft_mode="without_replacement" if wr else "iid", temperature=tau,
                      without_replacement=wr, with_kv=False)
    print(f"[teams] global slices B={B} V={V} team={team} slice={sl} mode={mode}", flush=True)
    _check(w, range(2))


@pytest.mark.parametrize("V", [1000, 32000])
def test_one_member_per_sequence(V):
    B = 300  # more sequences than 256 / 2: every team has one member
    cap = stv.spec_tree_reject_max_resident()
    team, sl = stv.spec_tree_reject_plan(B, 6, V, cap)
    assert team == 1 and sl == V
    w = make_workload(tag=610, B=B, Hq=2, Hkv=2, D=64, dtype="f32", V=V, prefix=[4] * B, tree="random", T=6,
                      max_depth=3, temperature=1.0, with_kv=False)
    print(f"[teams] one member per sequence B={B} V={V}", flush=True)
    _check(w, range(2))
    _check(w, [0], temperature=0.0)


def test_workspace_reused_across_shapes():
    # one workspace, zero-filled once, for batches of 4, 8, then 4 sequences and
    # two tree sizes: the slots the larger batch wrote sit where the smaller
    # batch's slots of other sequences lie, and must never pass for them
    lib = stv.load_library()
    ws = torch.zeros(int(lib.spec_tree_reject_workspace_size(8, 14, 5000)), dtype=torch.uint8, device="cuda")
    for i, (B, T) in enumerate([(4, 10), (8, 10), (4, 10), (8, 14), (4, 10)]):
        w = make_workload(tag=620 + B + T, B=B, Hq=2, Hkv=2, D=64, dtype="f32", V=5000, prefix=[4] * B,
                          tree="random", T=T, max_depth=4, temperature=1.0, with_kv=False)
        need = int(lib.spec_tree_reject_workspace_size(B, T, 5000))
        print(f"[teams] workspace reuse call {i}: B={B} T={T}", flush=True)
        _check(w, range(3), workspace=ws[:need])  # three calls of each shape, never zero-filled again
