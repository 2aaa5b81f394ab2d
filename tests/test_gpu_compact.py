"""GPU parity of spec_kv_compact: the whole cache after compaction must be
bit-identical to the oracle's, for every accepted path of the tiny tree, for
random paths on larger trees, for chains (no-op) and at full configuration
size; plus one verify step end to end (attention -> rejection -> compaction)."""
import numpy as np
import pytest
import torch

import oracle
import tree_verify_attention_masked_amd as stv
from helpers import DevWorkload, compare_reject, host_kv, oracle_reject
from workloads import make_config, make_workload

pytestmark = pytest.mark.gpu


def _paths_for(w, rng):
    acc = np.full((w.B, w.T), -1, dtype=np.int32)
    nacc = np.zeros(w.B, dtype=np.int32)
    for b in range(w.B):
        tree = oracle.tree_structure(w.parent[b])
        path = tree.anc[int(rng.integers(w.T))]
        acc[b, :len(path)] = path
        nacc[b] = len(path) - 1
    return acc, nacc


def _check(w, acc, nacc):
    d = DevWorkload(w)
    new_lens = d.compact(torch.from_numpy(acc).cuda(), torch.from_numpy(nacc).cuda())
    torch.cuda.synchronize()
    k_ref, v_ref, lens_ref = oracle.kv_compact(w.k_cache, w.v_cache, w.block_table, w.prefix_lens, acc, nacc)
    assert np.array_equal(host_kv(w, d.k).view(np.uint8), k_ref.view(np.uint8))
    assert np.array_equal(host_kv(w, d.v).view(np.uint8), v_ref.view(np.uint8))
    assert np.array_equal(new_lens.cpu().numpy(), lens_ref)
    assert int(d.status.abs().sum()) == 0


def test_every_path_of_the_tiny_tree():
    w = make_config(0)
    tree = oracle.tree_structure(w.parent[0])
    for end in range(w.T):
        path = tree.anc[end]
        acc = np.full((1, w.T), -1, dtype=np.int32)
        acc[0, :len(path)] = path
        _check(w, acc, np.array([len(path) - 1], dtype=np.int32))


@pytest.mark.parametrize("dtype,D", [("bf16", 128), ("f32", 64), ("f32", 128)])
def test_random_paths(dtype, D):
    w = make_workload(tag=600 + D, B=5, Hq=4, Hkv=2, D=D, dtype=dtype, V=8, prefix=[0, 15, 16, 100, 513],
                      tree="random", T=90, max_depth=80, shuffle_blocks=True)
    _check(w, *_paths_for(w, np.random.default_rng(D)))


def test_long_path_crosses_staging_chunks():
    w = make_workload(tag=610, B=1, Hq=2, Hkv=2, D=128, dtype="f32", V=8, prefix=[7], tree="fixed",
                      parent=[-1] + [0] * 3 + list(range(3, 3 + 150)))
    acc = np.full((1, w.T), -1, dtype=np.int32)
    path = oracle.tree_structure(w.parent[0]).anc[w.T - 1]
    acc[0, :len(path)] = path
    _check(w, acc, np.array([len(path) - 1], dtype=np.int32))


def test_chain_is_a_no_op():
    w = make_config(1)
    acc = np.array([[0, 1, 2, -1, -1]], dtype=np.int32)
    _check(w, acc, np.array([2], dtype=np.int32))


@pytest.mark.parametrize("cfg", [3, 4])
def test_config_size(cfg):
    w = make_config(cfg)
    print(f"[compact] config {cfg}", flush=True)
    _check(w, *_paths_for(w, np.random.default_rng(cfg)))


def test_bad_path_leaves_cache_untouched():
    w = make_workload(tag=620, B=2, Hq=2, Hkv=2, D=128, dtype="bf16", V=8, prefix=[3, 9], tree="random", T=8,
                      max_depth=3)
    d = DevWorkload(w)
    acc = torch.tensor([[0, 3, 2, -1, -1, -1, -1, -1], [1, 2, -1, -1, -1, -1, -1, -1]], dtype=torch.int32).cuda()
    new_lens = d.compact(acc, torch.tensor([2, 1], dtype=torch.int32).cuda())
    assert np.array_equal(host_kv(w, d.k).view(np.uint8), w.k_cache.view(np.uint8))
    assert (d.status.cpu().numpy() & 64).all()
    assert new_lens.cpu().tolist() == w.prefix_lens.tolist()


@pytest.mark.parametrize("cfg", [0, 1, 3])
def test_verify_step_end_to_end(cfg):
    """attention -> rejection -> compaction on the same device state, each checked."""
    w = make_config(cfg)
    d = DevWorkload(w)
    out = d.attn()
    acc, toks, nacc = d.reject()
    new_lens = d.compact(acc, nacc)
    torch.cuda.synchronize()
    from helpers import assert_attn_close, attn_to_f64, oracle_attn
    ref_out, ref_abs = oracle_attn(w)
    assert_attn_close(attn_to_f64(w, out), ref_out, w.dtype, "step attention", ref_abs)
    ref = oracle_reject(w)
    assert compare_reject((acc, toks, nacc), ref) == 0
    k_ref, v_ref, lens_ref = oracle.kv_compact(w.k_cache, w.v_cache, w.block_table, w.prefix_lens,
                                               ref["accepted_nodes"], ref["num_accepted"])
    assert np.array_equal(host_kv(w, d.k).view(np.uint8), k_ref.view(np.uint8))
    assert np.array_equal(new_lens.cpu().numpy(), lens_ref)
    assert int(d.status.abs().sum()) == 0


def _bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


@pytest.mark.parametrize("cfg", [0, 1, 2, 3, 4])
def test_fused_reject_compact_equals_separate_calls(cfg):
    """spec_tree_reject_compact == spec_tree_reject, then spec_kv_compact on its path:
    same path, tokens and lengths, and the whole K and V caches bit-equal."""
    w = make_config(cfg)
    print(f"[fused] config {cfg} {w.name}", flush=True)
    sep, fus = DevWorkload(w), DevWorkload(w)  # two independent copies of the caches
    acc1, toks1, n1 = sep.reject()
    lens1 = sep.compact(acc1, n1)
    acc2, toks2, n2, lens2 = stv.spec_tree_reject_compact(
        fus.logits, fus.probs, fus.tokens, fus.parent, w.temperature, fus.k, fus.v, fus.block_table,
        fus.prefix_lens, w.without_replacement, w.seed, w.offset, status=fus.status)
    torch.cuda.synchronize()
    for x, y, what in ((acc1, acc2, "accepted_nodes"), (toks1, toks2, "out_tokens"), (n1, n2, "num_accepted"),
                       (lens1, lens2, "new_lens"), (sep.status, fus.status, "status")):
        assert torch.equal(x, y), what
    assert torch.equal(_bits(sep.k), _bits(fus.k)) and torch.equal(_bits(sep.v), _bits(fus.v))
    moved = int((acc1[:, 1:] != torch.arange(1, w.T, device=acc1.device)).logical_and(acc1[:, 1:] >= 0).sum())
    print(f"[fused] config {cfg}: accepted {n1.tolist()[:8]}, rows off their place {moved}", flush=True)


def _caterpillar(n_spine):
    """Spine nodes 0, 2, 4, ...: node 2k has the leaf 2k + 1, then the next spine node 2k + 2."""
    parent = [-1]
    for k in range(n_spine - 1):
        parent += [2 * k, 2 * k]
    return parent


def test_random_paths_of_a_512_node_tree():
    w = make_workload(tag=630, B=3, Hq=4, Hkv=2, D=128, dtype="bf16", V=8, prefix=[0, 40, 1000], tree="random",
                      T=512, max_depth=12, shuffle_blocks=True)
    _check(w, *_paths_for(w, np.random.default_rng(6)))


def test_deep_path_of_a_511_node_tree():
    """Greedy verification of a caterpillar whose spine tokens are the target's argmax:
    the path is the 256-node spine, so 255 rows move; the fused call, the separate
    calls and the oracle agree on the path and on the whole cache."""
    parent = _caterpillar(256)
    w = make_workload(tag=631, B=2, Hq=2, Hkv=2, D=128, dtype="bf16", V=16, prefix=[3, 77], tree="fixed",
                      parent=parent, temperature=0.0)
    T = len(parent)
    for b in range(w.B):
        for k in range(255):
            top = int(np.argmax(w.target_logits[b, 2 * k]))
            w.draft_tokens[b, 2 * k + 1] = (top + 1) % w.V  # the leaf, tried first, is rejected
            w.draft_tokens[b, 2 * k + 2] = top
    ref = oracle_reject(w)
    assert ref["num_accepted"].tolist() == [255, 255]
    k_ref, v_ref, lens_ref = oracle.kv_compact(w.k_cache, w.v_cache, w.block_table, w.prefix_lens,
                                               ref["accepted_nodes"], ref["num_accepted"])
    sep, fus = DevWorkload(w), DevWorkload(w)
    acc1, toks1, n1 = sep.reject()
    lens1 = sep.compact(acc1, n1)
    acc2, toks2, n2, lens2 = stv.spec_tree_reject_compact(
        fus.logits, fus.probs, fus.tokens, fus.parent, w.temperature, fus.k, fus.v, fus.block_table,
        fus.prefix_lens, w.without_replacement, w.seed, w.offset, status=fus.status)
    torch.cuda.synchronize()
    assert compare_reject((acc1, toks1, n1), ref) == 0
    for x, y, what in ((acc1, acc2, "accepted_nodes"), (toks1, toks2, "out_tokens"), (n1, n2, "num_accepted"),
                       (lens1, lens2, "new_lens")):
        assert torch.equal(x, y), what
    for d in (sep, fus):
        assert np.array_equal(host_kv(w, d.k).view(np.uint8), k_ref.view(np.uint8))
        assert np.array_equal(host_kv(w, d.v).view(np.uint8), v_ref.view(np.uint8))
        assert int(d.status.abs().sum()) == 0
    assert np.array_equal(lens1.cpu().numpy(), lens_ref) and T == 511
