"""spec_tree_kv_write on the GPU against the oracle (oracle/rope.py), through
the C ABI: every tree node's V row lands bit for bit at logical slot
prefix + node, its K row and the queries rotated for position prefix + depth
within the rounding of the storage type, and every other cache slot is left as
it was.  Inputs: the synthetic workloads' caches, trees and block tables, with
new K/V rows drawn here (seeded)."""
import numpy as np
import pytest
import torch

import oracle
import tree_verify_attention_masked_amd as stv
from helpers import DevWorkload, dev_kv, host_kv
from workloads import make_workload
from workloads.gen import f32_to_bf16_bits

pytestmark = pytest.mark.gpu

# |gpu - oracle| for a rotated element: the GPU rotates in fp64 and rounds once
# to the storage type (fp32: 2^-24 relative; bf16: fp32 then bf16, within one
# bf16 unit, 2^-8 relative), plus a floor for results that cancel to near zero.
TOL = {"f32": (2.0 ** -23, 1e-12), "bf16": (2.0 ** -8, 1e-12)}


def _widen(w, a):
    if w.dtype == "bf16":
        return (np.ascontiguousarray(a, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return np.asarray(a, dtype=np.float64)


def _rows(w, seed, shape):
    x = np.random.default_rng(seed).normal(size=shape).astype(np.float32)
    return f32_to_bf16_bits(x) if w.dtype == "bf16" else x


def _close(got, ref, dtype, what):
    rtol, atol = TOL[dtype]
    err = np.abs(got - ref)
    bad = err > rtol * np.abs(ref) + atol
    assert not bad.any(), f"{what}: {int(bad.sum())} elements off, max err {err.max():.3e}"


def _run(w, theta, with_q=True, seed=0):
    print(f"[kv_write] {w.name} B={w.B} T={w.T} Hq={w.Hq} Hkv={w.Hkv} D={w.D} {w.dtype} theta={theta} "
          f"lens={w.prefix_lens.tolist()[:4]}", flush=True)
    d = DevWorkload(w)
    k_new = _rows(w, seed + 1, (w.B, w.T, w.Hkv, w.D))
    v_new = _rows(w, seed + 2, (w.B, w.T, w.Hkv, w.D))
    q = dev_kv(w, w.q) if with_q else None
    stv.spec_tree_kv_write(dev_kv(w, k_new), dev_kv(w, v_new), q, d.k, d.v, d.block_table, d.prefix_lens, d.parent,
                           theta, status=d.status)
    torch.cuda.synchronize()
    assert int(d.status.abs().sum()) == 0, d.status.tolist()
    q_ref, k_ref, v_ref = oracle.tree_kv_write(k_new, v_new, w.q if with_q else None, w.k_cache, w.v_cache,
                                               w.block_table, w.prefix_lens, w.parent, theta, dtype=w.dtype)
    k_got, v_got = host_kv(w, d.k), host_kv(w, d.v)
    written = np.zeros(k_got.shape[0] * 16, dtype=bool).reshape(k_got.shape[0], 16)
    for b in range(w.B):
        for i in range(w.T):
            t = int(w.prefix_lens[b]) + i
            blk, off = int(w.block_table[b][t // 16]), t % 16
            written[blk, off] = True
            assert np.array_equal(v_got[blk, :, off], v_new[b, i]), f"V row of node {i}, sequence {b}"
            _close(_widen(w, k_got[blk, :, off]), k_ref[blk, :, off], w.dtype, f"K row of node {i}, sequence {b}")
    untouched = ~written
    for name, got, before in (("K", k_got, w.k_cache), ("V", v_got, w.v_cache)):
        g = got.transpose(0, 2, 1, 3)[untouched]
        o = np.asarray(before).transpose(0, 2, 1, 3)[untouched]
        assert np.array_equal(g.view(np.uint8), o.view(np.uint8)), f"{name}: a slot outside the tree changed"
    if with_q:
        _close(_widen(w, host_kv(w, q)), q_ref, w.dtype, "queries")


CASES = [
    ("f32_d64_fixed_tree", dict(B=1, Hq=2, Hkv=2, D=64, dtype="f32", prefix=128, tree="fixed",
                                parent=[-1, 0, 0, 1, 1, 2, 3, 4]), 10000.0),
    ("f32_d128_gqa_random", dict(B=3, Hq=8, Hkv=2, D=128, dtype="f32", prefix=[0, 77, 1500], tree="random", T=20,
                                 max_depth=6, shuffle_blocks=True), 10000.0),
    ("bf16_chain", dict(B=1, Hq=40, Hkv=40, D=128, dtype="bf16", prefix=2048, tree="chain", gamma=4), 10000.0),
    ("bf16_gqa_random_long_prefix", dict(B=4, Hq=32, Hkv=8, D=128, dtype="bf16", prefix=[5, 900, 16000, 333],
                                         tree="random", T=16, max_depth=5, shuffle_blocks=True), 500000.0),
    ("bf16_deep_chain_t256", dict(B=1, Hq=2, Hkv=1, D=128, dtype="bf16", prefix=[37], tree="chain", gamma=255),
     10000.0),
    ("bf16_unrotated", dict(B=2, Hq=4, Hkv=2, D=128, dtype="bf16", prefix=[16, 31], tree="random", T=9,
                            max_depth=3), 0.0),
    # more than 256 nodes: two nodes per thread in the depth doubling
    ("bf16_tree_t512", dict(B=2, Hq=4, Hkv=2, D=128, dtype="bf16", prefix=[5, 300], tree="random", T=512,
                            max_depth=9, shuffle_blocks=True), 10000.0),
    ("f32_deep_chain_t300", dict(B=1, Hq=2, Hkv=1, D=64, dtype="f32", prefix=[21], tree="chain", gamma=299),
     10000.0),
]


@pytest.mark.parametrize("name,kw,theta", CASES, ids=[c[0] for c in CASES])
def test_kv_write_matches_oracle(name, kw, theta):
    w = make_workload(name=name, tag=700 + [c[0] for c in CASES].index(name), V=8, **kw)
    _run(w, theta)


def test_kv_write_without_queries():
    w = make_workload(name="no_q", tag=720, V=8, B=2, Hq=4, Hkv=2, D=128, dtype="bf16", prefix=[40, 3],
                      tree="random", T=7, max_depth=3)
    _run(w, 10000.0, with_q=False)


def test_kv_write_bad_inputs_leave_the_sequence_unwritten():
    w = make_workload(name="bad", tag=721, V=8, B=3, Hq=2, Hkv=1, D=128, dtype="bf16", prefix=[10, 20, 30],
                      tree="random", T=6, max_depth=3)
    d = DevWorkload(w)
    parent = w.parent.copy()
    parent[1, 3] = 5  # not topological
    lens = w.prefix_lens.copy()
    lens[2] = -4
    k_new = dev_kv(w, _rows(w, 9, (w.B, w.T, w.Hkv, w.D)))
    v_new = dev_kv(w, _rows(w, 10, (w.B, w.T, w.Hkv, w.D)))
    k_before, v_before = host_kv(w, d.k).copy(), host_kv(w, d.v).copy()
    stv.spec_tree_kv_write(k_new, v_new, None, d.k, d.v, d.block_table, torch.from_numpy(lens).cuda(),
                           torch.from_numpy(parent).cuda(), 10000.0, status=d.status)
    torch.cuda.synchronize()
    st = d.status.tolist()
    bit = {name: b for b, name in stv.DEV_ERRORS.items()}
    assert st[0] == 0 and st[1] & bit["parent"] and st[2] & bit["length"], st
    k_after, v_after = host_kv(w, d.k), host_kv(w, d.v)
    for b in (1, 2):  # nothing of sequences 1 and 2 was written
        for i in range(w.T):
            t = int(w.prefix_lens[b]) + i
            blk, off = int(w.block_table[b][t // 16]), t % 16
            assert np.array_equal(k_after[blk, :, off].view(np.uint8), k_before[blk, :, off].view(np.uint8))
            assert np.array_equal(v_after[blk, :, off].view(np.uint8), v_before[blk, :, off].view(np.uint8))


def test_kv_write_bad_block_index_skips_only_that_page():
    w = make_workload(name="bad_block", tag=722, V=8, B=2, Hq=4, Hkv=2, D=128, dtype="bf16", prefix=[10, 20],
                      tree="random", T=12, max_depth=3)
    print(f"[kv_write] bad block index B={w.B} T={w.T}", flush=True)
    d = DevWorkload(w)
    nb = d.k.shape[0]
    table = w.block_table.copy()
    assert table.shape[1] >= 2
    table[0, 1] = nb  # slots 16.. of sequence 0 (tree nodes 6..11) point outside the cache
    k_new = _rows(w, 11, (w.B, w.T, w.Hkv, w.D))
    v_new = _rows(w, 12, (w.B, w.T, w.Hkv, w.D))
    q = dev_kv(w, w.q)
    k_before, v_before = host_kv(w, d.k).copy(), host_kv(w, d.v).copy()
    stv.spec_tree_kv_write(dev_kv(w, k_new), dev_kv(w, v_new), q, d.k, d.v, torch.from_numpy(table).cuda(),
                           d.prefix_lens, d.parent, 10000.0, status=d.status)
    torch.cuda.synchronize()
    bit = {name: b for b, name in stv.DEV_ERRORS.items()}
    st = d.status.tolist()
    assert st[0] == bit["block"] and st[1] == 0, st
    q_ref, k_ref, v_ref = oracle.tree_kv_write(k_new, v_new, w.q, w.k_cache, w.v_cache, w.block_table,
                                               w.prefix_lens, w.parent, 10000.0, dtype=w.dtype)
    k_got, v_got = host_kv(w, d.k), host_kv(w, d.v)
    written = np.zeros((nb, 16), dtype=bool)
    for b in range(w.B):
        for i in range(w.T):
            t = int(w.prefix_lens[b]) + i
            if b == 0 and t >= 16:
                continue  # the skipped page
            blk, off = int(w.block_table[b][t // 16]), t % 16
            written[blk, off] = True
            assert np.array_equal(v_got[blk, :, off], v_new[b, i]), f"V row of node {i}, sequence {b}"
            _close(_widen(w, k_got[blk, :, off]), k_ref[blk, :, off], w.dtype, f"K row of node {i}, sequence {b}")
    for name, got, before in (("K", k_got, k_before), ("V", v_got, v_before)):
        g = got.transpose(0, 2, 1, 3)[~written]
        o = before.transpose(0, 2, 1, 3)[~written]
        assert np.array_equal(g.view(np.uint8), o.view(np.uint8)), f"{name}: a slot outside the written rows changed"
    _close(_widen(w, host_kv(w, q)), q_ref, w.dtype, "queries")  # the queries are rotated all the same
