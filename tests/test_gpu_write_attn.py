"""spec_tree_write_attn -- the tree's K/V write and the verify attention in one
launch -- on the GPU, through the C ABI:

* against the oracle: oracle/rope.py's rotated keys and queries (rounded to
  bf16 as the cache stores them) fed to oracle/attention.py, within the
  attention tolerance of test_gpu_attention.py; the written cache rows within
  one bf16 unit of oracle/rope.py's, every other slot unchanged;
* against the separate calls on the same inputs: spec_tree_kv_write, then
  spec_tree_attn on the queries it rotated, leave the same cache bit for bit;
  their outputs agree within the stated bf16 attention tolerance everywhere,
  and both are within the oracle's bound on the compared rows (the one-launch
  path shortens the stream-K ranges of the workgroups that write, so a
  (sequence, kv head) may be cut at other points: each piece rounds P to bf16
  against its own running max and the partials merge in another order);
* the caller's queries are left as they were; one workspace serves calls in a
  row (its counters are back at zero after each call); a bad parent row is
  reported and leaves that sequence's cache rows unwritten while the other
  sequences are exact.

Shapes: the one-launch path (ragged batches of 64 sequences in longest-first
order: 16-node random trees, and 64-node chains whose items and chains go past
the cosine table and the walked depths) and the two-launch path (64-row tiles
in plain order, 128-row tiles on a 70-node tree, a 300-node Sequoia-profile tree
and a 64-node chain, a chain of 5 rows on the streaming kernel, an unrotated
write).
"""
import numpy as np
import pytest
import torch

import oracle
import tree_verify_attention_masked_amd as stv
from helpers import BF16_ATOL, BF16_RTOL, DevWorkload, abs_values, assert_attn_close, attn_to_f64, dev_kv, host_kv
from workloads import make_workload
from workloads.gen import f32_to_bf16_bits

pytestmark = pytest.mark.gpu

CASES = [
    # (name, workload kwargs, rope theta, rows compared with the oracle: None = all)
    ("rows64_longest_first", dict(B=64, Hq=32, Hkv=8, prefix=[9000] + [16 + (37 * i) % 600 for i in range(63)],
                                  tree="random", T=16, max_depth=5, shuffle_blocks=True), 10000.0, 160),
    ("rows64_chains_one_launch", dict(B=64, Hq=3, Hkv=3, prefix=[3000] + [16 + (53 * i) % 900 for i in range(63)],
                                      tree="chain", gamma=63, shuffle_blocks=True), 10000.0, 200),
    ("rows64_plain_order", dict(B=3, Hq=8, Hkv=2, prefix=[1, 130, 700], tree="random", T=7, max_depth=4,
                                shuffle_blocks=True), 10000.0, None),
    ("rows128_tree", dict(B=1, Hq=16, Hkv=1, prefix=[900], tree="random", T=70, max_depth=8,
                          shuffle_blocks=True), 500000.0, None),
    ("rows128_t300_sequoia", dict(B=1, Hq=8, Hkv=2, prefix=[700], tree="sequoia", T=300, max_depth=12,
                                  shuffle_blocks=True), 10000.0, 200),
    ("deep_chain_direct_angles", dict(B=1, Hq=2, Hkv=1, prefix=[100], tree="chain", gamma=63), 10000.0, None),
    ("chain_rows5", dict(B=1, Hq=40, Hkv=40, prefix=[300], tree="chain", gamma=4), 10000.0, None),
    ("unrotated", dict(B=2, Hq=4, Hkv=2, prefix=[16, 31], tree="random", T=9, max_depth=3), 0.0, None),
    # the streaming kernel's launch (at most 16 rows per kv head), which rotates
    # its own queries and whose items holding tree keys write them: a tree that
    # straddles two pages over several KV splits, and an unrotated ragged batch
    ("stream_tail_straddles", dict(B=2, Hq=8, Hkv=8, prefix=[1918, 5000], tree="chain", gamma=4,
                                   shuffle_blocks=True), 10000.0, None),
    ("stream_unrotated", dict(B=3, Hq=8, Hkv=4, prefix=[0, 15, 333], tree="random", T=8, max_depth=3), 0.0, None),
]


def _rows(seed, shape):
    return f32_to_bf16_bits(np.random.default_rng(seed).normal(size=shape).astype(np.float32))


def _bf16(x):
    return f32_to_bf16_bits(np.asarray(x, dtype=np.float64).astype(np.float32))


def _bits(t):
    return t.view(torch.int16)


def _workload(name, kw, tag):
    return make_workload(name=name, tag=tag, V=8, D=128, dtype="bf16", **kw)


def _fused(w, d, k_new, v_new, theta, workspace=None):
    q = dev_kv(w, w.q)
    out = stv.spec_tree_write_attn(dev_kv(w, k_new), dev_kv(w, v_new), q, d.k, d.v, d.block_table, d.prefix_lens,
                                   d.parent, theta, scale=w.scale, status=d.status, workspace=workspace)
    torch.cuda.synchronize()
    assert torch.equal(_bits(q), _bits(dev_kv(w, w.q))), "the caller's queries changed"
    return out


def _separate(w, k_new, v_new, theta):
    d = DevWorkload(w)
    q = dev_kv(w, w.q)
    stv.spec_tree_kv_write(dev_kv(w, k_new), dev_kv(w, v_new), q, d.k, d.v, d.block_table, d.prefix_lens, d.parent,
                           theta, status=d.status)
    out = stv.spec_tree_attn(q, d.k, d.v, d.block_table, d.prefix_lens, d.parent, scale=w.scale, status=d.status)
    torch.cuda.synchronize()
    assert int(d.status.abs().sum()) == 0
    return d, out


def _assert_same_outputs(out, out_sep, what):
    """Outputs of the two paths everywhere: within the stated bf16 attention
    tolerance of each other (the tight bound is checked against the oracle)."""
    a, b = out.double(), out_sep.double()
    bad = ~((a - b).abs() <= BF16_ATOL + BF16_RTOL * b.abs())
    assert not bool(bad.any()), f"{what}: {int(bad.sum())} outputs differ from the separate calls"


def _oracle(w, k_new, v_new, theta, rows):
    """Oracle rows of the fused call: rotate (fp64), round to bf16 as stored, attend."""
    q_rot, kc, vc = oracle.tree_kv_write(k_new, v_new, w.q, w.k_cache, w.v_cache, w.block_table, w.prefix_lens,
                                         w.parent, theta, dtype="bf16")
    qb, kb, vb = _bf16(q_rot), _bf16(kc), _bf16(vc)
    va = abs_values(w, vb)
    if rows is None:
        f = lambda v: oracle.tree_attention(qb, kb, v, w.block_table, w.prefix_lens, w.parent, w.scale, dtype="bf16")
    else:
        f = lambda v: oracle.tree_attention_rows(qb, kb, v, w.block_table, w.prefix_lens, w.parent, w.scale, rows,
                                                 dtype="bf16")
    return f(vb), f(va), kc, vc


@pytest.mark.parametrize("name,kw,theta,n_rows", CASES, ids=[c[0] for c in CASES])
def test_write_attn(name, kw, theta, n_rows):
    w = _workload(name, kw, 900 + [c[0] for c in CASES].index(name))
    print(f"[write_attn] {name} B={w.B} T={w.T} Hq={w.Hq} Hkv={w.Hkv} theta={theta}", flush=True)
    k_new = _rows(11, (w.B, w.T, w.Hkv, w.D))
    v_new = _rows(12, (w.B, w.T, w.Hkv, w.D))
    d = DevWorkload(w)
    out = _fused(w, d, k_new, v_new, theta)
    assert int(d.status.abs().sum()) == 0, d.status.tolist()
    d_sep, out_sep = _separate(w, k_new, v_new, theta)
    assert torch.equal(_bits(d.k), _bits(d_sep.k)) and torch.equal(_bits(d.v), _bits(d_sep.v)), "cache differs"
    _assert_same_outputs(out, out_sep, name)
    if w.T * (w.Hq // w.Hkv) <= 16:  # the streaming launch runs the separate attention's own arithmetic
        assert torch.equal(_bits(out), _bits(out_sep)), f"{name}: outputs differ from the separate calls"
    rows = None
    if n_rows is not None:
        rng = np.random.default_rng(5)
        rows = [(int(rng.integers(w.B)), int(rng.integers(w.T)), int(rng.integers(w.Hq))) for _ in range(n_rows)]
        rows += [(w.B - 1, i, h) for i in range(w.T) for h in (0, w.Hq - 1)][:200]
    ref, ref_abs, kc, _ = _oracle(w, k_new, v_new, theta, rows)
    for label, o in (("one launch", out), ("separate calls", out_sep)):
        got = attn_to_f64(w, o)
        if rows is not None:
            got = np.stack([got[b, i, h] for b, i, h in rows])
        assert_attn_close(got, ref, "bf16", f"{name}, {label}", ref_abs)
    # the cache against the oracle: written rows within one bf16 unit (values
    # exact), every other slot bit for bit as it was (unused slots hold NaN)
    k_got, v_got = host_kv(w, d.k), host_kv(w, d.v)
    written = np.zeros(k_got.shape[0] * 16, dtype=bool).reshape(k_got.shape[0], 16)
    for b in range(w.B):
        for i in range(w.T):
            t = int(w.prefix_lens[b]) + i
            blk, off = int(w.block_table[b][t // 16]), t % 16
            written[blk, off] = True
            kf = (k_got[blk, :, off].astype(np.uint32) << 16).view(np.float32).astype(np.float64)
            ref_k = kc[blk, :, off]
            assert np.all(np.abs(kf - ref_k) <= 2.0 ** -8 * np.abs(ref_k) + 1e-12), f"K row of node {i}, seq {b}"
            assert np.array_equal(v_got[blk, :, off], v_new[b, i]), f"V row of node {i}, seq {b}"
    for got, before in ((k_got, w.k_cache), (v_got, w.v_cache)):
        g = got.transpose(0, 2, 1, 3)[~written]
        o = np.asarray(before).transpose(0, 2, 1, 3)[~written]
        assert np.array_equal(g.view(np.uint16), o.view(np.uint16)), "a slot outside the tree changed"


def test_workspace_serves_calls_in_a_row():
    """Three calls on one workspace (new rows each time): every call equals the separate calls."""
    name, kw, theta, _ = CASES[0]
    w = _workload("reuse", kw, 950)
    ws = torch.zeros(stv.spec_tree_write_attn_workspace_size(w.B, w.T, w.Hq, w.Hkv, w.D, w.max_blocks,
                                                             stv.SPEC_BF16), dtype=torch.uint8, device="cuda")
    for call in range(3):
        k_new = _rows(20 + call, (w.B, w.T, w.Hkv, w.D))
        v_new = _rows(30 + call, (w.B, w.T, w.Hkv, w.D))
        d = DevWorkload(w)
        out = _fused(w, d, k_new, v_new, theta, workspace=ws)
        d_sep, out_sep = _separate(w, k_new, v_new, theta)
        _assert_same_outputs(out, out_sep, f"call {call}")
        assert torch.equal(_bits(d.k), _bits(d_sep.k)), f"call {call}"
        n_chunks = (2 * w.T * w.Hkv + 63) // 64
        # arrival counters, [unused, workgroups done], written-chunk counts, chunk claims
        head = ws[: 4 * (w.B * w.Hkv * 1 + 2 + w.B + w.B * n_chunks)].view(torch.int32)
        assert int(head.abs().sum()) == 0, f"call {call} left counters set"


BAD_PARENT = [
    ("two_launches", dict(B=3, Hq=8, Hkv=2, prefix=[40, 200, 7], tree="random", T=12, max_depth=4)),
    ("one_launch", dict(B=64, Hq=32, Hkv=8, prefix=[9000, 200] + [16 + (37 * i) % 600 for i in range(62)],
                        tree="random", T=16, max_depth=5, shuffle_blocks=True)),
    ("stream_launch", dict(B=3, Hq=4, Hkv=4, prefix=[40, 200, 7], tree="random", T=6, max_depth=3)),
]


@pytest.mark.parametrize("name,kw", BAD_PARENT, ids=[c[0] for c in BAD_PARENT])
def test_bad_parent_is_reported_and_writes_nothing(name, kw):
    w = _workload("bad_parent_" + name, kw, 960 + [c[0] for c in BAD_PARENT].index(name))
    k_new = _rows(41, (w.B, w.T, w.Hkv, w.D))
    v_new = _rows(42, (w.B, w.T, w.Hkv, w.D))
    d = DevWorkload(w)
    d.parent[1, 5] = 9  # not an earlier node
    out = _fused(w, d, k_new, v_new, 10000.0)
    st = d.status.cpu().tolist()
    assert st[1] & 1 and st[0] == 0 and st[2] == 0 and sum(map(abs, st)) == st[1], st
    k_before = host_kv(w, dev_kv(w, w.k_cache))
    k_got = host_kv(w, d.k)
    for i in range(w.T):  # sequence 1's tree slots keep what the cache held
        t = int(w.prefix_lens[1]) + i
        blk, off = int(w.block_table[1][t // 16]), t % 16
        assert np.array_equal(k_got[blk, :, off], k_before[blk, :, off])
    ref, ref_abs, _, _ = _oracle(w, k_new, v_new, 10000.0, [(b, i, h) for b in (0, 2) for i in range(w.T)
                                                          for h in range(w.Hq)])
    got = attn_to_f64(w, out)
    got = np.stack([got[b, i, h] for b in (0, 2) for i in range(w.T) for h in range(w.Hq)])
    assert_attn_close(got, ref, "bf16", "other sequences", ref_abs)
