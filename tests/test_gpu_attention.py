"""GPU parity of spec_tree_attn against the fp64 oracle (called through the C ABI).

Tolerance: bf16 outputs |gpu - oracle| <= 2e-2 + 1e-2 |oracle| (the stated
bar) and also <= 2^-8 (attn(|V|) + |oracle|) + 1e-5, twice the effect of the
bf16 rounding of the probabilities and of the output (helpers.py derives it);
fp32 outputs 1e-5 + 1e-5 |oracle|.  Small cases compare every output and span several KV
tiles, several splits, a ragged last page and each kernel variant (streaming
for <= 16 rows per kv head, 64-row and 128-row tiles); the five configurations
run at full size, all outputs where the oracle is quick, sampled rows
otherwise.
"""
import numpy as np
import pytest
import torch

import oracle
from helpers import DevWorkload, assert_attn_close, attn_to_f64, oracle_attn
from workloads import make_config, make_workload
from workloads.gen import bf16_bits_to_f32, f32_to_bf16_bits

pytestmark = pytest.mark.gpu


def _run_full(w):
    d = DevWorkload(w)
    out = d.attn()
    torch.cuda.synchronize()
    ref, ref_abs = oracle_attn(w)
    err = assert_attn_close(attn_to_f64(w, out), ref, w.dtype, w.name, ref_abs)
    assert int(d.status.abs().sum()) == 0
    return err


SMALL = [
    # (name, kwargs)
    ("f32_d64_tree", dict(B=2, Hq=4, Hkv=2, D=64, dtype="f32", prefix=[0, 77], tree="random", T=9, max_depth=4)),
    ("f32_d128_chain", dict(B=1, Hq=3, Hkv=1, D=128, dtype="f32", prefix=[50], tree="chain", gamma=6)),
    ("keysplit_chain", dict(B=2, Hq=4, Hkv=4, D=128, dtype="bf16", prefix=[17, 1000], tree="chain", gamma=4)),
    ("keysplit_tree_gqa", dict(B=3, Hq=8, Hkv=4, D=128, dtype="bf16", prefix=[0, 15, 333], tree="random", T=8,
                               max_depth=3, shuffle_blocks=True)),
    ("rows64_tree", dict(B=3, Hq=8, Hkv=2, D=128, dtype="bf16", prefix=[1, 130, 700], tree="random", T=7,
                         max_depth=4, shuffle_blocks=True)),
    ("rows64_many_splits", dict(B=1, Hq=4, Hkv=1, D=128, dtype="bf16", prefix=[6000], tree="random", T=16,
                                max_depth=5)),
    ("rows256_tree", dict(B=1, Hq=16, Hkv=1, D=128, dtype="bf16", prefix=[900], tree="random", T=70,
                          max_depth=8, shuffle_blocks=True)),
    ("rows256_ragged", dict(B=2, Hq=32, Hkv=2, D=128, dtype="bf16", prefix=[5, 2222], tree="random", T=40,
                            max_depth=6)),
    ("single_node", dict(B=3, Hq=4, Hkv=2, D=128, dtype="bf16", prefix=[0, 1, 31], tree="fixed", parent=[-1])),
    ("deep_chain_t256", dict(B=1, Hq=2, Hkv=1, D=128, dtype="bf16", prefix=[100], tree="chain", gamma=255)),
    # few keys per row: a row sum that is not the sum over all four lanes of the
    # row shows up here (with thousands of keys it averages out)
    ("rows128_chain_short_prefix", dict(B=1, Hq=2, Hkv=1, D=128, dtype="bf16", prefix=[96], tree="chain",
                                        gamma=95)),
    ("rows256_tree_short_prefix", dict(B=1, Hq=16, Hkv=1, D=128, dtype="bf16", prefix=[5], tree="random", T=64,
                                       max_depth=6)),
    # the Sequoia-scale layer's launch shape (512 items, two rounds of one
    # workgroup a CU, splits of each row tile in both rounds, so first-round
    # splits are weighted) with prefixes long enough for weighted boundaries
    # (1500, 8 waves of tiles) and too short for them (300: equal splits)
    ("rows2048_weighted_splits", dict(B=1, Hq=64, Hkv=8, D=128, dtype="bf16", prefix=[1500], tree="random", T=256,
                                      max_depth=10)),
    ("rows2048_short_prefix", dict(B=1, Hq=64, Hkv=8, D=128, dtype="bf16", prefix=[300], tree="random", T=256,
                                   max_depth=10)),
    # routing boundaries: 17 rows (the first tile-kernel shape), 64 rows over a
    # ragged batch whose sequences need 1..3 splits (later splits exit at once),
    # 65 rows (a second 128-row tile that is almost empty)
    ("rows17_chain", dict(B=2, Hq=1, Hkv=1, D=128, dtype="bf16", prefix=[40, 300], tree="chain", gamma=16)),
    ("rows64_ragged_splits", dict(B=3, Hq=8, Hkv=2, D=128, dtype="bf16", prefix=[3, 9000, 700], tree="random", T=16,
                                  max_depth=5, shuffle_blocks=True)),
    ("rows65_tree", dict(B=1, Hq=5, Hkv=1, D=128, dtype="bf16", prefix=[1234], tree="random", T=13, max_depth=4)),
    # a ragged batch with more 64-row items than resident workgroups: dispatched
    # longest items first (full splits, then last splits by decreasing length);
    # every row is checked, so an item the id mapping skipped or repeated fails
    ("rows64_longest_first", dict(B=64, Hq=32, Hkv=8, D=128, dtype="bf16",
                                  prefix=[9000] + [16 + (37 * i) % 600 for i in range(63)], tree="random", T=16,
                                  max_depth=5, shuffle_blocks=True)),
    # the persistent kernel (ragged batch, more 64-row items than resident
    # workgroups) with last splits of 1 to 16 pages, i.e. items of 1 to 4 tiles,
    # so the issue of tiles waits on the next item's prefetch and runs dry
    ("rows64_persistent_tiny_items", dict(B=64, Hq=32, Hkv=8, D=128, dtype="bf16",
                                          prefix=[16000] + [16 * (252 * (i % 3) + 1 + i % 16) - 16 for i in range(63)],
                                          tree="random", T=16, max_depth=5, shuffle_blocks=True)),
    # fp32 kernel: ancestors past the first 64 lanes' words, GQA over a long and an almost empty prefix
    ("f32_d64_deep_chain", dict(B=1, Hq=2, Hkv=1, D=64, dtype="f32", prefix=[70], tree="chain", gamma=200)),
    ("f32_d128_gqa_tree", dict(B=2, Hq=6, Hkv=2, D=128, dtype="f32", prefix=[1300, 1], tree="random", T=40,
                               max_depth=7, shuffle_blocks=True)),
    # trees of more than 256 nodes: ancestor bitsets of up to 8 words, each item
    # keeping only its own nodes' (32 nodes per 128-row item at 4 query heads per
    # kv head; 128 for the chain, one head); tree keys in several 64-key tiles
    ("rows_t300_sequoia", dict(B=1, Hq=8, Hkv=2, D=128, dtype="bf16", prefix=[700], tree="sequoia", T=300,
                               max_depth=12, shuffle_blocks=True)),
    ("rows_t512_tree_ragged", dict(B=2, Hq=4, Hkv=2, D=128, dtype="bf16", prefix=[0, 1500], tree="random", T=512,
                                   max_depth=9)),
    ("deep_chain_t512", dict(B=1, Hq=1, Hkv=1, D=128, dtype="bf16", prefix=[40], tree="chain", gamma=511)),
    ("f32_t300_tree", dict(B=1, Hq=2, Hkv=1, D=64, dtype="f32", prefix=[33], tree="random", T=300, max_depth=20)),
]


@pytest.mark.parametrize("name,kw", SMALL, ids=[s[0] for s in SMALL])
def test_small_cases(name, kw):
    w = make_workload(name=name, tag=400 + SMALL.index((name, kw)), V=8, **kw)
    print(f"[attn] {name} B={w.B} T={w.T} Hq={w.Hq} Hkv={w.Hkv} lens={w.prefix_lens.tolist()}", flush=True)
    _run_full(w)


@pytest.mark.parametrize("Hq,T", [(16, 40), (8, 8)], ids=["rows320", "rows64"])
def test_rising_scores_move_the_reference_max(Hq, T):
    # Keys scaled up by 1 .. 9 along each sequence, so every row's largest score
    # keeps growing: the tile kernels' reference max (which moves only when a
    # row's max passes it by more than 2^8 in the exponent) moves many times,
    # each move rescaling what was accumulated against the old one.
    w = make_workload(name="rising", tag=470 + Hq, B=2, Hq=Hq, Hkv=2, D=128, dtype="bf16", V=8,
                      prefix=[3000, 900], tree="random", T=T, max_depth=5, shuffle_blocks=True)
    k = bf16_bits_to_f32(w.k_cache)
    for b in range(w.B):
        n = int(w.prefix_lens[b]) + w.T
        for t in range(n):
            k[w.block_table[b][t // 16], :, t % 16, :] *= 1.0 + 8.0 * t / n
    w.k_cache = f32_to_bf16_bits(k)
    print(f"[attn] rising scores B={w.B} T={w.T} Hq={w.Hq} Hkv={w.Hkv} lens={w.prefix_lens.tolist()}", flush=True)
    _run_full(w)


@pytest.mark.parametrize("cfg", [0, 1, 3])
def test_config_full(cfg):
    w = make_config(cfg)
    print(f"[attn] config {cfg} {w.name}", flush=True)
    _run_full(w)


@pytest.mark.parametrize("cfg", [2, 4])
def test_config_sampled_rows(cfg):
    w = make_config(cfg)
    print(f"[attn] config {cfg} {w.name} (sampled rows)", flush=True)
    d = DevWorkload(w)
    out = attn_to_f64(w, d.attn())
    assert int(d.status.abs().sum()) == 0
    rng = np.random.default_rng(cfg)
    rows = [(int(rng.integers(w.B)), int(rng.integers(w.T)), int(rng.integers(w.Hq))) for _ in range(200)]
    rows += [(w.B - 1, i, h) for i in range(w.T) for h in (0, w.Hq - 1)]  # every node of one sequence
    ref, ref_abs = oracle_attn(w, rows)
    got = np.stack([out[b, i, h] for b, i, h in rows])
    assert_attn_close(got, ref, w.dtype, w.name, ref_abs)


def test_bad_inputs_are_reported_not_faulted():
    w = make_workload(tag=480, B=3, Hq=4, Hkv=4, D=128, dtype="bf16", V=8, prefix=[20, 40, 60], tree="random",
                      T=6, max_depth=3)
    d = DevWorkload(w)
    d.parent[1, 3] = 5  # not topological
    d.block_table[2, 0] = w.num_blocks + 7  # outside the pool
    d.prefix_lens[0] = -4
    d.attn()
    st = d.status.cpu().numpy()
    assert st[0] & 4 and st[1] & 1 and st[2] & 2


def test_bad_inputs_are_reported_on_the_persistent_path():
    # a batch that takes the persistent kernel: a bad parent row, a block index
    # outside the pool and a bad prefix length are reported for their sequences,
    # and every row of every other sequence still matches the oracle
    w = make_workload(tag=484, B=64, Hq=32, Hkv=8, D=128, dtype="bf16", V=8,
                      prefix=[9000] + [16 + (37 * i) % 600 for i in range(63)], tree="random", T=16, max_depth=5,
                      shuffle_blocks=True)
    d = DevWorkload(w)
    bad = {3: "parent", 0: "block", 5: "length"}
    d.parent[3, 7] = 12  # not topological
    d.block_table[0, 300] = w.num_blocks + 7  # a page inside sequence 0's third split
    d.prefix_lens[5] = -4
    out = attn_to_f64(w, d.attn())
    st = d.status.cpu().numpy()
    assert st[3] & 1 and st[0] & 2 and st[5] & 4
    assert all(st[b] == 0 for b in range(w.B) if b not in bad)
    ref, ref_abs = oracle_attn(w)
    keep = [b for b in range(w.B) if b not in bad]
    assert_attn_close(out[keep], ref[keep], w.dtype, "persistent, good sequences", ref_abs[keep])


def test_bad_inputs_are_reported_not_faulted_f32():
    w = make_workload(tag=483, B=3, Hq=2, Hkv=2, D=64, dtype="f32", V=8, prefix=[20, 40, 60], tree="random",
                      T=6, max_depth=3)
    d = DevWorkload(w)
    d.parent[1, 3] = 5  # not topological
    d.block_table[2, 0] = w.num_blocks + 7  # outside the pool
    d.prefix_lens[0] = -4
    d.attn()
    st = d.status.cpu().numpy()
    assert st[0] & 4 and st[1] & 1 and st[2] & 2


def test_empty_batch_is_a_no_op():
    w = make_workload(tag=481, B=1, Hq=2, Hkv=2, D=128, dtype="bf16", V=8, prefix=[4], tree="chain", gamma=2)
    d = DevWorkload(w)
    import tree_verify_attention_masked_amd as stv
    out = stv.spec_tree_attn(d.q[:0], d.k, d.v, d.block_table[:0], d.prefix_lens[:0], d.parent[:0])
    assert out.shape[0] == 0


def test_block_permutation_invariance_on_gpu():
    w = make_workload(tag=482, B=2, Hq=8, Hkv=2, D=128, dtype="bf16", V=8, prefix=[300, 45], tree="random",
                      T=12, max_depth=4, extra_blocks=5)
    d = DevWorkload(w)
    a = d.attn().clone()
    perm = torch.from_numpy(np.random.default_rng(1).permutation(w.num_blocks)).cuda()
    inv = torch.argsort(perm).to(torch.int32)
    d.k = d.k[perm].contiguous()
    d.v = d.v[perm].contiguous()
    d.block_table = inv[d.block_table.long()].contiguous()
    b = d.attn()
    assert torch.equal(a, b)  # same data in the same order: bit-identical
