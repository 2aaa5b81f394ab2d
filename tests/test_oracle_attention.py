"""Pins for the oracle's tree-masked attention.

* a chain tree equals ordinary causal attention (torch SDPA, fp64, CPU);
* every root-to-leaf path run alone with causal attention equals the tree
  result at its nodes (brute force on tiny trees);
* with Q = 0 every output is the mean of V over prefix + ancestors-or-self;
* T = 1 equals single-token decode attention; permuting physical blocks
  together with the block table changes nothing; GQA maps head h to h // G.
"""
import numpy as np
import pytest
import torch

from oracle import tree_attention, tree_attention_rows, tree_structure
from workloads import bf16_bits_to_f32, make_config, make_workload


def _contig(w, cache, b, n):
    """[n, Hkv, D] float64 rows of logical positions 0..n-1, gathered by hand."""
    c = w.as_f32(cache).astype(np.float64)
    rows = [c[w.block_table[b][t // 16], :, t % 16, :] for t in range(n)]
    return np.stack(rows)


def _sdpa(q, k, v, mask, scale):
    """torch's SDPA in fp64 on the CPU: q [H, M, D], k/v [H, N, D], mask [M, N] bool."""
    out = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v),
        attn_mask=torch.from_numpy(mask), scale=scale)
    return out.numpy()


@pytest.mark.parametrize("dtype,Hq,Hkv", [("f32", 2, 2), ("bf16", 4, 2), ("f32", 6, 3)])
def test_chain_equals_causal_sdpa(dtype, Hq, Hkv):
    w = make_workload(tag=201, B=2, Hq=Hq, Hkv=Hkv, D=32, dtype=dtype, V=8, prefix=[21, 35],
                      tree="chain", gamma=5, shuffle_blocks=True)
    out = tree_attention(w.q, w.k_cache, w.v_cache, w.block_table, w.prefix_lens, w.parent,
                         w.scale, dtype=dtype)
    G = Hq // Hkv
    for b in range(w.B):
        L = int(w.prefix_lens[b])
        n = L + w.T
        K = _contig(w, w.k_cache, b, n)
        V = _contig(w, w.v_cache, b, n)
        mask = np.arange(n)[None, :] <= (L + np.arange(w.T))[:, None]
        q = w.as_f32(w.q[b]).astype(np.float64).transpose(1, 0, 2)  # [Hq, T, D]
        kk = np.repeat(K.transpose(1, 0, 2), G, axis=0)
        vv = np.repeat(V.transpose(1, 0, 2), G, axis=0)
        ref = _sdpa(q, kk, vv, mask, w.scale).transpose(1, 0, 2)
        np.testing.assert_allclose(out[b], ref, rtol=1e-12, atol=1e-12)


def _root_to_leaf_paths(parent):
    tree = tree_structure(parent)
    return [tree.anc[i] for i in range(tree.T) if not tree.children[i]]


@pytest.mark.parametrize("tree_kind", ["cfg0", "random"])
def test_each_path_alone_matches_tree(tree_kind):
    if tree_kind == "cfg0":
        w = make_config(0)
    else:
        w = make_workload(tag=202, B=3, Hq=4, Hkv=1, D=16, dtype="bf16", V=8, prefix=[0, 17, 40],
                          tree="random", T=8, max_depth=3, shuffle_blocks=True)
    out = tree_attention(w.q, w.k_cache, w.v_cache, w.block_table, w.prefix_lens, w.parent,
                         w.scale, dtype=w.dtype)
    G = w.Hq // w.Hkv
    for b in range(w.B):
        L = int(w.prefix_lens[b])
        K = _contig(w, w.k_cache, b, L + w.T)
        V = _contig(w, w.v_cache, b, L + w.T)
        for path in _root_to_leaf_paths(w.parent[b]):
            pos = list(range(L)) + [L + j for j in path]
            n = len(pos)
            mask = np.arange(n)[None, :] <= (L + np.arange(len(path)))[:, None]
            q = w.as_f32(w.q[b][path]).astype(np.float64).transpose(1, 0, 2)
            kk = np.repeat(K[pos].transpose(1, 0, 2), G, axis=0)
            vv = np.repeat(V[pos].transpose(1, 0, 2), G, axis=0)
            ref = _sdpa(q, kk, vv, mask, w.scale).transpose(1, 0, 2)
            np.testing.assert_allclose(out[b][path], ref, rtol=1e-12, atol=1e-12)


def test_zero_query_gives_mean_over_visible_rows():
    w = make_config(0)
    q0 = np.zeros_like(w.q)
    out = tree_attention(q0, w.k_cache, w.v_cache, w.block_table, w.prefix_lens, w.parent,
                         w.scale, dtype=w.dtype)
    V = _contig(w, w.v_cache, 0, 128 + 8)
    # cfg0 tree [-1,0,0,1,1,2,3,4]: node 6 sees prefix + {0,1,3,6}, node 5 sees prefix + {0,2,5}
    np.testing.assert_allclose(out[0, 6], V[list(range(128)) + [128, 129, 131, 134]].mean(0), atol=1e-13)
    np.testing.assert_allclose(out[0, 5], V[list(range(128)) + [128, 130, 133]].mean(0), atol=1e-13)
    np.testing.assert_allclose(out[0, 0], V[:129].mean(0), atol=1e-13)


def test_single_node_is_decode_attention():
    w = make_workload(tag=203, B=2, Hq=4, Hkv=2, D=16, dtype="f32", V=8, prefix=[5, 0],
                      tree="fixed", parent=[-1])
    out = tree_attention(w.q, w.k_cache, w.v_cache, w.block_table, w.prefix_lens, w.parent, w.scale)
    for b in range(2):
        L = int(w.prefix_lens[b])
        K = _contig(w, w.k_cache, b, L + 1)
        V = _contig(w, w.v_cache, b, L + 1)
        for h in range(4):
            s = w.scale * K[:, h // 2] @ w.q[b, 0, h].astype(np.float64)
            p = np.exp(s - s.max())
            np.testing.assert_allclose(out[b, 0, h], (p / p.sum()) @ V[:, h // 2], atol=1e-13)


def test_block_permutation_invariance():
    w = make_workload(tag=204, B=2, Hq=2, Hkv=2, D=16, dtype="bf16", V=8, prefix=[30, 50],
                      tree="random", T=6, max_depth=3, extra_blocks=3)
    out = tree_attention(w.q, w.k_cache, w.v_cache, w.block_table, w.prefix_lens, w.parent,
                         w.scale, dtype="bf16")
    perm = np.random.default_rng(5).permutation(w.num_blocks)
    inv = np.argsort(perm)
    k2, v2 = w.k_cache[perm], w.v_cache[perm]  # new block j holds old block perm[j]
    table2 = inv[w.block_table].astype(np.int32)
    out2 = tree_attention(w.q, k2, v2, table2, w.prefix_lens, w.parent, w.scale, dtype="bf16")
    np.testing.assert_array_equal(out, out2)


def test_rows_variant_matches_full():
    w = make_workload(tag=205, B=2, Hq=4, Hkv=2, D=16, dtype="bf16", V=8, prefix=[9, 33],
                      tree="random", T=7, max_depth=4)
    full = tree_attention(w.q, w.k_cache, w.v_cache, w.block_table, w.prefix_lens, w.parent,
                          w.scale, dtype="bf16")
    rows = [(0, 0, 0), (1, 6, 3), (1, 2, 1), (0, 5, 2)]
    part = tree_attention_rows(w.q, w.k_cache, w.v_cache, w.block_table, w.prefix_lens, w.parent,
                               w.scale, rows, dtype="bf16")
    for r, (b, i, h) in enumerate(rows):  # same arithmetic up to BLAS summation order
        np.testing.assert_allclose(part[r], full[b, i, h], rtol=1e-13, atol=1e-14)


def test_bf16_widening_is_exact():
    from oracle.attention import _widen
    bits = np.array([0x3F80, 0xBF80, 0x4049, 0x0001, 0x7F7F], dtype=np.uint16)
    want = np.array([1.0, -1.0, 3.140625, 2.0 ** -133, 3.3895313892515355e38])
    np.testing.assert_array_equal(_widen(bits, "bf16"), want)
    np.testing.assert_array_equal(bf16_bits_to_f32(bits).astype(np.float64), want)
