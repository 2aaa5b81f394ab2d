"""Tree-masked verify attention (oracle side), fp64.

What it computes ("Report: Support nextn speculative decoding", EAGLE
implementation summary step 3, with the attention_mask / tree_attention_mask
it names; the vLLM draft-model PR lists the multi-query PagedAttention used for
scoring as future work; the "Speculative Decoding" notes, "Draft Token
Validation", state that the drafted tokens are scored in one parallel pass):

For sequence b with Lb committed prefix tokens and a T-node draft tree whose
node i has its key/value row at logical position Lb + i, query head h of node i
(kv head g = h // (Hq / Hkv)) attends to

    K(i) = {0, ..., Lb - 1}  U  {Lb + j : j ancestor-or-self of i}

with s_t = scale * <q[b, i, h], k_t>, w = softmax(s) and
out[b, i, h] = sum_t w_t v_t.  Nothing else is applied (no causal mask inside
the prefix, no bias, no window).  Position t of sequence b is read at
cache[block_table[b][t // block_size], g, t % block_size, :].

Inputs may be float32/float64 arrays, or bfloat16 bit patterns (uint16) with
``kv_dtype="bf16"``; they are widened exactly to fp64 here.
"""
from __future__ import annotations

import numpy as np

from .tree import tree_structure


def _widen(a: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        bits = np.ascontiguousarray(a, dtype=np.uint16).astype(np.uint32) << 16
        return bits.view(np.float32).astype(np.float64)
    return np.asarray(a, dtype=np.float64)


def _gather(cache, table_row, n, block_size, dtype):
    """Rows of logical positions 0..n-1 of one sequence: [n, Hkv, D] fp64."""
    pos = np.arange(n)
    blocks = np.asarray(table_row)[pos // block_size]
    slots = pos % block_size
    return _widen(cache[blocks, :, slots, :], dtype)


def _attend(qrows, K, V, scale):
    """softmax(scale * q K^T) V for a few query rows over one key set, fp64."""
    s = scale * (qrows @ K.T)
    s = s - s.max(axis=-1, keepdims=True)
    w = np.exp(s)
    w = w / w.sum(axis=-1, keepdims=True)
    return w @ V


def tree_attention_rows(q, k_cache, v_cache, block_table, prefix_lens, parent, scale,
                        rows, dtype="f32", block_size=16):
    """Outputs for selected (b, i, h) triples only: returns fp64 [len(rows), D]."""
    Hq = q.shape[2]
    Hkv = k_cache.shape[1]
    G = Hq // Hkv
    by_b = {}
    for r, (b, i, h) in enumerate(rows):
        by_b.setdefault(int(b), []).append((r, int(i), int(h)))
    out = np.zeros((len(rows), q.shape[3]), dtype=np.float64)
    for b, items in by_b.items():
        tree = tree_structure(parent[b])
        L = int(prefix_lens[b])
        n = L + tree.T
        K = _gather(k_cache, block_table[b], n, block_size, dtype)
        V = _gather(v_cache, block_table[b], n, block_size, dtype)
        for r, i, h in items:
            keys = list(range(L)) + [L + j for j in tree.anc[i]]
            g = h // G
            qv = _widen(q[b, i, h], dtype)[None, :]
            out[r] = _attend(qv, K[keys, g, :], V[keys, g, :], scale)[0]
    return out


def tree_attention(q, k_cache, v_cache, block_table, prefix_lens, parent, scale,
                   dtype="f32", block_size=16):
    """Full output [B, T, Hq, D] in fp64."""
    B, T, Hq, D = q.shape
    Hkv = k_cache.shape[1]
    if Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    G = Hq // Hkv
    out = np.zeros((B, T, Hq, D), dtype=np.float64)
    for b in range(B):
        tree = tree_structure(parent[b])
        if tree.T != T:
            raise ValueError("parent row length must equal T")
        L = int(prefix_lens[b])
        n = L + T
        K = _gather(k_cache, block_table[b], n, block_size, dtype)
        V = _gather(v_cache, block_table[b], n, block_size, dtype)
        qb = _widen(q[b], dtype)  # [T, Hq, D]
        for i in range(T):
            keys = list(range(L)) + [L + j for j in tree.anc[i]]
            for g in range(Hkv):
                heads = slice(g * G, (g + 1) * G)
                out[b, i, heads] = _attend(qb[i, heads], K[keys, g, :], V[keys, g, :], scale)
    return out
