"""Rotary positions of the draft tree and the write of its K/V rows into the
paged cache (oracle side), fp64 -- TEST INFRASTRUCTURE ONLY.

Positions: the drafted tokens are scored in one pass, flattened, but each one
is at the position it would have in a plain sequence along its own path: the
vLLM issue ("Issue: Speculative Decoding on vLLM") notes that a sequence-based
verifier only has to adjust cache_position / position_ids, and the EAGLE
report ("Report: Support nextn speculative decoding", implementation summary)
flattens the tree into one input_ids row whose order is not the token order.
Reading taken: node i of sequence b is at position Lb + depth(i) (the committed
prefix, then its distance from the root).  Its K/V row goes to logical slot
Lb + i of the paged cache, where the verify attention reads it.

Rotation: the rotary position embedding of RoFormer (Su et al., "RoFormer:
Enhanced Transformer with Rotary Position Embedding", 2021; outside the pages),
in the half-split layout of Llama-family checkpoints (a reading: the pages name
no layout): for j < D/2 the pair (x_j, x_{j + D/2}) at position p is rotated by
the angle p * theta^(-2j/D),
    x_j'       = x_j cos(a) - x_{j+D/2} sin(a)
    x_{j+D/2}' = x_{j+D/2} cos(a) + x_j sin(a).
theta = 0 means no rotation (the rows are only written).
"""
from __future__ import annotations

import numpy as np

from .attention import _widen
from .tree import tree_structure


def tree_positions(parent, prefix_lens) -> np.ndarray:
    """[B, T] int64: Lb + depth(i)."""
    parent = np.asarray(parent)
    out = np.zeros(parent.shape, dtype=np.int64)
    for b in range(parent.shape[0]):
        depth = tree_structure(parent[b]).depth
        out[b] = int(prefix_lens[b]) + np.asarray(depth, dtype=np.int64)
    return out


def rope(x, pos, theta: float) -> np.ndarray:
    """x [..., D] (fp64), pos broadcastable to x.shape[:-1]: rotated copy, fp64."""
    x = np.asarray(x, dtype=np.float64)
    if theta == 0:
        return x.copy()
    D = x.shape[-1]
    h = D // 2
    j = np.arange(h, dtype=np.float64)
    inv_freq = float(theta) ** (-2.0 * j / D)
    ang = np.asarray(pos, dtype=np.float64)[..., None] * inv_freq
    c, s = np.cos(ang), np.sin(ang)
    lo, hi = x[..., :h], x[..., h:]
    return np.concatenate([lo * c - hi * s, hi * c + lo * s], axis=-1)


def tree_kv_write(k_new, v_new, q, k_cache, v_cache, block_table, prefix_lens, parent, theta, dtype="f32",
                  block_size=16):
    """k_new, v_new [B, T, Hkv, D]; q [B, T, Hq, D] or None; caches [blocks, Hkv, bs, D]
    (bf16 bit patterns with dtype="bf16").  Returns (q_rot, k_cache_new, v_cache_new) in
    fp64: the rotated queries, and the caches widened to fp64 with node i's rotated key
    and its value at logical slot Lb + i of sequence b."""
    pos = tree_positions(parent, prefix_lens)
    kc = _widen(k_cache, dtype).copy()
    vc = _widen(v_cache, dtype).copy()
    kr = rope(_widen(k_new, dtype), pos[:, :, None], theta)
    vn = _widen(v_new, dtype)
    B, T = pos.shape
    for b in range(B):
        for i in range(T):
            t = int(prefix_lens[b]) + i
            blk, off = int(block_table[b][t // block_size]), t % block_size
            kc[blk, :, off, :] = kr[b, i]
            vc[blk, :, off, :] = vn[b, i]
    qr = None if q is None else rope(_widen(q, dtype), pos[:, :, None], theta)
    return qr, kc, vc
