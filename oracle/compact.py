"""Selective KV-cache compaction (oracle side).

After verification only the accepted root-to-leaf path may stay in the cache:
the EAGLE report stresses updating the KV cache by the indices of accepted
tokens and calls the rewrite crucial for tree attention ("Report: Support nextn
speculative decoding", implementation detail and "Issue: Speculative Decoding on
vLLM"), and the SGLang doc notes that rejected tokens' KV must be evicted
("SpeculativeDecoding", "Prefix Match").

With path n_0 = 0, n_1, ..., n_L (node indices, increasing), for d = 1..L in
increasing order and every kv head, the K and V rows at logical position
Lb + n_d are copied to Lb + d.  Everything else is left untouched; slots past
the new length keep stale data.  new_len = Lb + L + 1 (the root and the L
accepted nodes; the emitted token has no KV yet).  Copies are plain element
copies, so the arrays may hold bf16 bit patterns or floats alike.
"""
from __future__ import annotations

import numpy as np


def kv_compact(k_cache, v_cache, block_table, prefix_lens, accepted_nodes, num_accepted,
               block_size=16):
    """Returns (k_new, v_new, new_lens); the inputs are not modified."""
    k = np.array(k_cache, copy=True)
    v = np.array(v_cache, copy=True)
    B = len(prefix_lens)
    new_lens = np.zeros(B, dtype=np.int32)
    for b in range(B):
        L = int(num_accepted[b])
        base = int(prefix_lens[b])
        path = [int(n) for n in accepted_nodes[b][:L + 1]]
        if path[0] != 0 or any(path[d] <= path[d - 1] for d in range(1, L + 1)):
            raise ValueError("accepted path must start at the root and increase")
        for d in range(1, L + 1):
            src = base + path[d]
            dst = base + d
            sb, ss = block_table[b][src // block_size], src % block_size
            db, ds = block_table[b][dst // block_size], dst % block_size
            k[db, :, ds, :] = k[sb, :, ss, :]
            v[db, :, ds, :] = v[sb, :, ss, :]
        new_lens[b] = base + L + 1
    return k, v, new_lens
