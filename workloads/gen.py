"""Seeded synthetic workloads for tree verification.

Every array is drawn from numpy's PCG64 through
``SeedSequence([seed, tag, stream])`` so that each kind of input (queries and
KV, logits, tree shape, draft tokens, prefix lengths, block placement) has a
stream of its own.  Nothing here verifies anything: this module only makes
inputs with the shapes and value distributions of the five layer-shaped
configurations (tiny, chain, EAGLE-style tree, Sequoia-scale tree, batched
serving) and of small custom cases used by the tests.

Layouts (the library's contract):
  q            [B, T, Hq, D]            bf16 bits (uint16) or float32
  k_cache/v_cache [num_blocks, Hkv, 16, D]  same element type as q
  block_table  [B, max_blocks] int32    logical page j of sequence b
  prefix_lens  [B] int32                committed tokens before the tree
  parent       [B, T] int32             parent[b][0] = -1, parent < child
  draft_tokens [B, T] int32             token of node i (entry 0 unused)
  target_logits[B, T, V] float32        row u: target logits after node u
  draft_probs  [B, T, V] float32        row u: draft distribution at node u
The K/V rows of tree node i sit at logical position prefix_lens[b] + i.
Slots of a sequence's last page past prefix+T are filled with NaN so that a
kernel that reads them shows up in the results.
"""
from __future__ import annotations

import heapq
import math
from dataclasses import dataclass, field

import numpy as np

BLOCK_SIZE = 16

CONFIG_NAMES = {
    0: "tiny",
    1: "chain",
    2: "eagle_tree",
    3: "sequoia_tree",
    4: "batched_serving",
}

# stream ids inside one workload's SeedSequence
_S_QKV, _S_LOGITS, _S_TREE, _S_TOKENS, _S_LENS, _S_BLOCKS = range(6)

_BF16_NAN = np.uint16(0x7FC0)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round finite float32 values to bfloat16 (round to nearest, ties to even); return the bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    one, half, sh = np.uint32(1), np.uint32(0x7FFF), np.uint32(16)
    return ((u + half + ((u >> sh) & one)) >> sh).astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns to float32."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def _rng(seed: int, tag: int, stream: int, sub: int = 0) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([int(seed), int(tag), int(stream), int(sub)]))


@dataclass
class Workload:
    name: str
    tag: int
    dtype: str  # "f32" or "bf16"
    B: int
    T: int
    Hq: int
    Hkv: int
    D: int
    V: int
    q: np.ndarray
    k_cache: np.ndarray
    v_cache: np.ndarray
    block_table: np.ndarray
    prefix_lens: np.ndarray
    parent: np.ndarray
    draft_tokens: np.ndarray
    target_logits: np.ndarray
    draft_probs: np.ndarray
    temperature: float
    without_replacement: bool
    seed: int = 0
    offset: int = 0
    block_size: int = BLOCK_SIZE
    info: dict = field(default_factory=dict)

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.D)

    @property
    def max_blocks(self) -> int:
        return int(self.block_table.shape[1])

    @property
    def num_blocks(self) -> int:
        return int(self.k_cache.shape[0])

    def as_f32(self, a: np.ndarray) -> np.ndarray:
        """Float32 view of q / k_cache / v_cache (widens bf16 bits exactly)."""
        return bf16_bits_to_f32(a) if self.dtype == "bf16" else a

    def summary(self) -> dict:
        return {
            "workload": self.name,
            "B": self.B, "T": self.T, "Hq": self.Hq, "Hkv": self.Hkv, "D": self.D,
            "V": self.V, "dtype": self.dtype,
            "prefix_lens": "U[%d,%d]" % (int(self.prefix_lens.min()), int(self.prefix_lens.max()))
            if self.B > 1 and self.prefix_lens.min() != self.prefix_lens.max()
            else int(self.prefix_lens[0]),
            "temperature": self.temperature,
            "without_replacement": bool(self.without_replacement),
        }


# ----------------------------------------------------------------------------
# tree shapes (parent arrays in topological order: parent[i] < i)
# ----------------------------------------------------------------------------

def _depth_list(parent) -> list:
    d = [0] * len(parent)
    for i in range(1, len(parent)):
        d[i] = d[parent[i]] + 1
    return d


def tree_chain(gamma: int) -> list:
    return [-1] + list(range(gamma))


def tree_random_recursive(n: int, max_depth: int, rng: np.random.Generator) -> list:
    """Node i picks its parent uniformly among earlier nodes shallower than max_depth."""
    parent = [-1]
    depth = [0]
    for i in range(1, n):
        cand = [j for j in range(i) if depth[j] < max_depth]
        p = int(cand[int(rng.integers(len(cand)))])
        parent.append(p)
        depth.append(depth[p] + 1)
    return parent


def sequoia_accept_profile(rng: np.random.Generator, rank_cap: int = 64) -> np.ndarray:
    """Acceptance by child rank: a_r = 0.8/r*(1+0.05*xi_r), xi ~ U(-1, 1), made non-increasing."""
    xi = rng.uniform(-1.0, 1.0, size=rank_cap)
    a = np.array([0.8 / r * (1.0 + 0.05 * xi[r - 1]) for r in range(1, rank_cap + 1)])
    return np.minimum.accumulate(a)


def tree_sequoia_profile(n: int, depth_cap: int, rng: np.random.Generator, rank_cap: int = 64):
    """Best-first tree on an acceptance-by-rank profile (the DP-style shape).

    The r-th child (r = 1, 2, ...) of any node has weight a_r (sequoia_accept_profile);
    a node's score is the product of the weights on its path.  The n highest-score
    nodes (depth <= depth_cap) are kept and numbered breadth first; children keep
    their rank order.  Returns (parent, rank, a) with rank[i] = 1-based child rank
    of node i.
    """
    a = sequoia_accept_profile(rng, rank_cap)
    # heap of (-score, creation, parent_creation, rank, depth, parent_score)
    heap = [(-1.0, 0, -1, 0, 0, 1.0)]
    created = 1
    kept = []  # (creation, parent_creation, rank, depth)
    while heap and len(kept) < n:
        negs, cid, pcid, rank, dep, ps = heapq.heappop(heap)
        kept.append((cid, pcid, rank, dep))
        s = -negs
        if dep < depth_cap:  # first child of the popped node
            heapq.heappush(heap, (-(s * a[0]), created, cid, 1, dep + 1, s))
            created += 1
        if pcid >= 0 and rank < rank_cap:  # next sibling of the popped node
            heapq.heappush(heap, (-(ps * a[rank]), created, pcid, rank + 1, dep, ps))
            created += 1
    # breadth-first renumbering: by depth, then parent's new index, then rank
    by_cid = {c[0]: c for c in kept}
    new_index = {}
    order = []
    level = [c for c in kept if c[3] == 0]
    while level:
        level.sort(key=lambda c: (new_index.get(c[1], -1), c[2]))
        for c in level:
            new_index[c[0]] = len(order)
            order.append(c)
        nxt_depth = level[0][3] + 1
        level = [c for c in kept if c[3] == nxt_depth]
    parent = [-1 if c[1] < 0 else new_index[c[1]] for c in order]
    rank = [c[2] for c in order]
    assert all(c[1] in by_cid or c[1] < 0 for c in kept)
    return parent, rank, a


# ----------------------------------------------------------------------------
# logits and draft distributions
# ----------------------------------------------------------------------------

def _draft_probs_from_logits(draft_logits: np.ndarray, tau_d: float) -> np.ndarray:
    """The synthetic drafter's distribution: softmax(draft_logits / tau_d), stored as float32."""
    z = draft_logits.astype(np.float64) / tau_d
    z -= z.max(axis=-1, keepdims=True)
    e = np.exp(z)
    e /= e.sum(axis=-1, keepdims=True)
    return e.astype(np.float32)


def _node_rows(rng: np.random.Generator, n: int, V: int, tau_d: float):
    """n rows of target logits ~ N(0, 2^2) and draft probs from target + N(0, 1)."""
    tl = (rng.standard_normal((n, V), dtype=np.float32) * np.float32(2.0)).astype(np.float32)
    dl = tl + rng.standard_normal((n, V), dtype=np.float32)
    return tl, _draft_probs_from_logits(dl, tau_d)


def _draw(rng: np.random.Generator, probs: np.ndarray) -> int:
    p = probs.astype(np.float64)
    p = p / p.sum()
    return int(rng.choice(p.shape[0], p=p))


def _draft_children(parent, rows_q, mode, rng):
    """Draft token for every non-root node from its parent's draft distribution.

    mode 'iid': each child independently ~ q_parent.
    mode 'without_replacement': the children of a node, in index order, are
    successive draws without replacement from q_parent.
    """
    T = len(parent)
    tok = np.zeros(T, dtype=np.int32)
    if mode == "iid":
        for i in range(1, T):
            tok[i] = _draw(rng, rows_q[parent[i]])
    elif mode == "without_replacement":
        for u in range(T):
            kids = [i for i in range(1, T) if parent[i] == u]
            if not kids:
                continue
            p = rows_q[u].astype(np.float64).copy()
            for c in kids:
                x = int(rng.choice(p.shape[0], p=p / p.sum()))
                tok[c] = x
                p[x] = 0.0
    else:
        raise ValueError(mode)
    return tok


def _eagle_tree(rng_rows, V, tau_d, depth=6, topk=4, n_keep=64):
    """Layer-wise top-k expansion of the highest-score nodes (EAGLE-style drafting).

    At each depth the `topk` best nodes of the layer (score = product of draft
    probabilities along the path) are expanded by the `topk` most probable
    tokens of their draft distribution.  The best deepest node and its
    ancestors are kept, the tree is filled to n_keep nodes by score and
    renumbered breadth first.  Returns parent, tokens, target rows, draft rows.
    """
    pool_parent = [-1]
    pool_tok = [0]
    pool_depth = [0]
    pool_score = [1.0]
    tl0, q0 = _node_rows(rng_rows, 1, V, tau_d)
    pool_tl = [tl0[0]]
    pool_q = [q0[0]]
    for d in range(depth):
        layer = [i for i in range(len(pool_parent)) if pool_depth[i] == d]
        layer.sort(key=lambda i: (-pool_score[i], i))
        for u in layer[:topk]:
            qu = pool_q[u].astype(np.float64)
            order = np.argsort(-qu, kind="stable")[:topk]
            for x in order:
                pool_parent.append(u)
                pool_tok.append(int(x))
                pool_depth.append(d + 1)
                pool_score.append(pool_score[u] * float(qu[x]))
                tl, q = _node_rows(rng_rows, 1, V, tau_d)
                pool_tl.append(tl[0])
                pool_q.append(q[0])
    n_pool = len(pool_parent)
    deepest = [i for i in range(n_pool) if pool_depth[i] == depth]
    best = min(deepest, key=lambda i: (-pool_score[i], i))
    keep = set()
    u = best
    while u >= 0:
        keep.add(u)
        u = pool_parent[u]
    for i in sorted(range(n_pool), key=lambda i: (-pool_score[i], i)):
        if len(keep) >= n_keep:
            break
        keep.add(i)
    assert all(pool_parent[i] in keep or i == 0 for i in keep)
    order = []
    new_index = {}
    level = [0]
    while level:
        for i in level:
            new_index[i] = len(order)
            order.append(i)
        level = [i for u in level for i in range(n_pool) if i in keep and pool_parent[i] == u]
    parent = [-1 if pool_parent[i] < 0 else new_index[pool_parent[i]] for i in order]
    tok = np.array([pool_tok[i] for i in order], dtype=np.int32)
    tl = np.stack([pool_tl[i] for i in order])
    q = np.stack([pool_q[i] for i in order])
    return parent, tok, tl, q


# ----------------------------------------------------------------------------
# paged KV placement
# ----------------------------------------------------------------------------

def _place_kv(seed, tag, lens_total, Hkv, D, dtype, block_table, num_blocks):
    """Fill the paged caches: logical position t of sequence b lives at
    cache[block_table[b][t // 16], :, t % 16, :].  Unused slots hold NaN.
    Sequence b draws its K and V from a stream of its own, so sequences can be
    generated on several threads with a deterministic result."""
    from concurrent.futures import ThreadPoolExecutor

    shape = (num_blocks, Hkv, BLOCK_SIZE, D)
    fill = _BF16_NAN if dtype == "bf16" else np.float32(np.nan)
    edt = np.uint16 if dtype == "bf16" else np.float32
    k = np.full(shape, fill, dtype=edt)
    v = np.full(shape, fill, dtype=edt)

    def one(b):
        n = lens_total[b]
        pages = -(-n // BLOCK_SIZE)
        rng = _rng(seed, tag, _S_QKV, 1 + b)
        for cache in (k, v):
            vals = rng.standard_normal((n, Hkv, D), dtype=np.float32)
            if dtype == "bf16":
                vals = f32_to_bf16_bits(vals)
            pad = np.full((pages * BLOCK_SIZE, Hkv, D), fill, dtype=edt)
            pad[:n] = vals
            cache[block_table[b, :pages]] = pad.reshape(pages, BLOCK_SIZE, Hkv, D).transpose(0, 2, 1, 3)

    with ThreadPoolExecutor(max_workers=8) as ex:
        list(ex.map(one, range(len(lens_total))))
    return k, v


def _block_tables(lens_total, shuffle, rng, extra_blocks=0):
    pages = [-(-n // BLOCK_SIZE) for n in lens_total]
    mb = max(max(pages), 1)
    total = sum(pages) + extra_blocks
    ids = np.arange(total, dtype=np.int32)
    if shuffle:
        ids = rng.permutation(total).astype(np.int32)
    table = np.zeros((len(lens_total), mb), dtype=np.int32)
    pos = 0
    for b, p in enumerate(pages):
        table[b, :p] = ids[pos:pos + p]
        pos += p
    return table, total


# ----------------------------------------------------------------------------
# workloads
# ----------------------------------------------------------------------------

def make_workload(*, name="custom", tag=100, B=1, Hq=2, Hkv=2, D=64, dtype="f32", V=16,
                  prefix=16, tree="fixed", parent=None, T=None, gamma=None, max_depth=5,
                  draft_mode="iid", temperature=1.0, draft_temperature=None,
                  without_replacement=False, shuffle_blocks=False, extra_blocks=0,
                  seed=0, offset=0, with_kv=True) -> Workload:
    """General builder.  `prefix` is an int (same for all) or a (lo, hi) range
    drawn uniformly per sequence, or an explicit list of lengths."""
    tau_d = float(temperature if draft_temperature is None else draft_temperature)
    if tau_d <= 0:
        tau_d = 1.0
    r_lens = _rng(seed, tag, _S_LENS)
    if isinstance(prefix, (list, np.ndarray)):
        lens = np.asarray(prefix, dtype=np.int32)
        assert lens.shape == (B,)
    elif isinstance(prefix, tuple):
        lens = r_lens.integers(prefix[0], prefix[1] + 1, size=B).astype(np.int32)
    else:
        lens = np.full(B, int(prefix), dtype=np.int32)

    r_tree = _rng(seed, tag, _S_TREE)
    r_rows = _rng(seed, tag, _S_LOGITS)
    r_tok = _rng(seed, tag, _S_TOKENS)
    parents, toks, tls, qs = [], [], [], []
    info = {}
    eagle = {}
    if tree == "eagle":  # each sequence has its own stream: build them on threads
        from concurrent.futures import ThreadPoolExecutor

        def one(b):
            return _eagle_tree(_rng(seed, tag, _S_LOGITS, b + 1), V, tau_d,
                               depth=max_depth, topk=4, n_keep=T or 64)
        with ThreadPoolExecutor(max_workers=8) as ex:
            eagle = dict(enumerate(ex.map(one, range(B))))
    for b in range(B):
        if tree == "eagle":
            p, tk, tl, q = eagle[b]
        else:
            if tree == "fixed":
                p = list(parent)
            elif tree == "chain":
                p = tree_chain(gamma)
            elif tree == "random":
                p = tree_random_recursive(T, max_depth, r_tree)
            elif tree == "sequoia":
                p, rank, a_rank = tree_sequoia_profile(T, max_depth, r_tree)
                if b == 0:
                    info["accept_profile"] = a_rank.tolist()
            else:
                raise ValueError(tree)
            tl, q = _node_rows(r_rows, len(p), V, tau_d)
            tk = _draft_children(p, q, draft_mode, r_tok)
        parents.append(p)
        toks.append(tk)
        tls.append(tl)
        qs.append(q)
    Tn = len(parents[0])
    assert all(len(p) == Tn for p in parents)
    parent_a = np.array(parents, dtype=np.int32)
    tok_a = np.stack(toks).astype(np.int32)
    tl_a = np.stack(tls).astype(np.float32)
    q_a = np.stack(qs).astype(np.float32)
    widths = np.bincount(np.array(_depth_list(parents[0])))
    info["depth"] = int(len(widths) - 1)
    info["width_profile"] = widths.tolist()

    lens_total = [int(n) + Tn for n in lens]
    r_blk = _rng(seed, tag, _S_BLOCKS)
    table, num_blocks = _block_tables(lens_total, shuffle_blocks, r_blk, extra_blocks)
    r_qkv = _rng(seed, tag, _S_QKV)
    qv = r_qkv.standard_normal((B, Tn, Hq, D), dtype=np.float32)
    if dtype == "bf16":
        qv = f32_to_bf16_bits(qv)
    if with_kv:
        kc, vc = _place_kv(seed, tag, lens_total, Hkv, D, dtype, table, num_blocks)
    else:
        kc = vc = None
    return Workload(name=name, tag=tag, dtype=dtype, B=B, T=Tn, Hq=Hq, Hkv=Hkv, D=D, V=V,
                    q=qv, k_cache=kc, v_cache=vc, block_table=table, prefix_lens=lens,
                    parent=parent_a, draft_tokens=tok_a, target_logits=tl_a, draft_probs=q_a,
                    temperature=float(temperature), without_replacement=bool(without_replacement),
                    seed=seed, offset=offset, info=info)


def make_config(cfg_id: int, seed: int = 0, **over) -> Workload:
    """The five layer-shaped configurations (see the module docstring)."""
    if cfg_id == 0:
        kw = dict(B=1, Hq=2, Hkv=2, D=64, dtype="f32", V=1000, prefix=128, tree="fixed",
                  parent=[-1, 0, 0, 1, 1, 2, 3, 4], draft_mode="iid", temperature=1.0)
    elif cfg_id == 1:
        kw = dict(B=1, Hq=40, Hkv=40, D=128, dtype="bf16", V=32000, prefix=2048, tree="chain",
                  gamma=4, draft_mode="iid", temperature=1.0)
    elif cfg_id == 2:
        kw = dict(B=8, Hq=32, Hkv=8, D=128, dtype="bf16", V=128256, prefix=4096, tree="eagle",
                  T=64, max_depth=6, temperature=0.7)
    elif cfg_id == 3:
        kw = dict(B=1, Hq=64, Hkv=8, D=128, dtype="bf16", V=32000, prefix=8192, tree="sequoia",
                  T=256, max_depth=10, draft_mode="without_replacement", temperature=0.6,
                  without_replacement=True)
    elif cfg_id == 4:
        kw = dict(B=64, Hq=32, Hkv=8, D=128, dtype="bf16", V=32000, prefix=(512, 16384),
                  tree="random", T=16, max_depth=5, draft_mode="iid", temperature=1.0,
                  shuffle_blocks=True)
    else:
        raise ValueError("config id must be 0..4")
    kw.update(over)
    return make_workload(name=CONFIG_NAMES[cfg_id], tag=cfg_id, seed=seed, **kw)


def sub_batch(w: Workload, seqs) -> Workload:
    """The sequences `seqs` of a workload as a workload of their own, with a
    cache that holds only their pages (block table renumbered in the same
    order, so each page keeps its contents).  Used to run a bounded sample of
    a large batch through a slow reference."""
    seqs = [int(b) for b in seqs]
    table = w.block_table[seqs]
    lens_total = [int(w.prefix_lens[b]) + w.T for b in seqs]
    pages = [-(-n // BLOCK_SIZE) for n in lens_total]
    used = np.concatenate([table[i, :p] for i, p in enumerate(pages)])
    new_table = np.zeros((len(seqs), max(pages)), dtype=np.int32)
    pos = 0
    for i, p in enumerate(pages):
        new_table[i, :p] = np.arange(pos, pos + p, dtype=np.int32)
        pos += p
    kc = None if w.k_cache is None else np.ascontiguousarray(w.k_cache[used])
    vc = None if w.v_cache is None else np.ascontiguousarray(w.v_cache[used])
    return Workload(name=w.name, tag=w.tag, dtype=w.dtype, B=len(seqs), T=w.T, Hq=w.Hq, Hkv=w.Hkv, D=w.D, V=w.V,
                    q=w.q[seqs], k_cache=kc, v_cache=vc, block_table=new_table,
                    prefix_lens=w.prefix_lens[seqs].copy(), parent=w.parent[seqs], draft_tokens=w.draft_tokens[seqs],
                    target_logits=w.target_logits[seqs], draft_probs=w.draft_probs[seqs],
                    temperature=w.temperature, without_replacement=w.without_replacement, seed=w.seed,
                    offset=w.offset, info=dict(w.info))
