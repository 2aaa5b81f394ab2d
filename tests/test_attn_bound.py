"""The bf16 rounding bound of the GPU parity tests, checked on the CPU.

Besides the stated tolerance, bf16 attention outputs must meet a bound derived
from the arithmetic (helpers.BF16_U2, derived there).  It must accept everything bf16
rounding can do to a correct kernel -- the oracle output rounded to bf16, and a
model that rounds the probabilities to bf16 before the P.V product -- and must
reject the mistakes it is there to catch, even with thousands of keys per row
where their effect averages down: a row sum taken from one of the four lanes
that share a row (times four), a row rescaled by 5 %, the heaviest key dropped.
"""
import numpy as np
import pytest

from helpers import assert_attn_close, oracle_attn
from workloads import bf16_bits_to_f32, f32_to_bf16_bits, make_workload


def _bf16(x):
    return bf16_bits_to_f32(f32_to_bf16_bits(np.asarray(x, dtype=np.float32))).astype(np.float64)


def _rows(w):
    """Per (b, node, head): scores, probabilities relative to the max, values,
    over the keys the row sees (prefix + ancestors-or-self), in logical order."""
    out = {}
    kc = bf16_bits_to_f32(w.k_cache).astype(np.float64)
    vc = bf16_bits_to_f32(w.v_cache).astype(np.float64)
    G = w.Hq // w.Hkv
    for b in range(w.B):
        L = int(w.prefix_lens[b])
        n = L + w.T
        pos = np.arange(n)
        blk = w.block_table[b][pos // 16]
        for i in range(w.T):
            anc, j = set(), i
            while j >= 0:
                anc.add(j)
                j = int(w.parent[b][j])
            keep = np.array([t < L or (t - L) in anc for t in range(n)])
            for h in range(w.Hq):
                g = h // G
                K = kc[blk, g, pos % 16][keep]
                V = vc[blk, g, pos % 16][keep]
                q = bf16_bits_to_f32(w.q[b, i, h]).astype(np.float64)
                s = K @ q * w.scale
                p = np.exp(s - s.max())
                out[(b, i, h)] = (pos[keep], p, V)
    return out


@pytest.fixture(scope="module")
def case():
    w = make_workload(tag=520, B=1, Hq=4, Hkv=1, D=128, dtype="bf16", V=8, prefix=[2000], tree="random", T=6,
                      max_depth=3)
    ref, ref_abs = oracle_attn(w)
    return w, ref, ref_abs, _rows(w)


def _assemble(w, rows, f):
    out = np.zeros((w.B, w.T, w.Hq, w.D))
    for (b, i, h), (pos, p, V) in rows.items():
        out[b, i, h] = f(pos, p, V)
    return out


def test_bf16_rounding_is_inside_the_bound(case):
    w, ref, ref_abs, rows = case
    assert_attn_close(_bf16(ref), ref, "bf16", "rounded output", ref_abs)
    got = _assemble(w, rows, lambda pos, p, V: _bf16((_bf16(p) @ V) / p.sum()))
    assert_attn_close(got, ref, "bf16", "bf16 probabilities", ref_abs)


@pytest.mark.parametrize("mistake", ["one_lane_row_sum", "rescaled_row", "dropped_key"])
def test_mistakes_are_outside_the_bound(case, mistake):
    w, ref, ref_abs, rows = case
    if mistake == "one_lane_row_sum":
        # keys 4q..4q+3 of every 16-key page sit in lane group q; use group 0's share times four
        f = lambda pos, p, V: (p @ V) / (4.0 * p[(pos % 16) // 4 == 0].sum())
    elif mistake == "rescaled_row":
        f = lambda pos, p, V: 1.05 * (p @ V) / p.sum()
    else:
        def f(pos, p, V):
            p = p.copy()
            p[np.argmax(p)] = 0.0
            return (p @ V) / p.sum()
    got = _assemble(w, rows, f)
    with pytest.raises(AssertionError):
        assert_attn_close(got, ref, "bf16", mistake, ref_abs)
