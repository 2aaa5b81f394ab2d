"""The library's calls under HIP graph capture, the way the benchmark and a
serving loop run them: the K/V write (without queries, so that a replay
repeats the same writes), the verify attention, the top-k / top-p truncation
out of place, and the sampler with compaction, captured once on the chain
workload and replayed several times with eager work and synchronisations in
between.  Every replay must reproduce the eager outputs bit for bit (the
calls are deterministic and no call records a memset into the graph)."""
import numpy as np
import pytest
import torch

import tree_verify_attention_masked_amd as stv
from helpers import dev_kv
from workloads import make_config

pytestmark = pytest.mark.gpu


def test_verify_path_replays_match_eager():
    w = make_config(1)
    print(f"[graph] {w.name} B={w.B} T={w.T}", flush=True)
    dev = "cuda"
    up = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    q, k, v = dev_kv(w, w.q), dev_kv(w, w.k_cache), dev_kv(w, w.v_cache)
    bt, lens, parent, tok = up(w.block_table), up(w.prefix_lens), up(w.parent), up(w.draft_tokens)
    logits, probs = up(w.target_logits), up(w.draft_probs)
    rng = np.random.default_rng(5)
    k_new = torch.from_numpy(rng.normal(size=(w.B, w.T, w.Hkv, w.D)).astype(np.float32)).to(dev).to(k.dtype)
    v_new = torch.from_numpy(rng.normal(size=(w.B, w.T, w.Hkv, w.D)).astype(np.float32)).to(dev).to(k.dtype)
    ws_a = stv.spec_tree_attn_workspace_size(w.B, w.T, w.Hq, w.Hkv, w.D, w.block_table.shape[1], stv.SPEC_BF16)
    attn_ws = torch.zeros(max(ws_a, 1), dtype=torch.uint8, device=dev)
    rej_ws = torch.zeros(int(stv.load_library().spec_tree_reject_workspace_size(w.B, w.T, w.V)), dtype=torch.uint8,
                         device=dev)
    out = torch.empty_like(q)
    trunc = torch.empty_like(logits)
    res = [torch.empty((w.B, w.T), dtype=torch.int32, device=dev) for _ in range(2)] + \
          [torch.empty((w.B,), dtype=torch.int32, device=dev) for _ in range(2)]
    status = torch.zeros(w.B, dtype=torch.int32, device=dev)

    def step():
        stv.spec_tree_kv_write(k_new, v_new, None, k, v, bt, lens, parent, 10000.0, status=status)
        stv.spec_tree_attn(q, k, v, bt, lens, parent, scale=w.scale, out=out, status=status,
                           workspace=attn_ws if ws_a else None)
        stv.spec_tree_truncate(logits, w.temperature, 50, 0.9, out=trunc, status=status)
        stv.spec_tree_reject_compact(trunc, probs, tok, parent, w.temperature, k, v, bt, lens, w.without_replacement,
                                     w.seed, w.offset, accepted_nodes=res[0], out_tokens=res[1], num_accepted=res[2],
                                     new_lens=res[3], status=status, workspace=rej_ws)

    def snapshot():
        torch.cuda.synchronize()
        return [t.cpu().clone() for t in (out, trunc, k, v, *res)]

    step()
    eager = snapshot()
    assert int(status.abs().sum()) == 0, status.tolist()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            step()
    torch.cuda.current_stream().wait_stream(s)
    for rep in range(4):
        for t in (out, trunc, *res):  # poison the outputs so that a skipped write cannot pass
            t.fill_(-1) if t.dtype == torch.int32 else t.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        got = snapshot()
        for name, a, b in zip(("out", "truncated", "k_cache", "v_cache", "accepted", "tokens", "L", "new_lens"),
                              got, eager):
            assert torch.equal(a.view(torch.uint8) if a.dtype == torch.bfloat16 else a,
                               b.view(torch.uint8) if b.dtype == torch.bfloat16 else b) or \
                (a.is_floating_point() and torch.equal(torch.nan_to_num(a), torch.nan_to_num(b))), \
                f"replay {rep}: {name} differs from the eager call"
        _ = torch.randn(1024, device=dev).sum()  # eager work between replays
    assert int(status.abs().sum()) == 0, status.tolist()
