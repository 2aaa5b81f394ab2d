"""Benchmark of one tree-verification step on one MI355X.

A step = spec_tree_write_attn (the tree's K/V rows into the paged cache,
rotated for their tree positions, and the tree-masked attention; spec_tree_attn
for the fp32 configuration) -> spec_tree_reject_compact (tree rejection
sampling, then compaction of the KV cache along the accepted path, in one
launch) over one batch of the synthetic workload.  Default workload: batched serving, the largest
configuration that fits one GPU (64 sequences, 32 query / 8 kv heads, head dim
128, bf16 paged KV with a shuffled block table, prefixes uniform in
[512, 16384], a random 16-node tree of depth <= 5 per sequence, vocabulary
32000, temperature 1).  Metric: verified tree tokens per second = B * T / step
time.  The chain workload (a Llama-2-13B-shaped layer, chain of 4 drafts) is
measured as well and reported under `extra`.

Inputs are resident in HBM before timing starts.  Several copies of every
input are cycled where they fit, so that consecutive steps do not find their
data in the 256 MB MALL / L2.  Steps are replayed from HIP graphs: one graph
holds G consecutive step slots, slot j on input copy j % R with its own Philox
offset (offset + j), so consecutive steps take different walks; the timed
region holds only GPU work and one host launch per G steps; the K timed steps
are bracketed by torch.cuda.synchronize().  Per-kernel average durations come
from HIP events around graphs that repeat one call many times on the current
stream (the stream the kernels run on).  `step_us` gives the spread (p10, p50,
p90) of 100 single-step replays, each bracketed by events.

The line also carries the same step without the write (`without_kv_write`) and
the step against a truncated target (`truncated_target`: top-k 50 then top-p
0.9, applied inside the sampler by spec_tree_reject_truncated to the rows its
walk visits; `separate_pass` beside it: the same target truncated by
spec_tree_truncate over every row before the plain sampler).  Its `kernels` also time spec_tree_kv_write (the write as a launch
of its own), spec_tree_truncate (the same truncation as a separate pass over
every target row, out of place) and the truncating sampler; none of these is
part of the timed step, whose target is not truncated.

Prints ONE JSON line on stdout; progress goes to stderr.

`roofline` covers the dominant (longest) kernel of the step; `step_roofline`
the whole step (algorithmic bytes of attention, walked logit rows and moved KV
rows over the step time).  `roofline.traffic` comes from the committed
rocprofv3 counter summary (profiles/pmc_<workload>.md, FETCH_SIZE and
WRITE_SIZE per dispatch, scaled by what the same counters read for a plain
1 GiB device copy); it is null when that summary was taken from other kernel
sources than the ones built now.  `--summarize trace|pmc|sq DIR...` turns
rocprofv3 CSV output into those summaries (host only, no GPU).
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import math
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, published
BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix, published
METRIC = "verified tree tokens/sec at 1 MI355X"
TRUNC_K, TRUNC_P = 50, 0.9  # the truncated target measured beside the step: top-k 50, then top-p 0.9


KERNEL_KEYS = (("tree_write_attn", ("attn_tile_kernel<1, true>", "attn_tile_kernel<2, true>", "attn_stream_kernel<1, 3, true>")), ("tree_attn", ("attn_",)), ("tree_reject_compact", ("reject",)), ("kv_compact", ("kv_compact",)),
               ("tree_kv_write", ("kv_write",)), ("tree_truncate", ("truncate_kernel",)))
CALIB_BYTES = 256 << 20  # the calibration copy reads and writes this many bytes
CALIB_BYTES_BIG = 1 << 30  # a second calibration copy, four times the 256 MB MALL


def log(*a):
    print(*a, file=sys.stderr, flush=True)


KERNEL_SOURCES = {  # the sources each kernel key is built from (with common.h and the C-ABI header)
    "tree_write_attn": ("attn_bf16.hip", "attn_stream.hip", "rope_dev.h"),
    "tree_attn": ("attn_bf16.hip", "attn_stream.hip", "attn_f32.hip"),
    "tree_reject_compact": ("reject.hip", "compact_dev.h"),
    "kv_compact": ("compact.hip", "compact_dev.h"),
    "tree_kv_write": ("kv_write.hip",),
    "tree_truncate": ("truncate.hip",),
}


def kernel_source_hash(kernel=None):
    """sha256 over the HIP sources and headers the library is built from (or those of one kernel key)."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "tree_verify_attention_masked_amd", "csrc")
    if kernel is None:
        files = sorted(glob.glob(os.path.join(csrc, "*")))
    else:
        files = [os.path.join(csrc, f) for f in sorted(KERNEL_SOURCES[kernel] + ("common.h",))]
    for f in files + [os.path.join(ROOT, "include", "spectree.h")]:
        h.update(os.path.basename(f).encode())
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def kernel_key(name):
    low = name.lower()
    for key, pats in KERNEL_KEYS:
        if any(p in low for p in pats):
            return key
    return None


def read_csvs(d, suffix):
    rows = []
    for f in glob.glob(os.path.join(d, "**", f"*{suffix}"), recursive=True):
        with open(f, newline="") as fh:
            rows.extend(csv.DictReader(fh))
    return rows


def summarize(kind, dirs, workload):
    """Markdown summary of rocprofv3 output (kernel trace stats, or FETCH_SIZE / WRITE_SIZE runs)."""
    out = []
    if kind == "trace":
        rows = read_csvs(dirs[0], "kernel_stats.csv")
        out.append("| kernel | calls | average duration (us) | total (us) | share |")
        out.append("|---|---|---|---|---|")
        for r in sorted(rows, key=lambda r: -float(r.get("TotalDurationNs", 0))):
            name = r.get("Name", "")
            avg = float(r.get("AverageNs", 0)) / 1e3
            out.append(f"| `{name[:90]}` | {r.get('Calls')} | {avg:.2f} | {float(r.get('TotalDurationNs', 0)) / 1e3:.1f} | "
                       f"{float(r.get('Percentage', 0)):.1f}% |")
        return "\n".join(out)
    if kind == "sq":
        return summarize_sq(dirs, workload)
    # pmc: dirs = [fetch_dir, write_dir]
    per = {}
    calib = {}  # counter -> [(dispatch id, KiB)] of the calibration copies, in dispatch order
    for d, counter in zip(dirs, ("FETCH_SIZE", "WRITE_SIZE")):
        disp = {}
        for r in read_csvs(d, "counter_collection.csv"):
            if r.get("Counter_Name") != counter:
                continue
            key = (int(r.get("Dispatch_Id", 0)), r.get("Kernel_Name", ""))
            disp[key] = disp.get(key, 0.0) + float(r.get("Counter_Value", 0))
        for (did, name), kib in sorted(disp.items()):
            k = kernel_key(name)
            if k:
                per.setdefault(k, {}).setdefault(counter, []).append(kib)
            elif "copy" in name.lower() and kib > 0.1 * CALIB_BYTES / 1024:
                calib.setdefault(counter, []).append(kib)
    # the first copy moves 256 MiB (the size of the MALL), the second 1 GiB; the
    # larger one scales the counters (its data cannot sit in the MALL)
    sizes = (CALIB_BYTES, CALIB_BYTES_BIG)
    by_size = {c: {f"{n >> 20}MiB": round(kib * 1024 / n, 4) for kib, n in zip(v, sizes)} for c, v in calib.items()}
    factors = {c: (v[-1] * 1024 / sizes[len(v) - 1] if v else None) for c, v in calib.items()}
    res = {"workload": workload, "source_sha256": kernel_source_hash(), "calibration": factors,
           "calibration_by_copy_size": by_size, "kernels": {}}
    out.append("| kernel | dispatches | FETCH_SIZE KiB/dispatch | WRITE_SIZE KiB/dispatch | HBM bytes/launch (scaled) |")
    out.append("|---|---|---|---|---|")
    for k, cs in sorted(per.items()):
        f = float(np.mean(cs.get("FETCH_SIZE", [0.0])))
        wv = float(np.mean(cs.get("WRITE_SIZE", [0.0])))
        ff, fw = factors.get("FETCH_SIZE") or 1.0, factors.get("WRITE_SIZE") or 1.0
        traffic = f * 1024 / ff + wv * 1024 / fw
        res["kernels"][k] = {"fetch_kib": round(f, 1), "write_kib": round(wv, 1), "traffic_bytes": int(traffic),
                             "source_sha256": kernel_source_hash(k)}
        out.append(f"| {k} | {len(cs.get('FETCH_SIZE', []))} | {f:.1f} | {wv:.1f} | {traffic / 1e6:.3f} MB |")
    out.append("")
    out.append(f"Calibration (plain device copies; counter KiB x 1024 / bytes copied): {json.dumps(by_size)}; "
               f"scaled by the largest copy: FETCH_SIZE {factors.get('FETCH_SIZE')}, "
               f"WRITE_SIZE {factors.get('WRITE_SIZE')}.")
    out.append("")
    out.append("```json")
    out.append(json.dumps(res))
    out.append("```")
    return "\n".join(out)


SIMDS = 1024  # MI355X: 256 compute units x 4 SIMDs
DIES = 8  # accelerator dies (XCDs); GRBM_GUI_ACTIVE counts on each


def summarize_sq(dirs, workload):
    """Markdown summary of rocprofv3 --pmc runs of SQ / GRBM counters: per kernel, each counter
    summed over its instances (shader engines, dies) per dispatch -- rocprofv3's CSV already holds
    that sum -- and averaged over dispatches, with MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / (kernel
    cycles x SIMDs), the kernel's cycles being GRBM_GUI_ACTIVE per die (its sum over the dies / 8:
    rocprofv3's own MFMA-utilisation expression takes the largest die), and wait = SQ_WAIT_ANY /
    SQ_WAVE_CYCLES (wave cycles spent waiting on a counter or a dependency)."""
    per = {}  # kernel key -> counter -> [per-dispatch value]
    for d in dirs:
        disp = {}
        for r in read_csvs(d, "counter_collection.csv"):
            k = kernel_key(r.get("Kernel_Name", ""))
            if not k:
                continue
            c = r.get("Counter_Name")
            key = (k, c, int(r.get("Dispatch_Id", 0)))
            v = float(r.get("Counter_Value", 0))
            disp[key] = disp.get(key, 0.0) + v
        for (k, c, _), v in disp.items():
            per.setdefault(k, {}).setdefault(c, []).append(v)
    res = {"workload": workload, "kernels": {}}
    out = ["| kernel | counter | dispatches | mean per dispatch |", "|---|---|---|---|"]
    for k, cs in sorted(per.items()):
        means = {c: float(np.mean(v)) for c, v in cs.items()}
        for c in sorted(means):
            out.append(f"| {k} | {c} | {len(cs[c])} | {means[c]:.4g} |")
        derived = {}
        if "SQ_VALU_MFMA_BUSY_CYCLES" in means and means.get("GRBM_GUI_ACTIVE"):
            derived["kernel_cycles"] = means["GRBM_GUI_ACTIVE"] / DIES
            derived["mfma_busy"] = means["SQ_VALU_MFMA_BUSY_CYCLES"] / (derived["kernel_cycles"] * SIMDS)
        if "SQ_WAIT_ANY" in means and means.get("SQ_WAVE_CYCLES"):
            derived["wait_any"] = means["SQ_WAIT_ANY"] / means["SQ_WAVE_CYCLES"]
        if "SQ_WAIT_INST_ANY" in means and means.get("SQ_WAVE_CYCLES"):
            derived["wait_inst_issue"] = means["SQ_WAIT_INST_ANY"] / means["SQ_WAVE_CYCLES"]
        if "SQ_INSTS_VALU_MFMA_MOPS_BF16" in means:
            derived["bf16_mfma_flops"] = means["SQ_INSTS_VALU_MFMA_MOPS_BF16"] * 512
        res["kernels"][k] = {"means": {c: round(v, 1) for c, v in means.items()},
                             "derived": {c: round(v, 4) for c, v in derived.items()},
                             "source_sha256": kernel_source_hash(k)}
    out += ["", "```json", json.dumps(res), "```"]
    return "\n".join(out)


def committed_traffic(workload, kernel):
    """HBM bytes per launch of `kernel` from profiles/pmc_<workload>.md, if taken from that kernel's current sources."""
    f = os.path.join(ROOT, "profiles", f"pmc_{workload}.md")
    if not os.path.exists(f):
        return None
    m = re.search(r"```json\n(.*?)\n```", open(f).read(), re.S)
    if not m:
        return None
    d = json.loads(m.group(1))
    k = d.get("kernels", {}).get(kernel)
    if not k or k.get("source_sha256") != kernel_source_hash(kernel):
        return None
    return int(k["traffic_bytes"])


def depths(parent_row):
    d = [0] * len(parent_row)
    for i in range(1, len(parent_row)):
        d[i] = d[parent_row[i]] + 1
    return d


def attn_work(w):
    elt = 2 if w.dtype == "bf16" else 4
    kv = sum((int(L) + w.T) for L in w.prefix_lens) * w.Hkv * w.D * elt * 2
    qo = 2 * w.B * w.T * w.Hq * w.D * elt
    pairs = sum(w.T * int(L) + sum(dd + 1 for dd in depths(w.parent[b])) for b, L in enumerate(w.prefix_lens))
    return kv + qo, 4.0 * w.Hq * w.D * pairs


def rope_theta(w):
    """Rotary base of the layer a workload follows: Llama-3 (vocabulary 128256) 500000, else Llama-2's 10000."""
    return 500000.0 if w.V == 128256 else 10000.0


def write_bytes(w):
    """Algorithmic bytes the tree's K/V write adds to a step: the nodes' new K and V rows read, and written
    into the cache (the queries are read once either way, counted with the attention)."""
    elt = 2 if w.dtype == "bf16" else 4
    return 4 * w.B * w.T * w.Hkv * w.D * elt


def reject_bytes(w, nacc, stop_rejections):
    """Bytes the walk needs: target-logit rows of the visited nodes, plus the
    draft row of a stop node whose residual had to be formed."""
    return sum((int(L) + 1) * w.V * 4 + (w.V * 4 if stop_rejections[b] else 0) for b, L in enumerate(nacc))


def compact_bytes(w, acc, nacc):
    elt = 2 if w.dtype == "bf16" else 4
    moved = 0
    for b, L in enumerate(nacc):
        path = acc[b][:int(L) + 1]
        moved += sum(1 for d, n in enumerate(path) if n != d)
    return moved * w.Hkv * w.D * elt * 2 * 2  # K and V, read + write


def cpu_baseline(w, budget_s, theta=None, max_seqs=8):
    """The oracle (as it stands) on the same workload, timed on the host cores.

    A batch of more than `max_seqs` sequences is sampled: the first `max_seqs`
    of them, with their own pages (the oracle's compaction copies the whole
    cache it is given).  The value is verified tree tokens per second of the
    oracle's step over the sample -- the tree's K/V write with rotation (when
    `theta` is given, as in the timed step), attention, walk, compaction --
    repeated until `budget_s` seconds have passed."""
    import oracle
    from workloads import sub_batch

    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = 1
    sample = w if w.B <= max_seqs else sub_batch(w, range(max_seqs))
    from workloads.gen import f32_to_bf16_bits

    rng = np.random.default_rng(7)
    kv_new = [rng.standard_normal((sample.B, sample.T, sample.Hkv, sample.D), dtype=np.float32) for _ in range(2)]
    if sample.dtype == "bf16":  # the oracle reads every input in the sample's storage type
        kv_new = [f32_to_bf16_bits(x) for x in kv_new]
    steps = 0
    t0 = time.perf_counter()
    while True:
        if theta is None:
            q, kc, vc, dt = sample.q, sample.k_cache, sample.v_cache, sample.dtype
        else:  # fp64 rows in, fp64 caches out
            q, kc, vc = oracle.tree_kv_write(kv_new[0], kv_new[1], sample.q, sample.k_cache, sample.v_cache,
                                             sample.block_table, sample.prefix_lens, sample.parent, theta,
                                             dtype=sample.dtype)
            dt = "f64"
        oracle.tree_attention(q, kc, vc, sample.block_table, sample.prefix_lens, sample.parent, sample.scale,
                              dtype=dt)
        r = oracle.tree_reject(sample.target_logits, sample.draft_probs, sample.draft_tokens, sample.parent,
                               sample.temperature, sample.without_replacement, sample.seed, steps)
        oracle.kv_compact(kc, vc, sample.block_table, sample.prefix_lens, r["accepted_nodes"], r["num_accepted"])
        steps += 1
        el = time.perf_counter() - t0
        if el >= budget_s or steps >= 200:
            break
    what = (f"sequences 0-{sample.B - 1} of the {w.B}-sequence batch" if sample is not w else "the whole batch")
    return {"value": sample.B * sample.T * steps / el, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{steps} steps over {what} (fp64 NumPy {'K/V write with rotation + ' if theta else ''}"
                      f"attention + walk + compaction), {el:.1f} s, "
                      f"{len(os.sched_getaffinity(0))} host cores visible"}


def capture_graph(fn_list):
    """A HIP graph of the calls in fn_list, captured on a side stream."""
    import torch

    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            for fn in fn_list:
                fn()
    torch.cuda.current_stream().wait_stream(s)
    return g


def seconds_per_call(fn, copies, reps, calls):
    """Average duration of fn(copy): HIP events on the current stream around
    replays of one graph of `reps` back-to-back calls cycling over the copies,
    about `calls` calls in all."""
    import torch

    g = capture_graph([lambda c=copies[i % len(copies)]: fn(c) for i in range(reps)])
    g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    rounds = max(1, calls // reps)
    e0.record()
    for _ in range(rounds):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e-3 / (rounds * reps)


SWEEP_SHAPES = (
    # name, layer shape of the configuration it follows, tree builder, tree sizes, prefix lengths
    ("sequoia_shape", 3, dict(), (1, 2, 4, 8, 16, 32, 64, 128, 256, 384, 512), (1024, 4096, 8192)),
    ("eagle_shape", 2, dict(tree="random"), (1, 2, 4, 8, 16, 32, 64, 128, 256, 512), (1024, 4096)),
)


def sweep():
    """Verify cost against tree size and prefix length (one JSON line per point):
    the layer shapes of the Sequoia-scale configuration (B1, 64 q / 8 kv heads,
    V 32000, tau 0.6, without replacement, Sequoia-profile trees of depth <= 10)
    and of the EAGLE-style one (B8, 32 q / 8 kv heads, V 128256, tau 0.7, random
    trees of depth <= 6), T from 1 to 512, timed per call as in the main run
    (graphs of back-to-back calls over input copies that together exceed the
    256 MB MALL where memory allows).  Each point times the attention and the
    sampler with compaction (the step), and the tree K/V write that precedes them
    (reported on its own), and spec_tree_write_attn, the write and the attention
    in one launch (the step with the write: it and the sampler with compaction).
    On the Sequoia shape each point also carries the
    expected tokens one step generates with the Sequoia-optimal tree of that size
    and depth bound for the generator's acceptance-by-rank vector
    (spec_sequoia_tree), and so the expected generated tokens per second of
    verification: the quantity the tree size is chosen by."""
    import torch

    import tree_verify_attention_masked_amd as stv
    from workloads import make_config

    lib = stv.load_library()
    dev = torch.device("cuda:0")
    for name, cfg, over, Ts, prefixes in SWEEP_SHAPES:
        for L in prefixes:
            for T in Ts:
                depth_cap = 10 if cfg == 3 else 6
                w = make_config(cfg, T=T, prefix=L, max_depth=min(depth_cap, max(T - 1, 0)), **over)
                log(f"[sweep] {name} T={T} prefix={L}")

                def up(a, kv=False):
                    t = torch.from_numpy(np.ascontiguousarray(a))
                    if kv:
                        t = t.view(torch.int16).view(torch.bfloat16)
                    return t.to(dev)

                per_copy = w.k_cache.nbytes * 2 + w.q.nbytes + w.target_logits.nbytes + w.draft_probs.nbytes
                R = max(1, min(8, math.ceil(512e6 / per_copy)))
                bt, lens, parent, tok = up(w.block_table), up(w.prefix_lens), up(w.parent), up(w.draft_tokens)
                cps = [dict(q=up(w.q, True), k=up(w.k_cache, True), v=up(w.v_cache, True), logits=up(w.target_logits),
                            probs=up(w.draft_probs)) for _ in range(R)]
                status = torch.zeros((w.B,), dtype=torch.int32, device=dev)
                ws_a = stv.spec_tree_attn_workspace_size(w.B, w.T, w.Hq, w.Hkv, w.D, w.max_blocks, stv.SPEC_BF16)
                attn_ws = torch.zeros(max(ws_a, 1), dtype=torch.uint8, device=dev)
                rej_ws = torch.zeros(int(lib.spec_tree_reject_workspace_size(w.B, w.T, w.V)), dtype=torch.uint8,
                                     device=dev)
                for c in cps:
                    c["out"] = torch.empty_like(c["q"])

                def attn(c):
                    stv.spec_tree_attn(c["q"], c["k"], c["v"], bt, lens, parent, scale=w.scale, out=c["out"],
                                       status=status, workspace=attn_ws if ws_a else None)

                def rejc(c):
                    stv.spec_tree_reject_compact(c["logits"], c["probs"], tok, parent, w.temperature, c["k"], c["v"],
                                                 bt, lens, w.without_replacement, w.seed, 0, status=status,
                                                 workspace=rej_ws)

                kv_new = torch.zeros((w.B, w.T, w.Hkv, w.D), dtype=cps[0]["k"].dtype, device=dev)

                theta = rope_theta(w)

                def kvw(c):
                    stv.spec_tree_kv_write(kv_new, kv_new, c["q"], c["k"], c["v"], bt, lens, parent, theta,
                                           status=status)

                ws_wa = stv.spec_tree_write_attn_workspace_size(w.B, w.T, w.Hq, w.Hkv, w.D, w.max_blocks,
                                                                stv.SPEC_BF16)
                wa_ws = torch.zeros(max(ws_wa, 1), dtype=torch.uint8, device=dev)

                def wattn(c):
                    stv.spec_tree_write_attn(kv_new, kv_new, c["q"], c["k"], c["v"], bt, lens, parent, theta,
                                             scale=w.scale, out=c["out"], status=status, workspace=wa_ws)

                us = {}
                for key, fn in (("attn_us", attn), ("reject_compact_us", rejc), ("kv_write_us", kvw),
                                ("write_attn_us", wattn)):
                    for c in cps:  # eager pass: validates every copy
                        fn(c)
                    torch.cuda.synchronize()
                    us[key] = seconds_per_call(fn, cps, R * max(1, 8 // R), 64) * 1e6
                if int(status.abs().sum()):
                    raise SystemExit(f"device reported input errors: {status.tolist()}")
                a_bytes, a_flops = attn_work(w)
                step = us["attn_us"] + us["reject_compact_us"]
                extra = {}
                if "accept_profile" in w.info:
                    _, e_tok = stv.spec_sequoia_tree(w.info["accept_profile"], w.T, depth_cap)
                    extra = {"expected_tokens": round(e_tok, 4),
                             "expected_tokens_per_s": round(w.B * e_tok / step * 1e6, 1)}
                print(json.dumps({"shape": name, "T": w.T, "prefix": L, "B": w.B, "depth": int(w.info["depth"]), **extra,
                                  "attn_us": round(us["attn_us"], 2),
                                  "reject_compact_us": round(us["reject_compact_us"], 2),
                                  "kv_write_us": round(us["kv_write_us"], 2),
                                  "write_attn_us": round(us["write_attn_us"], 2),
                                  "step_with_write_us": round(us["write_attn_us"] + us["reject_compact_us"], 2),
                                  "step_us": round(step, 2), "verified_tokens_per_s": round(w.B * w.T / step * 1e6, 1),
                                  "attn_GBps": round(a_bytes / us["attn_us"] / 1e3, 1),
                                  "attn_TFLOPs": round(a_flops / us["attn_us"] / 1e6, 2), "input_copies": R}),
                      flush=True)
                del cps, attn_ws, rej_ws
                torch.cuda.empty_cache()

def measure(cfg, args, quick=False):
    """One workload: the timed step line and its per-kernel figures (see the module docstring)."""
    import torch

    import tree_verify_attention_masked_amd as stv
    from workloads import make_config
    from workloads.gen import f32_to_bf16_bits

    dev = torch.device("cuda:0")
    log(f"[bench] building workload {cfg}")
    w = make_config(cfg)

    def up(a, kv=False):
        t = torch.from_numpy(np.ascontiguousarray(a))
        if kv and w.dtype == "bf16":
            t = t.view(torch.int16).view(torch.bfloat16)
        return t.to(dev)

    per_copy = (w.k_cache.nbytes * 2 + w.q.nbytes + w.target_logits.nbytes + w.draft_probs.nbytes)
    R = args.copies or max(1, min(16, math.ceil(768e6 / per_copy)))
    log(f"[bench] {R} input copies of {per_copy / 1e6:.1f} MB")
    shared = dict(bt=up(w.block_table), lens=up(w.prefix_lens), parent=up(w.parent), tok=up(w.draft_tokens))
    copies = []
    fused = w.dtype == "bf16"  # the step writes the tree's K/V rows in the attention launch
    theta = rope_theta(w)
    rng = np.random.default_rng(1000 + cfg)
    for _ in range(R):
        c = dict(q=up(w.q, True), k=up(w.k_cache, True), v=up(w.v_cache, True), logits=up(w.target_logits),
                 probs=up(w.draft_probs))
        if fused:  # the nodes' new K and V rows (before rotation), drawn here
            for key in ("k_new", "v_new"):
                x = rng.standard_normal((w.B, w.T, w.Hkv, w.D), dtype=np.float32)
                c[key] = torch.from_numpy(f32_to_bf16_bits(x)).view(torch.bfloat16).to(dev)
        c["out"] = torch.empty_like(c["q"])
        c["status"] = torch.zeros((w.B,), dtype=torch.int32, device=dev)
        copies.append(c)
    code = stv.SPEC_BF16 if w.dtype == "bf16" else stv.SPEC_F32
    ws_attn = stv.spec_tree_attn_workspace_size(w.B, w.T, w.Hq, w.Hkv, w.D, w.max_blocks, code)
    attn_ws = torch.zeros(max(ws_attn, 1), dtype=torch.uint8, device=dev)  # zero once: split arrival counters
    ws_wa = stv.spec_tree_write_attn_workspace_size(w.B, w.T, w.Hq, w.Hkv, w.D, w.max_blocks, code) if fused else 0
    wa_ws = torch.zeros(max(ws_wa, 1), dtype=torch.uint8, device=dev)  # zero once: work counter and flags
    rej_ws = torch.zeros(int(stv.load_library().spec_tree_reject_workspace_size(w.B, w.T, w.V)),
                         dtype=torch.uint8, device=dev)  # zero once: the sampler's epochs and tagged exchange slots
    rej_ws_t = torch.zeros(int(stv.spec_tree_reject_truncated_workspace_size(w.B, w.T, w.V, TRUNC_K)),
                           dtype=torch.uint8, device=dev)  # the truncating sampler's (slots and members' lists)

    # Step slots: one graph holds G consecutive steps; slot j runs on input copy
    # j % R with Philox offset (offset + j), so consecutive steps take different
    # walks, and keeps its own outputs.
    G = R * max(1, math.ceil(8 / R))
    slots = []
    for j in range(G):
        slots.append(dict(c=copies[j % R], offset=args.offset + j,
                          acc=torch.empty((w.B, w.T), dtype=torch.int32, device=dev),
                          toks=torch.empty((w.B, w.T), dtype=torch.int32, device=dev),
                          nacc=torch.empty((w.B,), dtype=torch.int32, device=dev),
                          new_lens=torch.empty((w.B,), dtype=torch.int32, device=dev)))

    def attn(c):
        stv.spec_tree_attn(c["q"], c["k"], c["v"], shared["bt"], shared["lens"], shared["parent"], scale=w.scale,
                           out=c["out"], status=c["status"], workspace=attn_ws if ws_attn else None)

    def write_attn(c):
        stv.spec_tree_write_attn(c["k_new"], c["v_new"], c["q"], c["k"], c["v"], shared["bt"], shared["lens"],
                                 shared["parent"], theta, scale=w.scale, out=c["out"], status=c["status"],
                                 workspace=wa_ws)

    def reject_compact(c, sl=None):
        sl = sl or slots[0]
        stv.spec_tree_reject_compact(c["logits"], c["probs"], shared["tok"], shared["parent"], w.temperature,
                                     c["k"], c["v"], shared["bt"], shared["lens"], w.without_replacement, w.seed,
                                     sl["offset"], accepted_nodes=sl["acc"], out_tokens=sl["toks"],
                                     num_accepted=sl["nacc"], new_lens=sl["new_lens"], status=c["status"],
                                     workspace=rej_ws)

    def reject_compact_trunc(c, sl=None):  # the same, against the target truncated inside the sampler
        sl = sl or slots[0]
        stv.spec_tree_reject_truncated(c["logits"], c["probs"], shared["tok"], shared["parent"], w.temperature,
                                       TRUNC_K, TRUNC_P, w.without_replacement, w.seed, sl["offset"],
                                       k_cache=c["k"], v_cache=c["v"], block_table=shared["bt"],
                                       prefix_lens=shared["lens"], accepted_nodes=sl["acc"], out_tokens=sl["toks"],
                                       num_accepted=sl["nacc"], new_lens=sl["new_lens"], status=c["status"],
                                       workspace=rej_ws_t)

    def step(sl):  # the timed step: (K/V write and) attention, then rejection + compaction
        (write_attn if fused else attn)(sl["c"])
        reject_compact(sl["c"], sl)

    def step_plain(sl):  # attention on rows already in the cache, then rejection + compaction
        attn(sl["c"])
        reject_compact(sl["c"], sl)

    def step_trunc(sl):  # the step against a top-k / top-p truncated target
        (write_attn if fused else attn)(sl["c"])
        reject_compact_trunc(sl["c"], sl)

    for c in copies:  # each copy's truncated target rows, written by the separate truncation pass
        c["logits_t"] = torch.empty_like(c["logits"])

    def step_trunc_pass(sl):  # the same target, truncated by a pass over every row before the plain sampler
        c = sl["c"]
        (write_attn if fused else attn)(c)
        stv.spec_tree_truncate(c["logits"], w.temperature, TRUNC_K, TRUNC_P, out=c["logits_t"], status=c["status"])
        reject_compact(dict(c, logits=c["logits_t"]), sl)

    if args.calib_copy and not quick:  # plain copies of known size, for scaling the HBM counters
        for nbytes in (CALIB_BYTES, CALIB_BYTES_BIG):
            src = torch.ones(nbytes // 4, dtype=torch.float32, device=dev)
            dst = torch.empty_like(src)
            dst.copy_(src)
            torch.cuda.synchronize()
            del src, dst

    for fn in ((step, step_plain, step_trunc, step_trunc_pass) if fused else (step, step_trunc, step_trunc_pass)):
        for sl in slots:  # eager pass: validates every copy and slot
            fn(sl)
        torch.cuda.synchronize()
        st = sum(int(c["status"].abs().sum()) for c in copies)
        if st:
            raise SystemExit(f"device reported input errors: {[c['status'].tolist() for c in copies]}")

    def timed(fn, what):
        """K steps of fn (graphs of G slots) between synchronisations, and the spread of single steps."""
        step_graphs = [capture_graph([lambda sl=sl: fn(sl)]) for sl in slots]
        run_graph = capture_graph([lambda sl=sl: fn(sl) for sl in slots])
        log(f"[bench] {what}: captured {len(step_graphs)} step graphs and one graph of {G} steps; "
            f"warmup {args.warmup}")
        for i in range(args.warmup):
            step_graphs[i % G].replay()
        torch.cuda.synchronize()
        K = args.steps
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(K // G):
            run_graph.replay()
        for i in range(K % G):
            step_graphs[i % G].replay()
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        log(f"[bench] {what}: {K} steps ({K // G} replays of {G} steps + {K % G} single steps): "
            f"wall {wall * 1e3:.3f} ms")
        # spread: single-step replays, each bracketed by events on the current stream
        n_spread = 30 if quick else 100
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(n_spread + 1)]
        evs[0].record()
        for i in range(n_spread):
            step_graphs[i % G].replay()
            evs[i + 1].record()
        torch.cuda.synchronize()
        per = np.array([evs[i].elapsed_time(evs[i + 1]) * 1e3 for i in range(n_spread)])
        spread = {"p10": round(float(np.percentile(per, 10)), 2), "p50": round(float(np.percentile(per, 50)), 2),
                  "p90": round(float(np.percentile(per, 90)), 2), "n": n_spread,
                  "note": "single-step graph replays, launch gap included"}
        return wall * 1e3 / K, w.B * w.T * K / wall, spread

    ms_per_step, value, spread = timed(step, "step")
    plain = None
    if fused:
        ms_plain, value_plain, spread_plain = timed(step_plain, "step without the K/V write")
        plain = {"value": round(value_plain, 1), "ms_per_step": round(ms_plain, 5), "step_us": spread_plain,
                 "note": "spec_tree_attn on rows already in the cache, then spec_tree_reject_compact"}

    ms_t, value_t, spread_t = timed(step_trunc, "step against the truncated target")
    truncated = {"value": round(value_t, 1), "ms_per_step": round(ms_t, 5), "step_us": spread_t,
                 "top_k": TRUNC_K, "top_p": TRUNC_P,
                 "note": "the step with spec_tree_reject_truncated (top-k then top-p applied inside the sampler to "
                         "the rows its walk visits) in place of spec_tree_reject_compact"}
    ms_tp, value_tp, spread_tp = timed(step_trunc_pass, "step with a separate truncation pass")
    truncated["separate_pass"] = {
        "value": round(value_tp, 1), "ms_per_step": round(ms_tp, 5), "step_us": spread_tp,
        "note": "the same target truncated by spec_tree_truncate over every row (out of place) before "
                "spec_tree_reject_compact"}

    # accepted tokens per step over every slot's walk (each slot has its own offset), untruncated target
    for sl in slots:
        step(sl)
    accs = [sl["acc"].cpu().numpy() for sl in slots]
    naccs = [sl["nacc"].cpu().numpy() for sl in slots]
    lp1 = np.concatenate([n + 1 for n in naccs]).astype(np.float64)

    # per-kernel average durations: one graph = reps launches of one call over the copies
    reps = args.kernel_reps or max(R, 8 * R if per_copy < 100e6 else R)
    kdur = {}
    timed_calls = (("tree_write_attn", write_attn),) if fused else ()
    for name, fn in timed_calls + (("tree_attn", attn), ("tree_reject_compact", reject_compact),
                                   ("tree_reject_compact_truncated", reject_compact_trunc)):
        kdur[name] = seconds_per_call(fn, copies, reps, 60 if quick else 200)
        log(f"[bench] {name}: {kdur[name] * 1e6:.2f} us per call")

    a_bytes, a_flops = attn_work(w)
    rb, cb = [], []
    for acc, nacc in zip(accs, naccs):
        stop_rej = []  # did the stop node form a residual (some child of it rejected)?
        for b in range(w.B):
            u = int(acc[b][int(nacc[b])])
            stop_rej.append(any(int(w.parent[b][i]) == u for i in range(1, w.T)))
        rb.append(reject_bytes(w, nacc, stop_rej))
        cb.append(compact_bytes(w, acc, nacc))
    rc_bytes = float(np.mean(rb)) + float(np.mean(cb))
    w_bytes = write_bytes(w) if fused else 0
    work = {"tree_attn": ("hbm", a_bytes, a_flops), "tree_reject_compact": ("hbm", rc_bytes, 0.0),
            "tree_reject_compact_truncated": ("hbm", rc_bytes, 0.0)}
    if fused:
        work["tree_write_attn"] = ("hbm", a_bytes + w_bytes, a_flops)
    kernels = {}
    for name, (b_, by, fl) in work.items():
        kernels[name] = {"us": round(kdur[name] * 1e6, 2), "bytes": int(by),
                         "GB/s": round(by / kdur[name] / 1e9, 1)}
        if fl:
            kernels[name]["TFLOP/s"] = round(fl / kdur[name] / 1e12, 2)
    for name in ("tree_write_attn", "tree_attn") if fused else ("tree_attn",):
        kernels[name]["hbm_frac"] = round(work[name][1] / kdur[name] / 1e9 / HBM_PEAK_GBS, 4)
        kernels[name]["mfma_frac"] = round(a_flops / kdur[name] / 1e12 / BF16_PEAK_TFLOPS, 4)
    if fused:
        kernels["tree_write_attn"]["rope_theta"] = theta
        kernels["tree_attn"]["in_step"] = False
    kernels["tree_reject_compact_truncated"].update(in_step=False, top_k=TRUNC_K, top_p=TRUNC_P)
    del work["tree_reject_compact_truncated"]
    step_bytes = a_bytes + w_bytes + rc_bytes
    step_roof = {"bound": "hbm", "bytes": int(step_bytes), "achieved": round(step_bytes / (ms_per_step * 1e-3) / 1e9, 1),
                 "peak": HBM_PEAK_GBS, "unit": "GB/s",
                 "frac": round(step_bytes / (ms_per_step * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                 "note": "algorithmic bytes of the whole step (the tree's K/V rows in and out, attention, the "
                         "walked rows, moved KV rows) / step time" if fused else
                         "algorithmic bytes of the whole step (attention, the walked rows, moved KV rows) / step time"}
    step_kernels = {k: v for k, v in kdur.items()
                    if not (fused and k == "tree_attn") and k != "tree_reject_compact_truncated"}
    return dict(w=w, value=value, ms_per_step=ms_per_step, spread=spread, lp1=lp1, kdur=step_kernels, work=work,
                kernels=kernels, step_roof=step_roof, copies=copies, slots=slots, shared=shared, R=R, reps=reps,
                a_bytes=a_bytes, a_flops=a_flops, fused=fused, plain=plain, theta=theta, truncated=truncated)


def roofline_of(m):
    """The `roofline` object for the dominant (longest) kernel of a measurement."""
    kdur, work = m["kdur"], m["work"]
    dominant = max(kdur, key=kdur.get)
    bound, bytes_, flops = work[dominant]
    if dominant in ("tree_attn", "tree_write_attn") and flops / max(bytes_, 1) > BF16_PEAK_TFLOPS / HBM_PEAK_GBS * 1e3:
        bound = "mfma"
    if bound == "hbm":
        achieved = bytes_ / kdur[dominant] / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None}
    else:
        achieved = flops / kdur[dominant] / 1e12
        roof = {"bound": "mfma", "achieved": round(achieved, 1), "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": round(achieved / BF16_PEAK_TFLOPS, 4), "traffic": None}
    roof["kernel"] = dominant
    t_bytes = committed_traffic(m["w"].name, dominant)
    if t_bytes is not None:
        roof["traffic"] = t_bytes
    return roof


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", type=int, default=4,
                    help="workload id 0..4 (default 4: batched serving, the largest single-GPU configuration)")
    ap.add_argument("--also", default="1",
                    help="comma-separated workload ids also measured (step and attention figures only) and "
                         "reported under `extra`; empty for none")
    ap.add_argument("--copies", type=int, default=0, help="input copies to rotate (0: auto, >= 768 MB)")
    ap.add_argument("--kernel-reps", type=int, default=0, help="launches per per-kernel timing graph")
    ap.add_argument("--cpu-budget", type=float, default=12.0, help="seconds of oracle time (0: skip)")
    ap.add_argument("--offset", type=int, default=0, help="Philox offset of the first step slot")
    ap.add_argument("--calib-copy", action="store_true",
                    help="run plain 256 MiB and 1 GiB device copies (counter calibration)")
    ap.add_argument("--summarize", nargs="+", metavar=("KIND", "DIR"),
                    help="trace DIR | pmc FETCH_DIR WRITE_DIR | sq DIR...: print a markdown summary of rocprofv3 output")
    ap.add_argument("--workload-name", default="batched_serving", help="workload name recorded by --summarize pmc")
    ap.add_argument("--sweep", action="store_true", help="verify cost against tree size and prefix length (one GPU)")
    args = ap.parse_args()

    if args.summarize:
        print(summarize(args.summarize[0], args.summarize[1:], args.workload_name))
        return

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    if args.sweep:
        sweep()
        return

    import torch

    import tree_verify_attention_masked_amd as stv

    stv.load_library()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    m = measure(args.config, args)
    w, copies, shared, reps = m["w"], m["copies"], m["shared"], m["reps"]
    roof = roofline_of(m)
    kernels = m["kernels"]
    value_main, ms_main, spread_main, step_roof_main, R_main = (m["value"], m["ms_per_step"], m["spread"],
                                                                 m["step_roof"], m["R"])
    fused_main, plain_main, theta_main, trunc_main = m["fused"], m["plain"], m["theta"], m["truncated"]

    # The step before attention as a launch of its own (the timed bf16 step does
    # it inside the attention launch): the tree's K/V rows into the cache, keys
    # and queries rotated for their tree positions.
    kv_new = dict(k=torch.zeros((w.B, w.T, w.Hkv, w.D), dtype=copies[0]["k"].dtype, device=dev))
    kv_new["v"] = torch.zeros_like(kv_new["k"])

    def kv_write(c):
        stv.spec_tree_kv_write(kv_new["k"], kv_new["v"], c["q"], c["k"], c["v"], shared["bt"], shared["lens"],
                               shared["parent"], rope_theta(w), status=c["status"])

    t_kvw = seconds_per_call(kv_write, copies, reps, 200)
    log(f"[bench] tree_kv_write: {t_kvw * 1e6:.2f} us per call")

    # Top-k / top-p truncation of the target logits (top-k 50, then top-p 0.9), out of place so that
    # every call sees the untruncated rows; not part of the timed step, whose target is not truncated.
    trunc_out = torch.empty_like(copies[0]["logits"])

    def truncate(c):
        stv.spec_tree_truncate(c["logits"], w.temperature, TRUNC_K, TRUNC_P, out=trunc_out, status=c["status"])

    t_trunc = seconds_per_call(truncate, copies, reps, 200)
    log(f"[bench] tree_truncate: {t_trunc * 1e6:.2f} us per call")
    elt = 2 if w.dtype == "bf16" else 4
    kvw_bytes = w.B * w.T * w.D * elt * (4 * w.Hkv + 2 * w.Hq)  # K, V in and out; Q in and out
    kernels["tree_kv_write"] = {"us": round(t_kvw * 1e6, 2), "bytes": int(kvw_bytes),
                                "GB/s": round(kvw_bytes / t_kvw / 1e9, 1), "in_step": False}
    trunc_bytes = w.B * w.T * w.V * 4 * 2  # every logit read once and written once (out of place)
    kernels["tree_truncate"] = {"us": round(t_trunc * 1e6, 2), "bytes": int(trunc_bytes),
                                "GB/s": round(trunc_bytes / t_trunc / 1e9, 1), "in_step": False,
                                "top_k": TRUNC_K, "top_p": TRUNC_P}
    lp1 = m["lp1"]
    accepted = {"mean": round(float(lp1.mean()), 3), "p10": float(np.percentile(lp1, 10)),
                "p90": float(np.percentile(lp1, 90)), "walks": int(lp1.size)}
    del m, copies, kv_new, trunc_out
    torch.cuda.empty_cache()

    extra = {}
    for e in [int(x) for x in args.also.split(",") if x.strip() != ""]:
        if e == args.config:
            continue
        me = measure(e, args, quick=True)
        re_ = roofline_of(me)
        extra[me["w"].name] = {"value": round(me["value"], 1), "unit": "tokens/s",
                               "ms_per_step": round(me["ms_per_step"], 5), "step_us": me["spread"],
                               "kv_write_in_step": me["fused"], "without_kv_write": me["plain"],
                               "truncated_target": me["truncated"],
                               "roofline": re_, "step_roofline": me["step_roof"], "kernels": me["kernels"],
                               "accepted_per_step": round(float(me["lp1"].mean()), 3), "config": me["w"].summary()}
        del me
        torch.cuda.empty_cache()

    cpu = None
    if args.cpu_budget > 0:
        log(f"[bench] oracle baseline (~{args.cpu_budget:.0f} s)")
        cpu = cpu_baseline(w, args.cpu_budget, theta_main if fused_main else None)

    cfg = w.summary()
    line = {
        "metric": METRIC, "value": round(value_main, 1), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_main, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16" if w.dtype == "bf16" else "f32",
        "data": "synthetic", "config": cfg, "roofline": roof, "step_roofline": step_roof_main,
        "cpu_baseline": cpu, "kernels": kernels, "step_us": spread_main, "accepted_per_step": accepted,
        "kv_write_in_step": fused_main, "without_kv_write": plain_main, "truncated_target": trunc_main,
        "input_copies": R_main, "extra": extra,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
