#!/usr/bin/env python3
"""Throughput of one draft step of the tree-causal draft head on one MI355X.

A step is the whole hot path over one batch of synthetic input:
  1. jf_tree_mask_build  -- ancestor bitmask of the 256-node tree
  2. jf_fuse_proj        -- fused projection of 3 target-layer hidden states
                            (one row per tree node, 3*4096 -> 4096, bf16 MFMA)
  3. jf_tree_attn_fwd    -- tree-causal attention over the 4096-token prefix
  4. jf_node_topk        -- per-node top-8 over a 151936-token vocabulary + lse
on the Qwen3-8B-shaped high-budget workload (1 sequence, 4096-token prefix,
256-node tree, 32/8 heads, head dim 128, bf16).  Inputs are generated on the
host, uploaded, and resident in HBM before the timed region.

Prints one JSON line: value = tree nodes per second over K back-to-back steps
(wall clock between device synchronisations), the steps run as HIP graphs of
four consecutive steps, each step joined on every stream before the next
begins (--steps-per-graph; the one-step graph and --eager's plain launches are
reported beside it), per-call HIP-event timings from an eager pass,
the roofline of the dominant call and of the tree attention, a cold-cache
variant (a 512 MiB read between steps evicts the 256 MiB last-level cache),
and the fp64 oracle timed on this host's cores on a bounded sample.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "draft-tree nodes/sec + tree-attn HBM GB/s (% of peak), 256-node tree @ 1 GPU"
HBM_PEAK_GBS = 8000.0        # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0    # MI355X dense bf16 MFMA
FP32_VECTOR_PEAK_TFLOPS = 157.3                          # MI355X fp32 vector
RIDGE = BF16_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9)   # flop per byte where the two bounds meet
FLUSH_BYTES = 512 * 1024 * 1024                          # > the 256 MiB last-level cache


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", type=int, default=2, help="workload id (synth.WORKLOADS)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cold-steps", type=int, default=20)
    ap.add_argument("--eager", action="store_true",
                    help="time the eager launches (no graph) for the headline value")
    ap.add_argument("--attn-cus", type=int, default=-1,
                    help="compute units the attention's key splits are planned for in the two-stream "
                         "step (-1: three quarters of the device's when mask + attention is the "
                         "shorter stream by the eager per-call times, else all; 0: all)")
    ap.add_argument("--fuse-cus", type=int, default=-1,
                    help="compute units the projection's K split is planned for in the two-stream "
                         "step (-1: three quarters of the device's; 0: all)")
    ap.add_argument("--topk-split", type=float, default=0.0,
                    help="fraction of the top-k rows run on the attention's stream in the two-stream "
                         "step (after the attention; the rest follow the projection on the other)")
    ap.add_argument("--steps-per-graph", type=int, default=4,
                    help="consecutive steps captured in one HIP graph, each joined on every stream "
                         "before the next begins (1: one step a graph)")
    ap.add_argument("--one-stream", action="store_true",
                    help="headline from the graph of the step on one stream (default: two streams)")
    ap.add_argument("--cpu-sample-nodes", type=int, default=256)
    ap.add_argument("--no-context-projection", action="store_true",
                    help="skip timing the projection at one row per prefix token")
    ap.add_argument("--no-tree-growth", action="store_true",
                    help="skip timing the path-score and expansion calls after the step")
    ap.add_argument("--no-lm-head", action="store_true",
                    help="skip timing the LM-head contraction (one-layer jf_fuse_proj to the vocabulary)")
    ap.add_argument("--topk-sweep", action="store_true",
                    help="also time jf_node_topk over the step's logits at k = 1, 8, 16, 32, 64")
    ap.add_argument("--no-attention-records", action="store_true",
                    help="skip timing the tree attention alone on the serving and MoE-shaped workloads")
    ap.add_argument("--attention-records-only", action="store_true",
                    help="only time the tree attention on the other workloads (profiling runs)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 256 MiB device copy 5 times (counter calibration)")
    return ap.parse_args()


KERNELS = {"mask": ["k_tree_mask"],
           "fuse": ["k_fuse_gemm_bf16", "k_fuse_reduce", "k_fuse_gemm_f32"],
           "attn": ["k_tree_attn_split", "k_tree_attn_merge", "k_tree_attn_f32"],
           "topk": ["k_topk_stage1", "k_topk_stage2"]}
TRAFFIC_JSON = os.path.join(ROOT, "profiles", "traffic.json")
COPY_BYTES = 256 * 1024 * 1024


def copy_calibration():
    """A plain device copy of known size, for scaling the fabric byte counters."""
    import torch
    src = torch.empty(COPY_BYTES, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"calibration": "copy", "bytes_each_way": COPY_BYTES, "launches": 5}), flush=True)


KERNEL_FILES = {"mask": ["k_mask.hip"], "fuse": ["k_fuse.hip"], "attn": ["k_attn.hip"],
                "topk": ["k_topk.hip"]}


def measured_traffic(call, workload):
    """HBM-side bytes per launch of a call's kernels from the committed counter
    record (FETCH_SIZE + WRITE_SIZE, copy-calibrated) and a note of where they
    come from, or (None, reason) when there is no record for this workload or
    the call's kernel source (or the shared internal header) changed since it
    was taken."""
    from tree_causal_draft_parent_amd import profsum
    try:
        with open(TRAFFIC_JSON) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None, "no counter record"
    if rec.get("workload") != workload:
        return None, f"no counter record for {workload}"
    measured = rec.get("file_sha256")
    cur = profsum.file_hashes()
    files = KERNEL_FILES[call] + ["jf_internal.h"]
    if measured is None or any(measured.get(fn) is None or measured.get(fn) != cur.get(fn) for fn in files):
        return None, "kernel sources changed since the counters were taken"
    total, found = 0, False
    for k, v in rec.get("kernels", {}).items():
        base = k.split("<")[0]
        if base in KERNELS[call] and v.get("fetch_bytes") is not None and v.get("write_bytes") is not None:
            total += v["fetch_bytes"] + v["write_bytes"]
            found = True
    if not found:
        return None, "no counters for the call's kernels"
    src = ("recorded: profiles/traffic.json, FETCH_SIZE + WRITE_SIZE per launch (copy-calibrated), "
           "kernel sources " + ", ".join(f"{fn} sha256 {measured[fn][:16]}" for fn in files))
    return total, src


def to_dev(a, dtype, torch):
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def algorithmic(wl, inp, fuse_out_bytes):
    """Bytes and flops each call must move / do at minimum (no re-reads)."""
    a = inp["attn"]
    B, N, Hq, Hkv, D = wl.B, wl.N, wl.Hq, wl.Hkv, wl.D
    e = 2 if wl.dtype == "bf16" else 4
    W = (N + 63) // 64
    sumP = int(np.sum(a["prefix_len"]))
    depth_sum = 0
    for b in range(B):
        par = a["parent"][b]
        d = np.zeros(N, np.int64)
        for i in range(N):
            d[i] = 1 if par[i] < 0 else d[par[i]] + 1
        depth_sum += int(d.sum())
    M, H, k = B * N, wl.H, wl.n_fused
    out = {}
    out["mask"] = dict(bytes=B * N * 4 + B * N * W * 8 + B * N * 4, flops=0)
    out["fuse"] = dict(bytes=k * M * H * e + H * k * H * e + M * H * fuse_out_bytes,
                       flops=2 * M * H * k * H)
    out["attn"] = dict(bytes=B * N * Hq * D * e + 2 * B * N * Hkv * D * e + 2 * sumP * Hkv * D * e
                       + B * N * W * 8 + B * N * Hq * D * e + B * N * Hq * 4,
                       flops=4 * Hq * D * (N * sumP + depth_sum))
    out["attn_prefix_kv_bytes"] = 2 * sumP * Hkv * D * e
    R = B * N
    out["topk"] = dict(bytes=R * wl.V * e + R * wl.topk * 8 + R * 4, flops=0)
    return out


def attn_algorithmic(a, Hq, Hkv, D, e=2, kv_e=None):
    """Algorithmic bytes and flops of one tree-attention call over the inputs
    `a` (uniform or packed trees): queries, tree K/V, mask, output and lse
    once, every prefix key and value once (kv_e bytes an element), and
    4 * Hq * D flops per visible (node, key) pair."""
    kv_e = e if kv_e is None else kv_e
    no = a.get("node_off")
    B = len(a["prefix_len"])
    if no is None:
        counts = [a["parent"].shape[1]] * B
        pars = [a["parent"][b] for b in range(B)]
    else:
        counts = list(np.diff(no))
        pars = [a["parent"][no[b]:no[b + 1]] for b in range(B)]
    N = max(counts)
    W = (N + 63) // 64
    T = int(sum(counts))
    sumP = int(np.sum(a["prefix_len"]))
    pairs = 0
    for b in range(B):
        par, n = pars[b], counts[b]
        d = np.zeros(n, np.int64)
        for i in range(n):
            d[i] = 1 if par[i] < 0 else d[par[i]] + 1
        pairs += n * int(a["prefix_len"][b]) + int(d.sum())
    bytes_ = (T * Hq * D * e + 2 * T * Hkv * D * e + 2 * sumP * Hkv * D * kv_e + T * W * 8
              + T * Hq * D * e + T * Hq * 4)
    return dict(bytes=int(bytes_), flops=int(4 * Hq * D * pairs),
                prefix_kv_bytes=int(2 * sumP * Hkv * D * kv_e))


def bound_of(flops, nbytes):
    """The roofline that binds a call: MFMA when its arithmetic intensity is
    above the ridge, else HBM (calls without flops: HBM)."""
    return "mfma" if nbytes > 0 and flops / nbytes > RIDGE else "hbm"


def roof_numbers(alg, ms):
    """GB/s, TFLOP/s, the binding bound and the fraction of its peak."""
    sec = ms * 1e-3
    gbs = alg["bytes"] / sec / 1e9
    tfs = alg["flops"] / sec / 1e12
    b = bound_of(alg["flops"], alg["bytes"])
    frac = tfs / BF16_PEAK_TFLOPS if b == "mfma" else gbs / HBM_PEAK_GBS
    return gbs, tfs, b, frac


def flush_cache(buf):
    """Evict the last-level cache and the L2s by reading `buf` (512 MiB, twice
    the 256 MiB last-level cache) in one reduction.  A read leaves clean
    lines behind; a write would leave dirty ones that the next call would
    pay to write back."""
    return buf.amax()


def time_calls(fn, n, torch, flush=None):
    """Median and mean per-call time (ms) of fn over n calls, HIP events on
    the current stream (the stream the binding launches on).  flush: a
    buffer written before each call (cold: the last-level cache holds none
    of the call's data), else the calls run back to back (warm)."""
    ts = []
    evs = []
    for k in range(n):
        if flush is not None:
            flush_cache(flush)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        fn()
        e1.record()
        evs.append((e0, e1))
        if flush is not None:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    ts = [a.elapsed_time(b) for a, b in evs]
    return float(np.median(ts)), float(np.mean(ts))


def attention_records(steps, torch, jf, flush):
    """The tree attention alone on the other workloads, each timed warm and
    flushed: the serving batch (bf16 and FP8 prefix caches, and packed trees
    of 16/64/256 nodes) and the 4 x 32768-token MoE-shaped batch."""
    from tree_causal_draft_parent_amd import synth
    out = {}
    n = max(10, min(steps, 30))

    def one(name, a, Hq, Hkv, D, kv_e=2, k_scale=1.0, v_scale=1.0):
        dev = {k: to_dev(a[k], "bf16", torch) for k in ("q", "k_tree", "v_tree")}
        for k in ("k_cache", "v_cache"):
            dev[k] = torch.from_numpy(np.ascontiguousarray(a[k])).cuda() if kv_e == 1 else \
                to_dev(a[k], "bf16", torch)
        parent = torch.from_numpy(a["parent"]).cuda()
        bt = torch.from_numpy(a["block_table"]).cuda()
        no = a.get("node_off")
        mask, _, _ = jf.jf_tree_mask_build(parent, node_off=no)
        outt = torch.empty_like(dev["q"])
        lse = torch.empty(dev["q"].shape[:-1], dtype=torch.float32, device="cuda")
        N = int(mask.shape[-2]) if no is None else int(np.max(np.diff(no)))
        need = jf.jf_tree_attn_workspace_size(len(a["prefix_len"]), N, Hq, Hkv, D, a["page_size"],
                                              a["prefix_len"], jf.JF_BF16, node_off=no)
        ws = torch.empty(max(need, 1), dtype=torch.uint8, device="cuda")
        st = torch.zeros(1, dtype=torch.int32, device="cuda")

        def call():
            jf.jf_tree_attn_fwd(dev["q"], dev["k_tree"], dev["v_tree"], mask, dev["k_cache"],
                                dev["v_cache"], bt, a["prefix_len"], out=outt, lse=lse, workspace=ws,
                                status=st, node_off=no, k_scale=k_scale, v_scale=v_scale)

        for _ in range(3):
            call()
        warm, warm_mean = time_calls(call, n, torch)
        cold, _ = time_calls(call, n, torch, flush=flush)
        assert int(st.item()) == 0
        alg = attn_algorithmic(a, Hq, Hkv, D, 2, kv_e)
        gbs, tfs, b, frac = roof_numbers(alg, cold)
        wgbs, wtfs, _, wfrac = roof_numbers(alg, warm)
        nodes = int(mask.shape[0] * mask.shape[1]) if no is None else int(no[-1])
        out[name] = {
            "call": "jf_tree_attn_fwd", "timing": "median per-call HIP events; cold: a 512 MiB read "
                                                  "before each call", "launches": n,
            "cold_ms": round(cold, 5), "warm_ms": round(warm, 5), "warm_mean_ms": round(warm_mean, 5),
            "nodes": nodes, "nodes_per_s": round(nodes / (cold * 1e-3), 1),
            "bound": b, "frac_of_bound": round(frac, 4),
            "hbm_GBps": round(gbs, 1), "hbm_frac": round(gbs / HBM_PEAK_GBS, 4),
            "TFLOPs": round(tfs, 2), "mfma_frac": round(tfs / BF16_PEAK_TFLOPS, 4),
            "prefix_kv_GBps": round(alg["prefix_kv_bytes"] / (cold * 1e-3) / 1e9, 1),
            "warm": {"hbm_frac": round(wgbs / HBM_PEAK_GBS, 4), "mfma_frac": round(wtfs / BF16_PEAK_TFLOPS, 4),
                     "frac_of_bound": round(wfrac, 4)},
            "algorithmic": alg, "workspace_bytes": int(need)}
        print(f"[bench] attention {name}: cold {cold:.4f} ms, warm {warm:.4f} ms, "
              f"{b} {frac:.3f} of peak", file=sys.stderr, flush=True)
        del dev, mask, outt, lse, ws

    w3, w4 = synth.workload(3), synth.workload(4)
    a3 = synth.make_workload(3, parts=("attn",))["attn"]
    one(w3.name, a3, w3.Hq, w3.Hkv, w3.D)
    del a3
    P3 = synth.prefix_lengths(3)
    a3f = synth.make_attn_inputs(B=w3.B, N=w3.N, Hq=w3.Hq, Hkv=w3.Hkv, D=w3.D, dtype="bf16",
                                 prefix_lens=P3, page_size=w3.page_size, shuffled_pages=True,
                                 max_depth=w3.max_depth, branching=w3.branching,
                                 seed=synth.config_seed(3), kv_dtype="fp8")
    one(w3.name + "-fp8kv", a3f, w3.Hq, w3.Hkv, w3.D, kv_e=1, k_scale=a3f["k_scale"],
        v_scale=a3f["v_scale"])
    del a3f
    counts = np.random.default_rng(synth.config_seed(3) + 5).choice([16, 64, 256], size=w3.B)
    a3p = synth.make_attn_inputs(B=w3.B, N=0, Hq=w3.Hq, Hkv=w3.Hkv, D=w3.D, dtype="bf16",
                                 prefix_lens=P3, page_size=w3.page_size, shuffled_pages=True,
                                 max_depth=w3.max_depth, branching=w3.branching,
                                 seed=synth.config_seed(3) + 6, node_counts=counts)
    one("serving-b32-ragged-paged-packed-n16-64-256", a3p, w3.Hq, w3.Hkv, w3.D)
    out["serving-b32-ragged-paged-packed-n16-64-256"]["node_counts"] = \
        {str(c): int(np.sum(counts == c)) for c in (16, 64, 256)}
    del a3p
    a4 = synth.make_workload(4, parts=("attn",))["attn"]
    one(w4.name, a4, w4.Hq, w4.Hkv, w4.D)
    del a4
    return out


def cpu_baseline(wl, inp, n_nodes, min_seconds=10.0):
    """The fp64 oracle (test infrastructure) on this host over a sample of the
    step: the first n_nodes tree nodes of sequence 0 through all four parts,
    repeated until at least min_seconds of CPU work have been timed."""
    import oracle
    from tree_causal_draft_parent_amd import synth
    a = inp["attn"]
    N, Hq = wl.N, wl.Hq
    n = min(n_nodes, N)
    rows_attn = np.arange(n * Hq, dtype=np.int64)           # sequence 0, nodes 0..n-1, all heads
    rows_node = np.arange(n, dtype=np.int64)
    x64 = synth.to_f64(inp["fuse"]["x"], wl.dtype)
    w64 = synth.to_f64(inp["fuse"]["w"], wl.dtype)
    lg64 = synth.to_f64(inp["logits"][:n], wl.dtype)
    f = {key: synth.to_f64(a[key], wl.dtype) for key in ("q", "k_tree", "v_tree", "k_cache", "v_cache")}
    reps = 0
    t0 = time.perf_counter()
    while True:
        oracle.tree_mask(a["parent"])
        oracle.fuse_proj(x64, w64, rows=rows_node)
        oracle.tree_attn(q=f["q"], k_tree=f["k_tree"], v_tree=f["v_tree"], parent=a["parent"],
                         k_cache=f["k_cache"], v_cache=f["v_cache"], block_table=a["block_table"],
                         prefix_len=a["prefix_len"], page_size=a["page_size"], rows=rows_attn)
        oracle.topk(lg64, wl.topk)
        reps += 1
        dt = time.perf_counter() - t0
        if dt >= min_seconds:
            break
    return {"value": n * reps / dt, "unit": "nodes/s", "cores": oracle.num_threads(), "kind": "oracle",
            "sample": f"{n} of {N} tree nodes of sequence 0 through mask, fused projection, "
                      f"tree attention (all {Hq} heads) and top-{wl.topk}+lse, {reps} times; {dt:.2f} s"}


def cpu_baseline_one_thread(wl, inp, n_nodes, min_seconds=5.0):
    """The same oracle sample on one host thread (a smaller node sample)."""
    import oracle
    all_threads = oracle.num_threads()
    oracle.set_num_threads(1)
    try:
        r = cpu_baseline(wl, inp, n_nodes, min_seconds)
    finally:
        oracle.set_num_threads(all_threads)
    return {"value": r["value"], "unit": "nodes/s", "cores": 1, "sample": r["sample"]}


def copy_bandwidth(torch, reps=10):
    """Achievable device-copy rate (bytes read + written per second) of a plain
    256 MiB torch copy, timed with events on the current stream."""
    src = torch.empty(COPY_BYTES // 4, dtype=torch.float32, device="cuda").fill_(1.0)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    return 2 * COPY_BYTES * reps / (e0.elapsed_time(e1) * 1e-3) / 1e9


def topk_sweep(logits, steps, torch, jf):
    """jf_node_topk over the step's logits (with the row log-sum-exp) at several
    k, each timed as a graph of 20 back-to-back calls."""
    R, V = logits.shape
    out = {}
    for k in (1, 8, 16, 32, 64):
        idx = torch.empty((R, k), dtype=torch.int32, device="cuda")
        val = torch.empty((R, k), dtype=torch.float32, device="cuda")
        lse = torch.empty((R,), dtype=torch.float32, device="cuda")
        ws = torch.empty(max(jf.jf_node_topk_workspace_size(R, V, k), 1), dtype=torch.uint8,
                         device="cuda")
        ms = graph_time(lambda: jf.jf_node_topk(logits, k, idx=idx, val=val, lse=lse, workspace=ws),
                        steps, torch)
        out[f"k{k}"] = {"ms": round(ms, 5),
                        "GBps": round(logits.numel() * logits.element_size() / (ms * 1e-3) / 1e9, 1)}
    out.update(rows=R, vocab=V, timing="graph of 20 back-to-back calls")
    return out


def tree_growth(wl, parent, depth, idx, val, rlse, steps, torch, jf, parent_np=None, logits=None):
    """The calls that grow the tree after a step (outside the timed step):
    jf_path_scores over the step's tree (per-node conditional log-probabilities
    drawn from a seeded generator) and one jf_tree_expand of that tree by N new
    nodes from the step's top-k lists.  Both are latency-bound (a few KiB per
    sequence)."""
    from tree_causal_draft_parent_amd import synth
    B, N, k = wl.B, wl.N, wl.topk
    lp = synth.make_path_inputs(B=B, N=N, seed=synth.config_seed(wl_id(wl)) + 17)["logp"]
    logp = torch.from_numpy(lp).cuda()
    score = torch.empty((B, N), dtype=torch.float32, device="cuda")
    st = torch.empty((B,), dtype=torch.int32, device="cuda")
    M = N
    outs = tuple(torch.empty((B, M), dtype=t, device="cuda")
                 for t in (torch.int32, torch.int32, torch.float32, torch.int32))
    idx3, val3, lse2 = idx.view(B, N, k), val.view(B, N, k), rlse.view(B, N)

    def path():
        jf.jf_path_scores(parent, logp, score=score, seq_status=st)

    # greedy verification of the same tree: the target's next tokens as the
    # top-1 of logits of the verification pass's shape (the step's logits
    # stand in for the target's), then the longest accepted path.  The drafted
    # tokens are also the tree the expansion grows.
    v = synth.make_verify_inputs(parent_np, q=0.9, seed=synth.config_seed(wl_id(wl)) + 19)
    vtok = torch.from_numpy(v["token"]).cuda()

    def expand():
        jf.jf_tree_expand(score, depth, idx3, val3, lse2, parent, vtok, M, wl.max_depth, out=outs)

    vnxt = torch.from_numpy(v["target_next"]).cuda()
    vroot = torch.from_numpy(v["root_next"]).cuda()
    aouts = (torch.empty((B,), dtype=torch.int32, device="cuda"),
             torch.empty((B,), dtype=torch.int32, device="cuda"),
             torch.empty((B,), dtype=torch.int32, device="cuda"),
             torch.empty((B, N), dtype=torch.int32, device="cuda"),
             torch.empty((B,), dtype=torch.int32, device="cuda"))
    R = logits.shape[0]
    t1 = (torch.empty((R, 1), dtype=torch.int32, device="cuda"),
          torch.empty((R, 1), dtype=torch.float32, device="cuda"))
    t1_ws = torch.empty(max(jf.jf_node_topk_workspace_size(R, logits.shape[1], 1), 1),
                        dtype=torch.uint8, device="cuda")

    def accept():
        jf.jf_tree_accept(parent, vtok, vnxt, vroot, out=aouts)

    def argmax():
        jf.jf_node_topk(logits, 1, with_lse=False, idx=t1[0], val=t1[1], workspace=t1_ws)

    # An isolated call would leave the GPU waiting for the host's launch, so
    # each call is captured REP times into a HIP graph and the replays are timed.
    REP = 20
    res = {}
    for name, fn in (("path_scores", path), ("tree_expand", expand), ("tree_accept", accept),
                     ("target_argmax", argmax)):
        fn()
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for _ in range(REP):
                fn()
        for _ in range(3):
            g.replay()
        torch.cuda.synchronize()
        ms = []
        for _ in range(max(5, steps // REP)):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            g.replay()
            e1.record()
            torch.cuda.synchronize()
            ms.append(e0.elapsed_time(e1) / REP)
        res[name] = {"ms": round(float(np.mean(ms)), 5), "p50_ms": round(float(np.median(ms)), 5),
                     "bound": "latency", "timing": f"graph of {REP} back-to-back calls"}
        del g
    assert bool((st == -1).all()) and bool((aouts[4] == -1).all())
    res["tree_expand"].update(candidates=B * N * k, budget=M)
    res["tree_accept"]["accepted_len"] = [int(x) for x in aouts[0].cpu()]
    res["target_argmax"].update(rows=R, vocab=int(logits.shape[1]),
                                GBps=round(logits.numel() * logits.element_size()
                                           / (res["target_argmax"]["ms"] * 1e-3) / 1e9, 1))
    res["new_nodes_per_s"] = round(B * M / (res["tree_expand"]["ms"] * 1e-3), 1)
    return res


def lm_head(wl, steps, torch, jf):
    """The draft layer's LM head as jf_fuse_proj with one layer: B*N tree-node
    rows x H hidden -> V vocabulary logits in bf16 (the top-k's input shape).
    The weights are random bf16 drawn on the device (timing only; parity is
    tested on the seeded generator's weights).  HBM-bound: the V x H weight
    stream dominates."""
    if wl.dtype != "bf16":
        return None
    M, H, V = wl.B * wl.N, wl.H, wl.V
    g = torch.Generator(device="cuda").manual_seed(31)
    w = (torch.randn((V, H), generator=g, device="cuda") * 0.02).to(torch.bfloat16)
    x = torch.randn((M, H), generator=g, device="cuda").to(torch.bfloat16)
    y = torch.empty((M, V), dtype=torch.bfloat16, device="cuda")
    need = jf.jf_fuse_proj_workspace_size(M, H, 1, V, jf.JF_BF16)
    ws = torch.empty(max(need, 1), dtype=torch.uint8, device="cuda")
    for _ in range(3):
        jf.jf_fuse_proj([x], w, y=y, workspace=ws)
    torch.cuda.synchronize()
    n = max(5, steps // 5)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(n):
        jf.jf_fuse_proj([x], w, y=y, workspace=ws)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / n
    nbytes = V * H * 2 + M * H * 2 + M * V * 2
    flops = 2 * M * H * V
    res = {"M": M, "K": H, "N": V, "ms": round(ms, 5), "bytes": nbytes,
           "hbm_GBps": round(nbytes / (ms * 1e-3) / 1e9, 1),
           "hbm_frac": round(nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
           "TFLOPs": round(flops / (ms * 1e-3) / 1e12, 2), "launches": n}
    del w, x, y, ws
    return res


def graph_time(fn, steps, torch, rep=20):
    """Mean time of fn over replays of a HIP graph of `rep` back-to-back calls."""
    fn()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(rep):
            fn()
    for _ in range(3):
        g.replay()
    torch.cuda.synchronize()
    ms = []
    for _ in range(max(5, steps // rep)):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        g.replay()
        e1.record()
        torch.cuda.synchronize()
        ms.append(e0.elapsed_time(e1) / rep)
    return float(np.mean(ms))


def norm_timing(wl, q, k_tree, steps, torch, jf):
    """jf_rmsnorm over the layer input (B*N rows x H) and per head over the
    step's queries and tree keys (copies), each timed as a graph of 20 calls."""
    B, N = wl.B, wl.N
    g = torch.Generator(device="cuda").manual_seed(41)
    tdt = torch.bfloat16 if wl.dtype == "bf16" else torch.float32
    hid = torch.randn((B * N, wl.H), generator=g, device="cuda").to(tdt)
    wh = torch.randn((wl.H,), generator=g, device="cuda").to(tdt)
    hy = torch.empty_like(hid)
    qc, kc = q.clone().view(-1, wl.D), k_tree.clone().view(-1, wl.D)
    wd = torch.randn((wl.D,), generator=g, device="cuda").to(tdt)
    t_h = graph_time(lambda: jf.jf_rmsnorm(hid, wh, y=hy), steps, torch)

    def heads():
        jf.jf_rmsnorm(qc, wd, y=qc)
        jf.jf_rmsnorm(kc, wd, y=kc)

    t_q = graph_time(heads, steps, torch)
    e = hid.element_size()
    return {"hidden": {"rows": B * N, "H": wl.H, "ms": round(t_h, 5),
                       "GBps": round(2 * hid.numel() * e / (t_h * 1e-3) / 1e9, 1)},
            "qk_heads": {"rows": qc.shape[0] + kc.shape[0], "H": wl.D, "ms": round(t_q, 5),
                         "GBps": round(2 * (qc.numel() + kc.numel()) * e / (t_q * 1e-3) / 1e9, 1),
                         "launches": 2},
            "bound": "latency", "timing": "graph of 20 back-to-back calls"}


def mlp_timing(wl, steps, torch, jf, inter=12288):
    """The draft layer's gated MLP over B*N rows: one projection to the gate
    and up columns (weights stacked, [2I, H]), jf_swiglu, and the down
    projection ([H, I]); device-drawn random bf16 weights (timing only)."""
    if wl.dtype != "bf16":
        return None
    M, H = wl.B * wl.N, wl.H
    g = torch.Generator(device="cuda").manual_seed(43)
    x = torch.randn((M, H), generator=g, device="cuda").to(torch.bfloat16)
    w_gu = (torch.randn((2 * inter, H), generator=g, device="cuda") * 0.02).to(torch.bfloat16)
    w_dn = (torch.randn((H, inter), generator=g, device="cuda") * 0.02).to(torch.bfloat16)
    gu = torch.empty((M, 2 * inter), dtype=torch.bfloat16, device="cuda")
    act = torch.empty((M, inter), dtype=torch.bfloat16, device="cuda")
    out = torch.empty((M, H), dtype=torch.bfloat16, device="cuda")
    ws1 = torch.empty(max(jf.jf_fuse_proj_workspace_size(M, H, 1, 2 * inter, jf.JF_BF16), 1),
                      dtype=torch.uint8, device="cuda")
    ws2 = torch.empty(max(jf.jf_fuse_proj_workspace_size(M, inter, 1, H, jf.JF_BF16), 1),
                      dtype=torch.uint8, device="cuda")
    t_gu = graph_time(lambda: jf.jf_fuse_proj([x], w_gu, y=gu, workspace=ws1), steps, torch, rep=5)
    t_act = graph_time(lambda: jf.jf_swiglu(gu, y=act), steps, torch)
    t_dn = graph_time(lambda: jf.jf_fuse_proj([act], w_dn, y=out, workspace=ws2), steps, torch, rep=5)
    wbytes = (w_gu.numel() + w_dn.numel()) * 2
    total = t_gu + t_act + t_dn
    res = {"rows": M, "hidden": H, "intermediate": inter, "gate_up_ms": round(t_gu, 5),
           "swiglu_ms": round(t_act, 5), "down_ms": round(t_dn, 5), "ms": round(total, 5),
           "weight_bytes": wbytes, "weight_GBps": round(wbytes / (total * 1e-3) / 1e9, 1),
           "swiglu_GBps": round(3 * M * inter * 2 / (t_act * 1e-3) / 1e9, 1)}
    del w_gu, w_dn, gu, act
    return res


def rope_timing(wl, q, k_tree, depth, prefix_len, steps, torch, jf):
    """jf_tree_rope over the step's queries and tree keys (copies), at the
    tree positions; latency-bound, timed as a HIP graph of 20 calls."""
    qc, kc = q.clone(), k_tree.clone()
    pl = torch.from_numpy(np.asarray(prefix_len, np.int32)).cuda()
    REP = 20
    jf.jf_tree_rope(qc, kc, depth, pl)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(REP):
            jf.jf_tree_rope(qc, kc, depth, pl)
    for _ in range(3):
        g.replay()
    torch.cuda.synchronize()
    ms = []
    for _ in range(max(5, steps // REP)):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        g.replay()
        e1.record()
        torch.cuda.synchronize()
        ms.append(e0.elapsed_time(e1) / REP)
    nbytes = 2 * (qc.numel() + kc.numel()) * qc.element_size()
    t = float(np.mean(ms))
    return {"ms": round(t, 5), "bytes": nbytes, "GBps": round(nbytes / (t * 1e-3) / 1e9, 1),
            "bound": "latency", "timing": f"graph of {REP} back-to-back calls"}


def wl_id(wl):
    from tree_causal_draft_parent_amd import synth
    return next(i for i, w in synth.WORKLOADS.items() if w.name == wl.name)


def projection_context(wl, M, steps, torch, jf):
    """The fused projection over one row per prefix token (M = sum of prefix
    lengths): the MFMA-bound use of the same call. Inputs are seeded device
    normals; only the time is used."""
    tdt = torch.bfloat16 if wl.dtype == "bf16" else torch.float32
    g = torch.Generator(device="cuda")
    g.manual_seed(1000 + M)
    xs = [(torch.randn((M, wl.H), generator=g, device="cuda")).to(tdt) for _ in range(wl.n_fused)]
    w = (0.02 * torch.randn((wl.H, wl.n_fused * wl.H), generator=g, device="cuda")).to(tdt)
    y = torch.empty((M, wl.H), dtype=tdt, device="cuda")
    ws = torch.empty(max(jf.jf_fuse_proj_workspace_size(M, wl.H, wl.n_fused, wl.H,
                                                        jf.JF_BF16 if wl.dtype == "bf16" else jf.JF_F32), 1),
                     dtype=torch.uint8, device="cuda")
    for _ in range(3):
        jf.jf_fuse_proj(xs, w, y=y, workspace=ws)
    n = max(1, min(steps, 20))
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(n):
        jf.jf_fuse_proj(xs, w, y=y, workspace=ws)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / n
    flops = 2 * M * wl.H * wl.n_fused * wl.H
    tfs = flops / (ms * 1e-3) / 1e12
    return {"M": M, "ms": round(ms, 5), "TFLOPs": round(tfs, 2), "mfma_frac": round(tfs / BF16_PEAK_TFLOPS, 4),
            "flops": flops, "launches": n}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the library has no multi-GPU path).", file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration()
        return
    import torch
    from tree_causal_draft_parent_amd import jf, synth
    if args.attention_records_only:
        flush = torch.ones(FLUSH_BYTES // 4, dtype=torch.float32, device="cuda")
        print(json.dumps({"workloads": attention_records(args.steps, torch, jf, flush)}), flush=True)
        return

    wl = synth.workload(args.workload)
    inp = synth.make_workload(args.workload)
    dt = wl.dtype
    tdt = torch.bfloat16 if dt == "bf16" else torch.float32
    a = inp["attn"]
    dev = {k: to_dev(a[k], dt, torch) for k in ("q", "k_tree", "v_tree", "k_cache", "v_cache")}
    parent = torch.from_numpy(a["parent"]).cuda()
    block_table = torch.from_numpy(a["block_table"]).cuda()
    prefix_len = a["prefix_len"]
    xt = to_dev(inp["fuse"]["x"], dt, torch)
    xs = [xt[l] for l in range(wl.n_fused)]
    w = to_dev(inp["fuse"]["w"], dt, torch)
    logits = to_dev(inp["logits"], dt, torch)

    B, N = wl.B, wl.N
    W = (N + 63) // 64
    mask = torch.empty((B, N, W), dtype=torch.int64, device="cuda")
    depth = torch.empty((B, N), dtype=torch.int32, device="cuda")
    seq_status = torch.empty((B,), dtype=torch.int32, device="cuda")
    fuse_out_dtype = tdt
    y = torch.empty((B * N, wl.H), dtype=fuse_out_dtype, device="cuda")
    fws = jf.jf_fuse_proj_workspace_size(B * N, wl.H, wl.n_fused, wl.H, jf.JF_BF16 if dt == "bf16" else jf.JF_F32)
    fuse_ws = torch.empty(max(fws, 1), dtype=torch.uint8, device="cuda")
    out = torch.empty_like(dev["q"])
    lse = torch.empty((B, N, wl.Hq), dtype=torch.float32, device="cuda")
    aws = jf.jf_tree_attn_workspace_size(B, N, wl.Hq, wl.Hkv, wl.D, a["page_size"], prefix_len,
                                         jf.JF_BF16 if dt == "bf16" else jf.JF_F32)
    attn_ws = torch.empty(max(aws, 1), dtype=torch.uint8, device="cuda")
    R = B * N
    idx = torch.empty((R, wl.topk), dtype=torch.int32, device="cuda")
    val = torch.empty((R, wl.topk), dtype=torch.float32, device="cuda")
    rlse = torch.empty((R,), dtype=torch.float32, device="cuda")
    tws = jf.jf_node_topk_workspace_size(R, wl.V, wl.topk)
    topk_ws = torch.empty(max(tws, 1), dtype=torch.uint8, device="cuda")
    page_status = torch.zeros(1, dtype=torch.int32, device="cuda")

    calls = ["mask", "fuse", "attn", "topk"]

    def step(ev=None):
        if ev is not None:
            ev[0].record()
        jf.jf_tree_mask_build(parent, mask, depth, seq_status)
        if ev is not None:
            ev[1].record()
        jf.jf_fuse_proj(xs, w, y=y, workspace=fuse_ws)
        if ev is not None:
            ev[2].record()
        jf.jf_tree_attn_fwd(dev["q"], dev["k_tree"], dev["v_tree"], mask, dev["k_cache"],
                            dev["v_cache"], block_table, prefix_len, out=out, lse=lse,
                            workspace=attn_ws, status=page_status)
        if ev is not None:
            ev[3].record()
        jf.jf_node_topk(logits, wl.topk, idx=idx, val=val, lse=rlse, workspace=topk_ws)
        if ev is not None:
            ev[4].record()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    print(f"[bench] workload {wl.name}: warmup done", file=sys.stderr, flush=True)

    # ---- timed region: K back-to-back steps --------------------------------
    K = args.steps
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(K)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(K):
        step(evs[k])
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    eager_ms_per_step = (t1 - t0) * 1e3 / K
    call_ms = {c: [evs[k][i].elapsed_time(evs[k][i + 1]) for k in range(K)] for i, c in enumerate(calls)}
    per_call = {c: float(np.mean(v)) for c, v in call_ms.items()}
    gpu_step_ms = float(np.mean([evs[k][0].elapsed_time(evs[k][4]) for k in range(K)]))
    print(f"[bench] eager: {K} steps, {eager_ms_per_step:.4f} ms/step", file=sys.stderr, flush=True)

    # ---- the step as one HIP graph: captured once, replayed K times ----------
    # (the host-side launch work of the eager loop is what a serving loop
    # removes this way; the replayed kernels and their arguments are the same)
    # The same step on two streams: the projection and then the top-k on a
    # second stream beside the mask and then the attention (the projection and
    # the top-k depend on neither).  The calls of one stream fill each other's
    # tails, and the small kernels (split-K reduce, split merge) overlap the
    # other stream's work.  Same kernels, same arguments.
    s_side = torch.cuda.Stream()
    # The projection's K split and the attention's key splits can be planned
    # for fewer compute units than the chip has (fewer, longer splits): the
    # units they leave go to the other stream, and they write fewer partial
    # results.  The plans tried are listed below.
    n_cus = torch.cuda.get_device_properties(0).multi_processor_count
    # top-k rows [0, r_split) follow the projection, [r_split, R) the attention
    r_split = R - int(round(R * min(max(args.topk_split, 0.0), 1.0)))
    f_b = (R - r_split) / R
    shorter = (per_call["mask"] + per_call["attn"] + f_b * per_call["topk"]
               < per_call["fuse"] + (1 - f_b) * per_call["topk"])
    code = jf.JF_BF16 if dt == "bf16" else jf.JF_F32
    topk_ws_b = torch.empty(max(jf.jf_node_topk_workspace_size(max(R - r_split, 1), wl.V, wl.topk), 1),
                            dtype=torch.uint8, device="cuda")

    s_third = torch.cuda.Stream()

    def make_step_streams(fuse_cus, attn_cus, topk_apart=False):
        """The multi-stream step with the projection's K split planned for
        fuse_cus compute units and the attention's key splits for attn_cus
        (0: all), each with its own workspace.  topk_apart: the top-k on a
        third stream of its own instead of after the projection."""
        aws = jf.jf_tree_attn_workspace_size(B, N, wl.Hq, wl.Hkv, wl.D, a["page_size"], prefix_len,
                                             code, attn_cus)
        attn_ws_s = torch.empty(max(aws, 1), dtype=torch.uint8, device="cuda")
        fws = jf.jf_fuse_proj_workspace_size(B * N, wl.H, wl.n_fused, wl.H, code, fuse_cus)
        fuse_ws_s = torch.empty(max(fws, 1), dtype=torch.uint8, device="cuda")

        def step_streams():
            main = torch.cuda.current_stream()
            s_side.wait_stream(main)
            if topk_apart:
                s_third.wait_stream(main)
            with torch.cuda.stream(s_side):
                jf.jf_fuse_proj(xs, w, y=y, workspace=fuse_ws_s, cus=fuse_cus)
            with torch.cuda.stream(s_third if topk_apart else s_side):
                if r_split > 0:
                    jf.jf_node_topk(logits[:r_split], wl.topk, idx=idx[:r_split], val=val[:r_split],
                                    lse=rlse[:r_split], workspace=topk_ws)
            jf.jf_tree_mask_build(parent, mask, depth, seq_status)
            jf.jf_tree_attn_fwd(dev["q"], dev["k_tree"], dev["v_tree"], mask, dev["k_cache"],
                                dev["v_cache"], block_table, prefix_len, out=out, lse=lse,
                                workspace=attn_ws_s, status=page_status, cus=attn_cus)
            if r_split < R:
                jf.jf_node_topk(logits[r_split:], wl.topk, idx=idx[r_split:], val=val[r_split:],
                                lse=rlse[r_split:], workspace=topk_ws_b)
            main.wait_stream(s_side)
            if topk_apart:
                main.wait_stream(s_third)

        return step_streams

    # Compute-unit budgets of the two streams.  Given on the command line they
    # are used as they are; otherwise a few plans are timed briefly as graphs
    # and the fastest is kept:
    #   "three_quarters": the projection's K split for 3/4 of the units, the
    #       attention for 3/4 when mask + attention is the shorter stream;
    #   "fit_together": 1/2 and 3/8, so both streams' workgroups fit on the
    #       chip at once (the attention's fewer, longer splits leave units to
    #       the projection and the top-k);
    #   "fuse_half": 1/2 for the projection, all units for the attention;
    #   "fit_five_eighths": 5/8 and 3/8;
    #   "fit_nine_sixteenths": 9/16 and 7/16;
    #   "topk_apart": as fuse_half, the top-k on a third stream of its own.
    # The 16-node workload (id 1) times the one-stream graph only.  Its step
    # is launch-bound and every multi-stream plan measured slower than one
    # stream (66.7-108.4 us against 58.3 us), and one run of its multi-stream
    # plan loop ended in a host segmentation fault whose cause is not known
    # (an ASan/UBSan host build of every planner and workspace query at its
    # shapes and budgets found nothing), so that loop is not run for it.
    multi_stream_ok = wl_id(wl) != 1
    if not multi_stream_ok:
        plans = {"one_stream_only": (0, 0, False)}
    elif args.attn_cus >= 0 or args.fuse_cus >= 0:
        plans = {"given": ((3 * n_cus) // 4 if args.fuse_cus < 0 else args.fuse_cus,
                           (((3 * n_cus) // 4 if shorter else 0) if args.attn_cus < 0 else args.attn_cus),
                           False)}
    else:
        plans = {"three_quarters": ((3 * n_cus) // 4, (3 * n_cus) // 4 if shorter else 0, False),
                 "fit_together": (n_cus // 2, (3 * n_cus) // 8, False),
                 "fuse_half": (n_cus // 2, 0, False),
                 "fit_five_eighths": ((5 * n_cus) // 8, (3 * n_cus) // 8, False),
                 "fit_nine_sixteenths": ((9 * n_cus) // 16, (7 * n_cus) // 16, False),
                 "topk_apart": (n_cus // 2, 0, True)}

    # A graph holds S consecutive steps.  Each step's streams join before the
    # next step forks, so the steps run one after another exactly as in a
    # draft loop that grows its tree over several steps per verification and
    # captures them together; what S > 1 saves is the launch of a graph per
    # step (its first kernels wait for the previous graph's last ones).
    S = max(1, args.steps_per_graph)

    def time_graph(fn, reps=None, per_graph=None):
        """Time `reps` steps of fn: reps // S replays of a graph of S steps,
        then one replay of a graph of the remaining reps % S steps."""
        reps = K if reps is None else reps
        per_graph = S if per_graph is None else per_graph
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            fn()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        graphs = []
        for n in (per_graph, reps % per_graph):
            if n == 0:
                graphs.append(None)
                continue
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                for _ in range(n):
                    fn()
            graphs.append(g)
        graph, tail = graphs
        for _ in range(args.warmup):
            graph.replay()
        if tail is not None:
            tail.replay()
        torch.cuda.synchronize()
        a0 = time.perf_counter()
        for _ in range(reps // per_graph):
            graph.replay()
        if tail is not None:
            tail.replay()
        torch.cuda.synchronize()
        a1 = time.perf_counter()
        return a0, a1

    ms_per_step = eager_ms_per_step
    serial_graph_ms = None
    one_step_graph_ms = None
    plan_ms = {}
    plan = next(iter(plans))
    fuse_cus, attn_cus, topk_apart = plans[plan]
    if not args.eager:
        g0, g1 = time_graph(step)
        serial_graph_ms = (g1 - g0) * 1e3 / K
        print(f"[bench] graph, one stream: {K} steps, {S} a graph, {serial_graph_ms:.4f} ms/step",
              file=sys.stderr, flush=True)
        chosen = step
        if args.one_stream or not multi_stream_ok:
            t0, t1 = g0, g1
            plan = "one_stream"
            fuse_cus, attn_cus, topk_apart = 0, 0, False
        else:
            if len(plans) > 1:
                for name, (fc, ac, ta) in plans.items():
                    p0, p1 = time_graph(make_step_streams(fc, ac, ta), reps=max(20, K // 5))
                    plan_ms[name] = round((p1 - p0) * 1e3 / max(20, K // 5), 5)
                # the one-stream graph (already timed over K replays) competes too:
                # for a small step the cross-stream waits cost more than they overlap
                plan_ms["one_stream"] = round(serial_graph_ms, 5)
                plan = min(plan_ms, key=plan_ms.get)
                print(f"[bench] step plans (ms/step): {plan_ms}; using {plan}", file=sys.stderr,
                      flush=True)
            if plan == "one_stream":
                t0, t1 = g0, g1
                fuse_cus, attn_cus, topk_apart = 0, 0, False
            else:
                fuse_cus, attn_cus, topk_apart = plans[plan]
                chosen = make_step_streams(fuse_cus, attn_cus, topk_apart)
                t0, t1 = time_graph(chosen)
        ms_per_step = (t1 - t0) * 1e3 / K
        print(f"[bench] graph: {K} steps, {S} a graph, {ms_per_step:.4f} ms/step", file=sys.stderr, flush=True)
        if S > 1:
            o0, o1 = time_graph(chosen, per_graph=1)
            one_step_graph_ms = (o1 - o0) * 1e3 / K
            print(f"[bench] graph of one step, same plan: {one_step_graph_ms:.4f} ms/step",
                  file=sys.stderr, flush=True)

    # ---- cold-cache steps: evict the last-level cache before each step -------
    flush_buf = torch.ones(FLUSH_BYTES // 4, dtype=torch.float32, device="cuda")
    cold = []
    cold_call = {c: [] for c in calls}
    for k in range(args.cold_steps):
        flush_cache(flush_buf)
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(5)]
        step(ev)
        torch.cuda.synchronize()
        cold.append(ev[0].elapsed_time(ev[4]))
        for i, c in enumerate(calls):
            cold_call[c].append(ev[i].elapsed_time(ev[i + 1]))
    assert int(page_status.item()) == 0 and bool((seq_status == -1).all())
    records = None
    if not args.no_attention_records:
        records = attention_records(K, torch, jf, flush_buf)
    del flush_buf
    copy_gbs = copy_bandwidth(torch)
    print(f"[bench] device copy: {copy_gbs:.1f} GB/s", file=sys.stderr, flush=True)
    proj_ctx = None
    if not args.no_context_projection:
        proj_ctx = projection_context(wl, int(np.sum(prefix_len)), K, torch, jf)
        print(f"[bench] context projection: M={proj_ctx['M']} {proj_ctx['ms']:.4f} ms", file=sys.stderr, flush=True)

    growth = None
    if not args.no_tree_growth:
        growth = tree_growth(wl, parent, depth, idx, val, rlse, K, torch, jf,
                             parent_np=a["parent"], logits=logits)
        print(f"[bench] tree growth: path scores {growth['path_scores']['ms']:.4f} ms, "
              f"expansion {growth['tree_expand']['ms']:.4f} ms, acceptance "
              f"{growth['tree_accept']['ms']:.4f} ms, target top-1 {growth['target_argmax']['ms']:.4f} ms",
              file=sys.stderr, flush=True)

    head = None
    if not args.no_lm_head:
        rope = rope_timing(wl, dev["q"], dev["k_tree"], depth, prefix_len, K, torch, jf)
        head = lm_head(wl, K, torch, jf)
        if head is not None:
            head["rope"] = rope
            head["rmsnorm"] = norm_timing(wl, dev["q"], dev["k_tree"], K, torch, jf)
            head["mlp"] = mlp_timing(wl, K, torch, jf)
        if head is not None:
            print(f"[bench] LM head {head['M']}x{head['K']}->{head['N']}: {head['ms']:.4f} ms, "
                  f"{head['hbm_GBps']:.0f} GB/s", file=sys.stderr, flush=True)

    sweep = None
    if args.topk_sweep:
        sweep = topk_sweep(logits, K, torch, jf)
        print(f"[bench] top-k sweep (ms): " + ", ".join(f"{c} {v['ms']:.4f}" for c, v in sweep.items()
                                                        if isinstance(v, dict)),
              file=sys.stderr, flush=True)

    def med(v):
        return float(np.median(v)) if len(v) else float("nan")

    alg = algorithmic(wl, inp, 2 if fuse_out_dtype == torch.bfloat16 else 4)

    def bound_c(c):
        # the roofline that binds each call, from its arithmetic intensity
        if c == "mask":
            return "latency"
        if wl.dtype == "f32" and c in ("fuse", "attn"):
            return "alu"                      # fp32 vector arithmetic
        return bound_of(alg[c]["flops"], alg[c]["bytes"])

    def roof(c, ms):
        sec = ms * 1e-3
        return alg[c]["bytes"] / sec / 1e9, alg[c]["flops"] / sec / 1e12

    PEAKS = {"hbm": (HBM_PEAK_GBS, "GB/s"), "mfma": (BF16_PEAK_TFLOPS, "TFLOP/s"),
             "alu": (FP32_VECTOR_PEAK_TFLOPS, "TFLOP/s")}

    def achieved(c, ms):
        gbs, tfs = roof(c, ms)
        return gbs if bound_c(c) == "hbm" else tfs

    # Rooflines come from the flushed per-call medians (a 512 MiB read before
    # each step evicts the last-level cache, so every call starts from HBM);
    # the warm (back-to-back) figures are reported beside them.
    have_cold = args.cold_steps > 0
    cold_ms = {c: med(cold_call[c]) for c in calls}
    prim = cold_ms if have_cold else per_call
    dom = max(("fuse", "attn", "topk"), key=lambda c: prim[c])
    b = bound_c(dom)
    peak, unit = PEAKS[b]
    traffic, traffic_src = measured_traffic(dom, wl.name)
    roofline = {"bound": b, "achieved": round(achieved(dom, prim[dom]), 2), "peak": peak, "unit": unit,
                "frac": round(achieved(dom, prim[dom]) / peak, 4), "traffic": traffic,
                "traffic_source": traffic_src,
                "timing": ("flushed: median per-call HIP-event time over the cold steps (a 512 MiB "
                           "read before each step)" if have_cold else
                           "warm: mean per-call HIP-event time of back-to-back eager steps"),
                "kernels": [k for k in KERNELS[dom]],
                "avg_launch_us": round(prim[dom] * 1e3, 2),
                "warm": {"achieved": round(achieved(dom, per_call[dom]), 2),
                         "frac": round(achieved(dom, per_call[dom]) / peak, 4),
                         "avg_launch_us": round(per_call[dom] * 1e3, 2)},
                "kernel": {"fuse": "jf_fuse_proj (k_fuse_gemm_bf16 + k_fuse_reduce)",
                           "attn": "jf_tree_attn_fwd (k_tree_attn_split + k_tree_attn_merge)",
                           "topk": "jf_node_topk (k_topk_stage1 + k_topk_stage2)"}[dom],
                "algorithmic": {"bytes": alg[dom]["bytes"], "flops": alg[dom]["flops"],
                                "flop_per_byte": round(alg[dom]["flops"] / alg[dom]["bytes"], 1)}}

    def call_block(c):
        gbs, tfs = roof(c, prim[c])
        wgbs, wtfs = roof(c, per_call[c])
        bc = bound_c(c)
        d = {"ms": round(prim[c], 5), "cold_ms": round(cold_ms[c], 5), "warm_ms": round(per_call[c], 5),
             "bound": bc, "hbm_GBps": round(gbs, 1), "hbm_frac": round(gbs / HBM_PEAK_GBS, 4),
             "TFLOPs": round(tfs, 2), "mfma_frac": round(tfs / BF16_PEAK_TFLOPS, 4),
             "warm_hbm_frac": round(wgbs / HBM_PEAK_GBS, 4), "warm_mfma_frac": round(wtfs / BF16_PEAK_TFLOPS, 4)}
        if bc in PEAKS:
            d["frac_of_bound"] = round(achieved(c, prim[c]) / PEAKS[bc][0], 4)
        return d

    tree_attn = call_block("attn")
    tree_attn.update(nodes_per_s=round(B * N / (prim["attn"] * 1e-3), 1), algorithmic=alg["attn"],
                     # the prefix K/V stream alone (2 * sum(P) * Hkv * D elements),
                     # the part the attention must bring from HBM
                     prefix_kv_bytes=alg["attn_prefix_kv_bytes"],
                     prefix_kv_GBps=round(alg["attn_prefix_kv_bytes"] / (prim["attn"] * 1e-3) / 1e9, 1))
    projection = call_block("fuse")
    projection["algorithmic"] = alg["fuse"]
    calls_out = {}
    for c in calls:
        p10, p50, p90 = np.percentile(call_ms[c], [10, 50, 90])
        calls_out[c] = call_block(c)
        calls_out[c].update(p10_ms=round(float(p10), 5), p50_ms=round(float(p50), 5),
                            p90_ms=round(float(p90), 5))
        if calls_out[c]["bound"] == "hbm":
            calls_out[c]["frac_of_copy"] = round(roof(c, prim[c])[0] / copy_gbs, 4)

    cpu = None
    if not args.no_cpu_baseline:
        print("[bench] timing the oracle on host cores", file=sys.stderr, flush=True)
        cpu = cpu_baseline(wl, inp, args.cpu_sample_nodes)
        cpu["one_thread"] = cpu_baseline_one_thread(wl, inp, max(1, args.cpu_sample_nodes // 16))

    value = B * N * K / (t1 - t0)
    rec = {
        "metric": METRIC, "value": round(value, 1), "unit": "nodes/s", "n_gpus": 1, "steps": K,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": wl.dtype, "data": "synthetic",
        "config": {"workload": wl.name, "batch": B, "prefix": int(np.max(prefix_len)), "tree_nodes": N,
                   "q_heads": wl.Hq, "kv_heads": wl.Hkv, "head_dim": wl.D, "hidden": wl.H,
                   "fused_layers": wl.n_fused, "vocab": wl.V, "topk": wl.topk,
                   "step": "mask+fuse_proj+tree_attn+topk"},
        "launch": ("eager" if args.eager else
                   "hip_graph" if args.one_stream or plan == "one_stream" else
                   "hip_graph_3_streams" if topk_apart else "hip_graph_2_streams"),
        "steps_per_graph": None if args.eager else S,
        "graph_one_step_ms_per_step": (None if args.eager else
                                       round(ms_per_step if S == 1 else one_step_graph_ms, 5)),
        "graph_one_stream_ms_per_step": None if serial_graph_ms is None else round(serial_graph_ms, 5),
        "attn_cus_two_streams": attn_cus,
        "step_plan": plan,
        "topk_own_stream": topk_apart,
        "step_plans_ms": plan_ms or None,
        "fuse_cus_two_streams": fuse_cus,
        "topk_rows_on_attention_stream": R - r_split,
        "eager_ms_per_step": round(eager_ms_per_step, 5),
        "gpu_step_ms": round(gpu_step_ms, 5),
        "cold_step_ms": round(med(cold), 5),
        "cold_nodes_per_s": round(B * N / (med(cold) * 1e-3), 1),
        "calls": calls_out,
        "tree_attn": tree_attn,
        "projection": projection,
        "projection_context": proj_ctx,
        "tree_growth": growth,
        "draft_layer": head,
        "topk_sweep": sweep,
        "copy_GBps": round(copy_gbs, 1),
        "workloads": records,
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
