"""Benchmark of the chain verification step on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

Workload: the batched chain verification, B=64 requests, gamma=4, V=128256,
bf16 logits; even requests sample at T=0.7, odd requests are greedy (draft
noise sigma ~ U[0.3, 2.0]).  A step is one spec_verify_chain_hinted call
over one batch: the host passes which requests sample (a mask built once from
the temperatures it set), which lets the GPU stream the sampling requests
first and draw them while the greedy rows stream; the same calls without the
hint are timed too (`without_hint`; `--no-hint` makes them the headline).
Inputs sit in HBM before timing starts; calls rotate over R copies of the
batch (more than 512 MB together) so each call reads cold data rather than
the 256 MB Infinity Cache.

Prints one JSON line: verified (request x position) rows per second, the
achieved algorithmic HBM bandwidth against the 8 TB/s peak, and the fp64
oracle timed on this host's cores on a bounded sample.

Other workloads (--workload) report the same line for the single-request
latency case (B=1, V=32000, also replayed from a HIP graph), the deep case
(B=256, gamma=8, V=151936, Zipf logits), the batched inputs as a ragged call
(request b drafts 1 + b % 4 tokens; rows are the rounds' own rows), the
batched inputs under a consistent top-k filter (k=50 on p and q), the
batched inputs under consistent top-p 0.9 over the whole vocabulary
(spec_verify_chain_filtered), the token-tree cases (B=32, 64 nodes, greedy,
naive sampling or multi-step speculative sampling; rows are node rows) and
the tree attention mask builder on the same tree shape (rows are mask rows).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import subprocess
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "verified (request×position) rows/sec and achieved HBM GB/s vs peak, 1 GPU"
PEAK_HBM_GBPS = 8000.0
MALL_BYTES = 256 << 20


def read_bytes(ci, gammas=None) -> int:
    """Logit bytes the path must read once: 2*g+1 rows of a sampling request
    (g+1 target, g draft), g+1 target rows of a greedy one, g being gamma or
    the request's own length in a ragged call."""
    es = 2 if ci.dtype == "bf16" else 4
    g = [ci.gamma] * ci.B if gammas is None else [int(x) for x in gammas]
    rows = sum((2 * g[b] + 1) if float(ci.temperature[b]) > 0 else (g[b] + 1) for b in range(ci.B))
    return rows * ci.V * es


RAGGED_LENGTHS = (1, 2, 3, 4)    # request b drafts RAGGED_LENGTHS[b % 4] tokens


def small_bytes(ci) -> int:
    """Tokens, uniforms, temperature read and emitted tokens / counts written."""
    return ci.B * (4 * ci.gamma + 4 * (ci.gamma + 1) + 4 + 4 * (ci.gamma + 1) + 4)


# Sources of each kernel whose HBM traffic is stored under profiles/.
KERNEL_SOURCES = {
    "chain_verify": ("rejection_sampling_verify_15_amd/csrc/sv_chain.hip",
                     "rejection_sampling_verify_15_amd/csrc/sv_device.hpp"),
    "filter_rows": ("rejection_sampling_verify_15_amd/csrc/sv_filter.hip",
                    "rejection_sampling_verify_15_amd/csrc/sv_device.hpp"),
    "topk_rows": ("rejection_sampling_verify_15_amd/csrc/sv_topk.hip",
                  "rejection_sampling_verify_15_amd/csrc/sv_device.hpp"),
}
# The stored counter summary of each workload.
TRAFFIC_FILES = {"batched": "traffic_batched_chain.json", "deep": "traffic_deep_chain.json",
                 "single": "traffic_single_chain.json", "topp": "traffic_topp_filter.json",
                 "topk": "traffic_topk_rows.json"}


def source_digest(kernel: str = "chain_verify") -> str:
    """Hash of a kernel's sources; a stored traffic figure is valid only for
    the sources it was measured on."""
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES[kernel]:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def stored_traffic(workload: str, kernel: str):
    """HBM bytes per launch of `kernel` in `workload` from the committed
    rocprofv3 counter summary, or None when it is missing or the kernel's
    sources changed since."""
    name = TRAFFIC_FILES.get(workload)
    if name is None:
        return None
    try:
        with open(os.path.join(ROOT, "profiles", name)) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    k = rec.get("kernels", {}).get(kernel)
    if k is None or k.get("source_sha256") != source_digest(k.get("digest_of", kernel)):
        return None
    return k.get("traffic_bytes_per_launch")


TOPK = 50                        # k of every sampling request in the top-k workload
TOPP = 0.9                       # p of every sampling request in the top-p workload


WORKLOADS = ("batched", "single", "deep", "ragged", "topk", "topp", "tree-greedy", "tree-sampling", "tree-mss", "tree-mask")


def percentiles(xs):
    xs = np.sort(np.asarray(xs, dtype=np.float64))
    return {f"p{q}": float(np.percentile(xs, q)) for q in (10, 50, 90, 99)}


def time_calls(torch, stream, step, k):
    """The timed region: k calls between two events (ms), and the host time
    spent enqueueing them (us per call)."""
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    a.record(stream)
    h0 = time.perf_counter()
    for i in range(k):
        step(i)
    host_us = 1e6 * (time.perf_counter() - h0) / k
    b.record(stream)
    torch.cuda.synchronize()
    return a.elapsed_time(b), host_us


def per_call_us(torch, stream, step, k):
    """Device time of each call from an event recorded between consecutive
    calls (the events add a little to each)."""
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(k + 1)]
    torch.cuda.synchronize()
    ev[0].record(stream)
    for i in range(k):
        step(i)
        ev[i + 1].record(stream)
    torch.cuda.synchronize()
    return [1e3 * ev[i].elapsed_time(ev[i + 1]) for i in range(k)]


def chain_case(name, synth):
    if name == "batched":
        return synth.batched_chain(), ("batched chain verify: B=64, gamma=4, V=128256, bf16 logits, "
                                       "even requests sample at T=0.7, odd requests greedy")
    if name == "ragged":
        return synth.batched_chain(), ("ragged chain verify: the batched inputs (B=64, gamma padded to 4, "
                                       "V=128256, bf16, even requests T=0.7, odd greedy) with request b "
                                       "drafting 1 + b % 4 tokens")
    if name == "topk":
        ci = synth.batched_chain()
        ci.draft_tokens = synth.topk_draft_tokens(ci, np.full(ci.B, TOPK), 51_000)
        return ci, ("consistent top-k chain verify: the batched inputs (B=64, gamma=4, V=128256, bf16, even "
                    f"requests T=0.7, odd greedy), p and q of every sampling request filtered to k={TOPK}, "
                    "draft tokens drawn from the filtered draft rows")
    if name == "topp":
        ci = synth.batched_chain()
        ci.draft_tokens = synth.topp_draft_tokens(ci, np.full(ci.B, TOPP, np.float32), 52_000)
        return ci, ("consistent top-p chain verify over the whole vocabulary: the batched inputs (B=64, gamma=4, "
                    f"V=128256, bf16, even requests T=0.7, odd greedy), p and q of every sampling request cut to "
                    f"their top-p={TOPP} mass, draft tokens drawn from the cut draft rows")
    if name == "single":
        return synth.single_chain(), ("single-request chain verify: B=1, gamma=4, V=32000, bf16 logits, "
                                      "T=1, fixed logits with fresh uniforms every call (latency)")
    return synth.deep_chain(), ("deep chain verify: B=256, gamma=8, V=151936, bf16 Zipf logits, T=1")


def run_chain(args, torch, synth, sv):
    dev = torch.device("cuda:0")
    ci, desc = chain_case(args.workload, synth)
    set_bytes = ci.target.nbytes + ci.draft.nbytes
    # the single-request case is latency-bound and meant to run from cache;
    # the others rotate over enough copies to read past the Infinity Cache
    R = 1 if args.workload == "single" else max(2, math.ceil(2 * MALL_BYTES / set_bytes) + 1)

    def dl(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)
    tgt0, drf0 = dl(ci.target), dl(ci.draft)
    sets = [(tgt0, drf0)] + [(tgt0.clone(), drf0.clone()) for _ in range(R - 1)]
    tok = torch.from_numpy(ci.draft_tokens.astype(np.int32)).to(dev)
    n_u = 64 if args.workload == "single" else 1
    u_sets = [torch.from_numpy(ci.uniforms if j == 0 else ci.fresh_uniforms(50_000 + j)).to(dev) for j in range(n_u)]
    T = torch.from_numpy(ci.temperature).to(dev)
    out_t = torch.empty((ci.B, ci.gamma + 1), dtype=torch.int32, device=dev)
    out_n = torch.empty((ci.B,), dtype=torch.int32, device=dev)
    topk = args.workload == "topk"
    topp = args.workload == "topp"
    pp_d = torch.from_numpy(np.full(ci.B, TOPP, np.float32)).to(dev) if topp else None
    ws_query = (sv.lib().sv_chain_topk_workspace_bytes if topk else
                sv.lib().sv_chain_filtered_workspace_bytes if topp else sv.lib().sv_chain_workspace_bytes)
    ws_bytes = ws_query(ci.B, ci.gamma, ci.V, sv.SV_BF16)
    ws = sv.workspace(ws_bytes, dev)
    stream = torch.cuda.current_stream(dev)
    ragged = args.workload == "ragged"
    k_np = np.full(ci.B, TOPK, np.int32)
    k_d = torch.from_numpy(k_np).to(dev)
    p_np = np.full(ci.B, args.top_p, np.float32) if topk and args.top_p is not None else None
    p_d = torch.from_numpy(p_np).to(dev) if p_np is not None else None
    gam = np.array([RAGGED_LENGTHS[b % len(RAGGED_LENGTHS)] for b in range(ci.B)], np.int32) if ragged else None
    gam_d = torch.from_numpy(gam).to(dev) if ragged else None
    # the batched call passes which requests sample (host data a serving
    # scheduler holds), built once; it only reorders the work on the GPU
    hinted = args.workload == "batched" and not args.no_hint
    hint = sv.binding.sampling_hint_array(ci.temperature > 0, ci.B) if hinted else None

    # plain chain calls go through prepared calls (the binding's checks done
    # once per input set, as a serving loop reusing its buffers would)
    plain_chain = not (ragged or topk or topp)
    prepared = ([[sv.prepare_chain(t, d, tok, u_sets[j], T, out_t, out_n, ws, sampling_hint=hint)
                  for j in range(n_u)] for (t, d) in sets] if plain_chain else None)

    def step(i):
        t, d = sets[i % R]
        if plain_chain:
            prepared[i % R][i % n_u]()
        elif ragged:
            sv.verify_chain_ragged(t, d, tok, u_sets[i % n_u], T, gam_d, ws=ws)
        elif topk:
            sv.verify_chain_topk(t, d, tok, u_sets[i % n_u], T, k_d, top_p=p_d, ws=ws)
        elif topp:
            sv.verify_chain_filtered(t, d, tok, u_sets[i % n_u], T, None, pp_d, out_tokens=out_t,
                                     out_num_accepted=out_n, ws=ws)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    total_ms, host_us = time_calls(torch, stream, step, args.steps)
    # the same steps again with a pair of events attached to every kernel
    # dispatch: per-kernel durations (the attached events add a few
    # microseconds between launches, so the whole-call figure comes from the
    # region above)
    with sv.KernelTimer(4 * args.steps) as kt:
        events_ms, _ = time_calls(torch, stream, step, args.steps)
    calls = per_call_us(torch, stream, step, min(args.steps, 2000))

    rows = ci.B * (ci.gamma + 1) if gam is None else int(np.sum(gam + 1))
    rd, sm = read_bytes(ci, gam), small_bytes(ci)
    call_us = 1e3 * total_ms / args.steps
    dominant = "topk_rows" if topk else "chain_verify"
    rd_kernel = rd   # algorithmic bytes of one launch of the dominant kernel
    if topp and kt.ms["filter_rows"] > kt.ms["chain_verify"]:
        # the cuts' launch reads the sampling requests' rows only
        dominant = "filter_rows"
        rd_kernel = sum((2 * ci.gamma + 1) * ci.V * 2 for b in range(ci.B) if float(ci.temperature[b]) > 0)
    k_us = kt.mean_us(dominant)
    if dominant == "filter_rows":
        # the cuts take one launch per digit: all of them together against one
        # read of the rows they cut
        k_us = 1e3 * kt.ms["filter_rows"] / args.steps
    achieved = rd_kernel / (k_us * 1e-6) / 1e9
    cfg = {"workload": desc, "B": ci.B, "gamma": ci.gamma, "V": ci.V, "rotating_input_sets": R}
    if hinted:
        cfg["sampling_hint"] = "host mask of the sampling requests (spec_verify_chain_hinted)"
    if ragged:
        cfg["lengths"] = "1 + b % 4"
        cfg["rows_per_call"] = rows
    if topp:
        cfg["top_p"] = TOPP
    if topk:
        cfg["top_k"] = TOPK
        if p_np is not None:
            cfg["top_p"] = args.top_p
    result = head(args, rows * args.steps / (total_ms * 1e-3), total_ms, cfg)
    result.update({
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                     "frac": achieved / PEAK_HBM_GBPS,
                     "traffic": stored_traffic(args.workload, dominant),
                     "kernel": dominant, "kernel_us": k_us, "algorithmic_bytes": rd_kernel},
        "kernels_us": {name: kt.mean_us(name) for name in kt.launches},
        "kernels_us_per_call": {name: 1e3 * kt.ms[name] / args.steps for name in kt.launches},
        "whole_call": {"us": call_us, "us_with_kernel_events": 1e3 * events_ms / args.steps,
                       "per_call_us": percentiles(calls), "host_enqueue_us": host_us,
                       "algorithmic_bytes": rd + sm,
                       "GBps": (rd + sm) / (call_us * 1e-6) / 1e9,
                       "frac": (rd + sm) / (call_us * 1e-6) / 1e9 / PEAK_HBM_GBPS},
    })
    if hinted:
        # the same calls without the hint, for comparison
        unhinted = [[sv.prepare_chain(t, d, tok, u_sets[j], T, out_t, out_n, ws) for j in range(n_u)]
                    for (t, d) in sets]

        def step_plain(i):
            unhinted[i % R][i % n_u]()
        for i in range(args.warmup):
            step_plain(i)
        plain_ms, _ = time_calls(torch, stream, step_plain, args.steps)
        with sv.KernelTimer(4 * args.steps) as kp:
            time_calls(torch, stream, step_plain, args.steps)
        result["without_hint"] = {"kernel_us": kp.mean_us(dominant), "whole_call_us": 1e3 * plain_ms / args.steps,
                                  "frac": rd / (kp.mean_us(dominant) * 1e-6) / 1e9 / PEAK_HBM_GBPS}
    if args.workload == "single":
        result["graph_replay"] = graph_replay(torch, stream, sv, sets[0], tok, u_sets[0], T, out_t, out_n, ws,
                                              args.steps)
    return result


def graph_replay(torch, stream, sv, tgt_drf, tok, u, T, out_t, out_n, ws, steps):
    """Latency of one call captured in a HIP graph and replayed: per replay
    device time (events between replays); the first replay's outputs are
    checked against an eager call."""
    t, d = tgt_drf
    sv.verify_chain(t, d, tok, u, T, out_tokens=out_t, out_num_accepted=out_n, ws=ws)
    torch.cuda.synchronize()
    eager = (out_t.clone(), out_n.clone())
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            sv.verify_chain(t, d, tok, u, T, out_tokens=out_t, out_num_accepted=out_n, ws=ws)
    torch.cuda.current_stream().wait_stream(s)
    g.replay()
    torch.cuda.synchronize()
    same = bool(torch.equal(eager[0], out_t) and torch.equal(eager[1], out_n))
    k = min(steps, 2000)
    times = per_call_us(torch, torch.cuda.current_stream(), lambda i: g.replay(), k)
    return {"per_call_us": percentiles(times), "replays": k, "matches_eager": same}


def run_tree(args, torch, synth, sv, oracle_sample=True):
    dev = torch.device("cuda:0")
    mss = args.workload == "tree-mss"
    temp = 0.0 if args.workload == "tree-greedy" else 1.0
    ti = synth.tree_inputs(temperature=temp, keep_draft=mss)
    mode = ("greedy" if temp == 0 else
            "multi-step speculative sampling, T=1, children drawn without replacement from each node's "
            "draft row" if mss else "naive sampling, T=1")
    desc = (f"token-tree verify ({mode}): B=32, N=64 nodes, depth <= 8, branching 1..4, V=128256, "
            f"bf16 logits")
    all_nodes = getattr(args, "tree_all_nodes", False) and not mss
    if all_nodes:
        desc += ("; the all-nodes statistics design (every node's row reduced up front, then the "
                 "descent; the SV_HOOK_TREE_ALL_NODES control)")
    set_bytes = ti.logits.nbytes * (2 if mss else 1)
    R = max(2, math.ceil(2 * MALL_BYTES / set_bytes) + 1)

    def dev_bf16(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)

    lg0 = dev_bf16(ti.logits)
    sets = [lg0] + [lg0.clone() for _ in range(R - 1)]
    if mss:
        dr0 = dev_bf16(ti.draft_logits)
        dsets = [dr0] + [dr0.clone() for _ in range(R - 1)]
        ud = torch.from_numpy(ti.draw_uniforms).to(dev)
    tok = torch.from_numpy(ti.node_tokens).to(dev)
    par = torch.from_numpy(ti.parents).to(dev)
    u = torch.from_numpy(ti.uniforms).to(dev)
    T = torch.from_numpy(ti.temperature).to(dev)
    query = sv.lib().sv_tree_mss_workspace_bytes if mss else sv.lib().sv_tree_workspace_bytes
    ws = sv.workspace(query(ti.B, ti.N, ti.V, sv.SV_BF16), dev)
    stream = torch.cuda.current_stream(dev)
    outs = {}

    def step(i):
        if mss:
            outs["r"] = sv.verify_tree_mss(sets[i % R], dsets[i % R], tok, par, u, ud, T, ti.max_depth, ws=ws)
        else:
            outs["r"] = sv.verify_tree(sets[i % R], tok, par, u, T, ti.max_depth, ws=ws)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    total_ms, host_us = time_calls(torch, stream, step, args.steps)
    with sv.KernelTimer(64 * args.steps) as kt:
        events_ms, _ = time_calls(torch, stream, step, args.steps)
    calls = per_call_us(torch, stream, step, min(args.steps, 2000))
    nacc = outs["r"][2].cpu().numpy()
    path = outs["r"][1].cpu().numpy()
    visited = int(np.sum(nacc + 1))  # the root and every accepted node are read
    es = 2
    rows = visited
    if mss:
        # a visited node with children also has its draft row read
        for b in range(ti.B):
            for n in [0] + [int(x) for x in path[b, :nacc[b]]]:
                rows += int(np.any(ti.parents[b] == n))
    rd = rows * ti.V * es
    if all_nodes:
        rd = ti.B * ti.N * ti.V * es   # every node's row, whatever the path
    call_us = 1e3 * total_ms / args.steps
    per_call = {name: kt.ms[name] * 1e3 / args.steps for name in kt.launches}
    dominant = max(per_call, key=per_call.get)  # tree_verify; tree_node_pass in the multi-launch form
    dom_us = per_call[dominant]
    achieved = rd / (dom_us * 1e-6) / 1e9 if dom_us > 0 else 0.0
    result = head(args, ti.B * ti.N * args.steps / (total_ms * 1e-3), total_ms,
                  {"workload": desc, "B": ti.B, "N": ti.N, "V": ti.V, "max_depth": ti.max_depth,
                   "rotating_input_sets": R, "visited_nodes_per_call": visited})
    result.update({
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                     "frac": achieved / PEAK_HBM_GBPS, "traffic": None, "kernel": dominant,
                     "kernel_us_per_call": dom_us, "algorithmic_bytes": rd,
                     "note": "bytes of the visited nodes' rows (and, for MSS, the draft rows of "
                             "visited nodes that have children) per call over the summed duration of "
                             f"that call's {dominant} launches; the descent is a chain of dependent "
                             "levels (and, for MSS, of residual passes), so the time is latency, not "
                             "bytes"},
        "kernels_us_per_call": per_call,
        "launches_per_call": {name: kt.launches[name] / args.steps for name in kt.launches},
        "whole_call": {"us": call_us, "us_with_kernel_events": 1e3 * events_ms / args.steps,
                       "per_call_us": percentiles(calls), "host_enqueue_us": host_us,
                       "algorithmic_bytes": rd, "GBps": rd / (call_us * 1e-6) / 1e9,
                       "frac": rd / (call_us * 1e-6) / 1e9 / PEAK_HBM_GBPS},
    })
    result["config"]["rows_read_per_call"] = rows
    return result


def mask_bytes(B, N) -> int:
    """Parents read; row words, depths and tree depths written."""
    return B * N * 4 + B * N * ((N + 63) // 64) * 8 + B * N * 4 + B * 4


def run_mask(args, torch, synth, sv):
    """spec_tree_mask on the token-tree workload's shape (B=32, N=64, depth
    <= 8), plus the same timing at B=4096, N=256 to show the store-bound
    regime.  Rows are mask rows (one per node)."""
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)

    def measure(B, N, max_depth, steps):
        par = torch.from_numpy(synth.tree_parent_arrays(15005, B, N, max_depth, 4)).to(dev)
        m = torch.empty((B, N, (N + 63) // 64), dtype=torch.int64, device=dev)
        d = torch.empty((B, N), dtype=torch.int32, device=dev)
        t = torch.empty((B,), dtype=torch.int32, device=dev)

        def step(i):
            sv.tree_mask(par, max_depth, m, d, t)

        for i in range(args.warmup):
            step(i)
        torch.cuda.synchronize()
        total_ms, host_us = time_calls(torch, stream, step, steps)
        with sv.KernelTimer(4 * steps) as kt:
            time_calls(torch, stream, step, steps)
        k_us = kt.mean_us("tree_mask")
        nb = mask_bytes(B, N)
        return {"B": B, "N": N, "max_depth": max_depth, "call_us": 1e3 * total_ms / steps,
                "kernel_us": k_us, "host_enqueue_us": host_us, "algorithmic_bytes": nb,
                "GBps": nb / (k_us * 1e-6) / 1e9, "rows_per_s": B * N / (total_ms * 1e-3 / steps),
                "total_ms": total_ms}

    small = measure(32, 64, 8, args.steps)
    large = measure(4096, 256, 16, max(20, args.steps // 10))
    result = head(args, small["rows_per_s"], small["total_ms"],
                  {"workload": "tree attention mask and depth positions: B=32 trees of N=64 nodes, "
                               "depth <= 8, branching 1..4 (the token-tree verify shape)",
                   "B": 32, "N": 64, "max_depth": 8},
                  metric="tree mask rows/sec (one row per node) and achieved HBM GB/s vs peak, 1 GPU")
    result["dtype"] = "int32/uint64"
    result.update({
        "roofline": {"bound": "hbm", "achieved": small["GBps"], "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                     "frac": small["GBps"] / PEAK_HBM_GBPS, "traffic": None, "kernel": "tree_mask",
                     "kernel_us_per_call": small["kernel_us"],
                     "algorithmic_bytes": small["algorithmic_bytes"],
                     "note": "32.9 KB per call: the launch and the walk's dependent LDS reads set the "
                             "time, not bytes; large_shape shows the store-bound regime"},
        "large_shape": {k: v for k, v in large.items() if k != "total_ms"},
    })
    return result


# ---------------------------------------------------------------------------
# the oracle timed on the host (a child process started before the GPU is
# touched; its pool forks from that child)
# ---------------------------------------------------------------------------
BOX_CPU_SHARE = 16          # host cores granted to a job that holds one GPU
SINGLE_BUDGET_S = 10.0
POOL_BUDGET_S = 6.0
_BASELINE = {}


def host_cpu() -> dict:
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    if model is None:
        try:
            out = subprocess.run(["lscpu"], capture_output=True, text=True, timeout=20).stdout
            for line in out.splitlines():
                if line.startswith("Model name"):
                    model = line.split(":", 1)[1].strip()
        except (OSError, subprocess.SubprocessError):
            pass
    return {"cpu_model": model, "logical_cpus": os.cpu_count(),
            "cpus_in_affinity": len(os.sched_getaffinity(0))}


def oracle_units(workload, top_p):
    """The oracle's work on one workload's batch as (units, fn, what): fn(b, s)
    verifies unit b (a request, a tree, or the whole mask batch) in pass s and
    returns the rows that covers.  Chain passes after the first draw fresh
    uniforms, as the GPU calls do."""
    import oracle
    import synth

    if workload == "tree-mask":
        parents = synth.tree_parent_arrays(15005, 32, 64, 8, 4)

        def fn(b, s):
            oracle.tree_attention_mask(parents, 8)
            return parents.size
        return 1, fn, "masks of the B=32, N=64 batch (python loops)"
    if workload.startswith("tree"):
        mss = workload == "tree-mss"
        ti = synth.tree_inputs(temperature=0.0 if workload == "tree-greedy" else 1.0, keep_draft=mss)

        def fn(b, s):
            sl = slice(b, b + 1)
            if mss:
                oracle.verify_tree_mss(ti.logits[sl], ti.draft_logits[sl], ti.node_tokens[sl], ti.parents[sl],
                                       ti.uniforms[sl], ti.draw_uniforms[sl], ti.temperature[sl], ti.dtype,
                                       ti.max_depth)
            else:
                oracle.verify_tree(ti.logits[sl], ti.node_tokens[sl], ti.parents[sl], ti.uniforms[sl],
                                   ti.temperature[sl], ti.dtype, ti.max_depth)
            return ti.N
        return ti.B, fn, "tree verifications of the batch, numpy fp64"
    ci, _ = chain_case(workload, synth)
    gam = (np.array([RAGGED_LENGTHS[b % len(RAGGED_LENGTHS)] for b in range(ci.B)], np.int32)
           if workload == "ragged" else None)
    k_np = np.full(ci.B, TOPK, np.int32) if workload == "topk" else None
    pp_np = np.full(ci.B, TOPP, np.float32) if workload == "topp" else None
    p_np = np.full(ci.B, top_p, np.float32) if (k_np is not None and top_p is not None) else None
    u_pass = {}

    def fn(b, s):
        if s not in u_pass:
            u_pass.clear()
            u_pass[s] = ci.uniforms if s == 0 else ci.fresh_uniforms(90_000 + s)
        u, sl = u_pass[s], slice(b, b + 1)
        if pp_np is not None:
            oracle.verify_chain_filtered(ci.target[sl], ci.draft[sl], ci.draft_tokens[sl], u[sl], ci.temperature[sl],
                                         ci.dtype, top_p=pp_np[sl])
        elif k_np is not None:
            oracle.verify_chain_topk(ci.target[sl], ci.draft[sl], ci.draft_tokens[sl], u[sl], ci.temperature[sl],
                                     k_np[sl], ci.dtype, top_p=None if p_np is None else p_np[sl])
        elif gam is None:
            oracle.verify_chain(ci.target[sl], ci.draft[sl], ci.draft_tokens[sl], u[sl], ci.temperature[sl],
                                ci.dtype)
        else:
            oracle.verify_chain_ragged(ci.target[sl], ci.draft[sl], ci.draft_tokens[sl], u[sl],
                                       ci.temperature[sl], gam[sl], ci.dtype)
            return int(gam[b]) + 1
        return ci.gamma + 1
    return ci.B, fn, "request verifications of the batch with fresh uniforms per pass, numpy fp64"


def _oracle_loop(job):
    """Worker w of W walks the whole batch in order, starting at unit
    w * units / W, with pass numbers of its own, until its budget is spent:
    every worker sees the batch's mix of requests, as one process does."""
    w, W, budget_s = job
    units, fn = _BASELINE["units"], _BASELINE["fn"]
    rows = n = 0
    j = 0
    w0, c0 = time.perf_counter(), time.process_time()
    while time.perf_counter() - w0 < budget_s:
        rows += fn((j + (w * units) // W) % units, (j // units) * W + w)
        n += 1
        j += 1
    return rows, n, time.perf_counter() - w0, time.process_time() - c0


def cpu_baseline_only(workload, top_p) -> dict:
    """Single process, then a pool of min(16, CPUs in this process's affinity)
    forked workers over the same batch; `value` is the pool's rate."""
    import multiprocessing as mp

    units, fn, what = oracle_units(workload, top_p)
    _BASELINE.update(units=units, fn=fn)
    rows1, n1, wall1, cpu1 = _oracle_loop((0, 1, SINGLE_BUDGET_S))
    W = max(1, min(BOX_CPU_SHARE, len(os.sched_getaffinity(0))))
    t0 = time.perf_counter()
    with mp.get_context("fork").Pool(W) as pool:
        parts = pool.map(_oracle_loop, [(w, W, POOL_BUDGET_S) for w in range(W)])
    wall = time.perf_counter() - t0
    rows, n, cpu = sum(p[0] for p in parts), sum(p[1] for p in parts), sum(p[3] for p in parts)
    return {"value": rows / wall, "unit": "rows/s", "cores": W, "kind": "oracle",
            "sample": f"{n} {what}, {W} single-threaded worker processes for {wall:.1f} s wall "
                      f"({rows} rows, {cpu:.1f} s CPU)",
            "single_process": {"value": rows1 / wall1, "unit": "rows/s", "cores": 1,
                               "sample": f"{n1} units, {rows1} rows in {wall1:.1f} s wall, {cpu1:.1f} s CPU"},
            "host": host_cpu()}


def cpu_baseline_child(workload, top_p):
    """Runs the oracle timing in a child process with one thread per process,
    before this process touches the GPU."""
    cmd = [sys.executable, os.path.abspath(__file__), "--workload", workload, "--cpu-baseline-only"]
    if top_p is not None:
        cmd += ["--top-p", repr(top_p)]
    env = dict(os.environ, OMP_NUM_THREADS="1", OPENBLAS_NUM_THREADS="1", MKL_NUM_THREADS="1")
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=600, env=env, cwd=ROOT)
    lines = [x for x in r.stdout.splitlines() if x.startswith("{")]
    if r.returncode != 0 or not lines:
        raise RuntimeError(f"oracle timing failed (exit {r.returncode}): {r.stderr[-2000:]}")
    return json.loads(lines[-1])


def head(args, value, total_ms, config, metric=METRIC):
    return {
        "metric": metric,
        "value": value,
        "unit": "rows/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": total_ms / args.steps,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": config,
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None,
                    help="timed calls (default 200; 10000 for the single-request workload)")
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", choices=WORKLOADS, default="batched",
                    help="batched is the headline; the others are reported alongside it")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-hint", action="store_true",
                    help="batched: call spec_verify_chain without the sampling hint")
    ap.add_argument("--cpu-baseline-only", action="store_true",
                    help="time the oracle on the host only and print its JSON (no GPU use)")
    ap.add_argument("--tree-all-nodes", action="store_true",
                    help="tree-greedy / tree-sampling: time the all-nodes statistics design instead of "
                         "path descent")
    ap.add_argument("--top-p", type=float, default=None,
                    help="topk workload: also filter to this top-p mass after top-k (draft tokens stay top-k draws)")
    args = ap.parse_args()
    if args.steps is None:
        args.steps = 10000 if args.workload == "single" else 200
    if args.gpus != 1:
        print("bench.py measures one GPU only: requests shard across GPUs with no exchange, so a "
              "multi-GPU figure is N independent copies of this one", file=sys.stderr)
        sys.exit(2)
    if args.cpu_baseline_only:
        print(json.dumps(cpu_baseline_only(args.workload, args.top_p)), flush=True)
        return
    baseline = None if args.no_cpu_baseline else cpu_baseline_child(args.workload, args.top_p)

    import torch
    import synth
    import rejection_sampling_verify_15_amd as sv
    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)
    if args.workload == "tree-mask":
        result = run_mask(args, torch, synth, sv)
    elif args.workload.startswith("tree"):
        if args.tree_all_nodes and args.workload in ("tree-greedy", "tree-sampling"):
            with sv.library_control(sv.SV_HOOK_TREE_ALL_NODES, 1):
                result = run_tree(args, torch, synth, sv)
        else:
            result = run_tree(args, torch, synth, sv)
    else:
        result = run_chain(args, torch, synth, sv)
    if baseline is not None:
        result["cpu_baseline"] = baseline
    print(json.dumps(result), flush=True)
    # leave no device memory for torch's allocator to free during exit()
    del result
    sv.binding.release_workspaces()


if __name__ == "__main__":
    main()
