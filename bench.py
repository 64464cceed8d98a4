"""Benchmark of the chain verification step on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W]

Workload: the batched chain verification, B=64 requests, gamma=4, V=128256,
bf16 logits; even requests sample at T=0.7, odd requests are greedy (draft
noise sigma ~ U[0.3, 2.0]).  A step is one spec_verify_chain call over one
batch.  Inputs sit in HBM before timing starts; calls rotate over R copies of
the batch (more than 512 MB together) so each call reads cold data rather
than the 256 MB Infinity Cache.

Prints one JSON line: verified (request x position) rows per second, the
achieved algorithmic HBM bandwidth against the 8 TB/s peak, and the fp64
oracle timed on this host's cores on a bounded sample.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "verified (request×position) rows/sec and achieved HBM GB/s vs peak, 1 GPU"
PEAK_HBM_GBPS = 8000.0
MALL_BYTES = 256 << 20


def read_bytes(ci) -> int:
    """Logit bytes the path must read once: 2*gamma+1 rows of a sampling
    request (gamma+1 target, gamma draft), gamma+1 target rows of a greedy one."""
    es = 2 if ci.dtype == "bf16" else 4
    rows = sum((2 * ci.gamma + 1) if float(ci.temperature[b]) > 0 else (ci.gamma + 1)
               for b in range(ci.B))
    return rows * ci.V * es


def small_bytes(ci) -> int:
    """Tokens, uniforms, temperature read and emitted tokens / counts written."""
    return ci.B * (4 * ci.gamma + 4 * (ci.gamma + 1) + 4 + 4 * (ci.gamma + 1) + 4)


def source_digest() -> str:
    """Hash of the chain kernel sources; a stored traffic figure is valid only
    for the sources it was measured on."""
    h = hashlib.sha256()
    for rel in ("rejection_sampling_verify_15_amd/csrc/sv_chain.hip",
                "rejection_sampling_verify_15_amd/csrc/sv_device.hpp"):
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def stored_traffic(kernel: str):
    """HBM bytes per launch of `kernel` from the committed rocprofv3 counter
    summary, or None when it is missing or the kernel changed since."""
    path = os.path.join(ROOT, "profiles", "traffic_batched_chain.json")
    try:
        with open(path) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    k = rec.get("kernels", {}).get(kernel)
    if k is None or rec.get("source_sha256") != source_digest():
        return None
    return k.get("traffic_bytes_per_launch")


def cpu_baseline(ci, budget_s: float = 15.0):
    """The fp64 oracle as it stands, timed on this host's cores: it verifies
    the same batch over and over with fresh uniforms until the budget is
    spent.  `cores` is the CPU time it used divided by the wall time."""
    import oracle
    rows = 0
    passes = 0
    requests = 0
    w0 = time.perf_counter()
    c0 = time.process_time()
    while time.perf_counter() - w0 < budget_s:
        u = ci.uniforms if passes == 0 else ci.fresh_uniforms(90_000 + passes)
        for b in range(ci.B):
            oracle.verify_chain(ci.target[b:b + 1], ci.draft[b:b + 1], ci.draft_tokens[b:b + 1],
                                u[b:b + 1], ci.temperature[b:b + 1], ci.dtype)
            rows += ci.gamma + 1
            requests += 1
            if time.perf_counter() - w0 >= budget_s:
                break
        passes += 1
    wall = time.perf_counter() - w0
    cpu = time.process_time() - c0
    return {"value": rows / wall, "unit": "rows/s", "cores": max(1, round(cpu / wall)),
            "kind": "oracle",
            "sample": f"{requests} request verifications ({rows} rows) of the same batch with "
                      f"fresh uniforms, numpy fp64, {wall:.1f} s wall, {cpu:.1f} s CPU"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU only: requests shard across GPUs with no exchange, so a "
              "multi-GPU figure is N independent copies of this one", file=sys.stderr)
        sys.exit(2)

    import torch
    import synth
    import rejection_sampling_verify_15_amd as sv
    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    ci = synth.batched_chain()
    set_bytes = ci.target.nbytes + ci.draft.nbytes
    R = max(2, math.ceil(2 * MALL_BYTES / set_bytes) + 1)

    def dl(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)
    tgt0, drf0 = dl(ci.target), dl(ci.draft)
    sets = [(tgt0, drf0)] + [(tgt0.clone(), drf0.clone()) for _ in range(R - 1)]
    tok = torch.from_numpy(ci.draft_tokens.astype(np.int32)).to(dev)
    u = torch.from_numpy(ci.uniforms).to(dev)
    T = torch.from_numpy(ci.temperature).to(dev)
    out_t = torch.empty((ci.B, ci.gamma + 1), dtype=torch.int32, device=dev)
    out_n = torch.empty((ci.B,), dtype=torch.int32, device=dev)
    ws = sv.workspace(sv.lib().sv_chain_workspace_bytes(ci.B, ci.gamma, ci.V, sv.SV_BF16), dev)
    stream = torch.cuda.current_stream(dev)

    def step(i):
        t, d = sets[i % R]
        sv.verify_chain(t, d, tok, u, T, out_tokens=out_t, out_num_accepted=out_n, ws=ws)

    def timed(k):
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a.record(stream)
        for i in range(k):
            step(i)
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    # the timed region
    total_ms = timed(args.steps)
    # the same steps again with a pair of events attached to every kernel
    # dispatch: per-kernel durations (the attached events themselves add a few
    # microseconds between launches, so the whole-call figure comes from the
    # region above)
    with sv.KernelTimer(4 * args.steps) as kt:
        events_ms = timed(args.steps)

    ms_per_step = total_ms / args.steps
    rows = ci.B * (ci.gamma + 1)
    rd, sm = read_bytes(ci), small_bytes(ci)
    call_us = 1e3 * ms_per_step
    dominant = "chain_verify"
    k_us = kt.mean_us(dominant)
    achieved = rd / (k_us * 1e-6) / 1e9
    traffic = stored_traffic(dominant)

    result = {
        "metric": METRIC,
        "value": rows * args.steps / (total_ms * 1e-3),
        "unit": "rows/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "batched chain verify: B=64, gamma=4, V=128256, bf16 logits, "
                               "even requests sample at T=0.7, odd requests greedy",
                   "B": ci.B, "gamma": ci.gamma, "V": ci.V, "rotating_input_sets": R},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                     "frac": achieved / PEAK_HBM_GBPS, "traffic": traffic,
                     "kernel": dominant, "kernel_us": k_us, "algorithmic_bytes": rd},
        "kernels_us": {name: kt.mean_us(name) for name in kt.launches},
        "whole_call": {"us": call_us, "us_with_kernel_events": 1e3 * events_ms / args.steps,
                       "algorithmic_bytes": rd + sm,
                       "GBps": (rd + sm) / (call_us * 1e-6) / 1e9,
                       "frac": (rd + sm) / (call_us * 1e-6) / 1e9 / PEAK_HBM_GBPS},
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(ci)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
