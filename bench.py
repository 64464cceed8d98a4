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


def algorithmic_bytes(ci) -> int:
    """Every needed logit read once (sampling request: 2*gamma+1 rows, greedy
    request: gamma+1 rows) plus tokens, uniforms, temperature and outputs."""
    es = 2 if ci.dtype == "bf16" else 4
    total = 0
    for b in range(ci.B):
        rows = (2 * ci.gamma + 1) if float(ci.temperature[b]) > 0 else (ci.gamma + 1)
        total += rows * ci.V * es
    total += ci.B * (4 * ci.gamma + 4 * (ci.gamma + 1) + 4 + 4 * (ci.gamma + 1) + 4)
    return total


def cpu_baseline(ci, budget_s: float = 15.0):
    """The fp64 oracle as it stands on a bounded sample of the same batch."""
    import oracle
    done_rows = 0
    t0 = time.perf_counter()
    b = 0
    while time.perf_counter() - t0 < budget_s and b < ci.B:
        oracle.verify_chain(ci.target[b:b + 1], ci.draft[b:b + 1], ci.draft_tokens[b:b + 1],
                            ci.uniforms[b:b + 1], ci.temperature[b:b + 1], ci.dtype)
        done_rows += ci.gamma + 1
        b += 1
    dt = time.perf_counter() - t0
    return {"value": done_rows / dt, "unit": "rows/s", "cores": 1, "kind": "oracle",
            "sample": f"first {b} of {ci.B} requests of one batch, one process, numpy fp64, "
                      f"{dt:.1f} s"}


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

    def step(i):
        t, d = sets[i % R]
        sv.verify_chain(t, d, tok, u, T, out_tokens=out_t, out_num_accepted=out_n, ws=ws)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(args.steps)]
    start_all = torch.cuda.Event(enable_timing=True)
    end_all = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start_all.record(stream)
    for i in range(args.steps):
        ev[i][0].record(stream)
        step(i)
        ev[i][1].record(stream)
    end_all.record(stream)
    torch.cuda.synchronize()
    total_ms = start_all.elapsed_time(end_all)
    per_call = np.array([a.elapsed_time(b) for a, b in ev])
    ms_per_step = total_ms / args.steps
    rows = ci.B * (ci.gamma + 1)
    alg = algorithmic_bytes(ci)
    call_ms = float(per_call.mean())
    achieved = alg / (call_ms * 1e-3) / 1e9

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
        "config": {"workload": "batched chain verify: B=64, gamma=4, V=128256, bf16, "
                               "even requests T=0.7 sampling, odd greedy",
                   "B": ci.B, "gamma": ci.gamma, "V": ci.V, "rotating_input_sets": R,
                   "algorithmic_bytes_per_call": alg},
        "achieved_GBps": achieved,
        "call_us": {"mean": call_ms * 1e3, "p10": float(np.percentile(per_call, 10)) * 1e3,
                    "p50": float(np.percentile(per_call, 50)) * 1e3,
                    "p90": float(np.percentile(per_call, 90)) * 1e3},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                     "frac": achieved / PEAK_HBM_GBPS, "traffic": None,
                     "kernel": "whole spec_verify_chain call (all its kernels), HIP events"},
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(ci)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
