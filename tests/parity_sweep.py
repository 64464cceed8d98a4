"""Large parity sweeps of the chain and tree verification paths against the
fp64 oracle: at least 1e5 decisions per workload, over several freshly
seeded logit sets and many uniform sets each.

Two phases, so that the oracle's CPU work does not hold a GPU:

  python tests/parity_sweep.py gpu --out DIR [--only NAME ...]
      runs the library on every (logit seed, uniform set) pair of each
      workload and stores the outputs with a fingerprint of the inputs;
  python tests/parity_sweep.py compare --dir DIR [--workers N]
      regenerates the same seeded inputs, checks the fingerprints, runs the
      oracle in a process pool split by request, and prints one JSON tally
      per workload (decisions, sampled decisions, in-window, boundary
      mismatches, hard failures).

The pass bar is the one of every parity test: no disagreement outside the
1e-5 window, and in-window disagreements below 0.01% of all decisions.
Uniform set 0 of each logit seed is the workload's own uniform array; set s
> 0 is drawn from default_rng(seed * 100003 + s) (second array for MSS from
the same stream).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import multiprocessing as mp
import os
import sys
import time

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
for p in (ROOT, HERE):
    if p not in sys.path:
        sys.path.insert(0, p)

import synth  # noqa: E402

# workload name -> (kind, input builder by seed, logit seeds, uniform sets per seed)
WORKLOADS = {
    "batched_B64_g4_V128256": (
        "chain", lambda s: synth.batched_chain(seed=s), [synth.SEED_BASE + 3, 21101, 21102, 21103], 300),
    "deep_B256_g8_V151936": (
        "chain", lambda s: synth.deep_chain(seed=s), [synth.SEED_BASE + 4, 21201], 60),
    "tree_naive_B32_N64_V128256": (
        "tree", lambda s: synth.tree_inputs(seed=s, temperature=1.0),
        [synth.SEED_BASE + 5, 21301, 21302], 1100),
    "tree_mss_B32_N64_V128256": (
        "mss", lambda s: synth.tree_inputs(seed=s, temperature=1.0, keep_draft=True),
        [synth.SEED_BASE + 5, 21401, 21402], 250),
    "topp09_B64_g4_V128256": (
        "filtered", lambda s: topp_batched(s), [synth.SEED_BASE + 3, 21501, 21502, 21503], 200),
    "filtered_mixed_B64_g4_V128256": (
        "filtered", lambda s: mixed_filters(s), [21601, 21602, 21603, 21604], 200),
    "filtered_mixed_f32_B64_g4_V128256": (
        "filtered", lambda s: mixed_filters(s, dtype="f32"), [21701, 21702, 21703, 21704], 200),
    "filtered_small_T_B64_g4_V128256": (
        "filtered", lambda s: mixed_filters(s, small_t=True), [21801, 21802, 21803, 21804], 200),
    "ragged_B64_g1to4_V128256": (
        "ragged", lambda s: ragged_batched(s), [synth.SEED_BASE + 3, 21901, 21902, 21903], 210),
    "topk_mixed_B64_g4_V128256": (
        "topk", lambda s: topk_mixed(s), [22001, 22002, 22003, 22004], 200),
}


class Filtered:
    """Chain inputs plus the per-request filter arrays of a filtered call."""

    def __init__(self, ci, top_k, top_p):
        self.ci, self.top_k, self.top_p = ci, top_k, top_p

    def __getattr__(self, name):
        return getattr(self.ci, name)


def topp_batched(seed):
    """The batched inputs, every sampling request cut to its top-p 0.9 mass,
    draft tokens from the cut draft rows."""
    ci = synth.batched_chain(seed=seed)
    p = np.full(ci.B, 0.9, np.float32)
    ci.draft_tokens = synth.topp_draft_tokens(ci, p, seed + 7)
    return Filtered(ci, None, p)


def mixed_filters(seed, dtype="bf16", small_t=False):
    """The batched shape (bf16, or fp32 logits of the same recipe) with a
    filter per request: top-k 50 or 1024 or none, then top-p 0.8 or 0.9 or
    none; draft tokens drawn from the draft rows cut alike (by the oracle's
    filter, as a draft model decoding with it would).  small_t: the sampling
    requests' temperatures drawn log-uniformly from [0.005, 0.1]."""
    from test_gpu_chain_filtered import filtered_draft_tokens
    if dtype == "bf16":
        ci = synth.batched_chain(seed=seed)
    else:
        ci = synth.chain_inputs(seed, 64, 4, 128256, dtype=dtype, family="peaked", draft_sigma=(0.3, 2.0),
                                temperature=0.7, greedy_odd=True, name="batched-f32")
    rng = np.random.default_rng(seed + 11)
    if small_t:
        t = np.exp(rng.uniform(np.log(0.005), np.log(0.1), size=ci.B)).astype(np.float32)
        ci.temperature = np.where(ci.temperature > 0, t, 0.0).astype(np.float32)
    k = rng.choice(np.array([50, 1024, ci.V], np.int32), size=ci.B)
    p = rng.choice(np.array([0.8, 0.9, 1.0], np.float32), size=ci.B)
    ci.draft_tokens = filtered_draft_tokens(ci, k, p, seed + 13)
    return Filtered(ci, k, p)


class Ragged:
    """Chain inputs plus a draft length per request."""

    def __init__(self, ci, gammas):
        self.ci, self.gammas = ci, gammas

    def __getattr__(self, name):
        return getattr(self.ci, name)


def ragged_batched(seed):
    """The batched inputs with request b drafting 1 + b % 4 tokens (the
    padded arrays of gamma 4)."""
    ci = synth.batched_chain(seed=seed)
    return Ragged(ci, (1 + np.arange(ci.B) % 4).astype(np.int32))


def topk_mixed(seed):
    """The batched inputs under the limited top-k entry point: k per request
    from {1, 5, 50, 128}, then top-p 0.8, 0.9 or none; draft tokens drawn
    from the draft rows cut alike."""
    from test_gpu_chain_topk import filtered_draft_tokens
    ci = synth.batched_chain(seed=seed)
    rng = np.random.default_rng(seed + 17)
    k = rng.choice(np.array([1, 5, 50, 128], np.int32), size=ci.B)
    p = rng.choice(np.array([0.8, 0.9, 1.0], np.float32), size=ci.B)
    ci.draft_tokens = filtered_draft_tokens(ci, k, seed + 19, top_p=p)
    return Filtered(ci, k, p)


def fingerprint(*arrays) -> str:
    h = hashlib.sha256()
    for a in arrays:
        if a is None:
            h.update(b"none")
            continue
        a = np.ascontiguousarray(a)
        h.update(str((a.dtype.str, a.shape)).encode())
        h.update(a.view(np.uint8).reshape(-1).data)
    return h.hexdigest()


def inputs_fingerprint(kind, x) -> str:
    if kind == "chain":
        return fingerprint(x.target, x.draft, x.draft_tokens, x.temperature, x.uniforms)
    if kind in ("filtered", "topk"):
        return fingerprint(x.target, x.draft, x.draft_tokens, x.temperature, x.uniforms, x.top_k, x.top_p)
    if kind == "ragged":
        return fingerprint(x.target, x.draft, x.draft_tokens, x.temperature, x.uniforms, x.gammas)
    return fingerprint(x.logits, x.draft_logits, x.node_tokens, x.parents, x.temperature,
                       x.uniforms, x.draw_uniforms)


def uniform_sets(kind, x, seed, n_sets):
    """[(u,)] for chain and naive trees, [(u_accept, u_draw)] for MSS."""
    shape = (x.B, x.gamma + 1) if kind in ("chain", "filtered", "ragged", "topk") else (x.B, x.N)
    first = (x.uniforms,) if kind != "mss" else (x.uniforms, x.draw_uniforms)
    out = [first]
    for s in range(1, n_sets):
        rng = np.random.default_rng(seed * 100003 + s)
        if kind == "mss":
            out.append((synth.uniforms(rng, shape), synth.uniforms(rng, shape)))
        else:
            out.append((synth.uniforms(rng, shape),))
    return out


# ---------------------------------------------------------------------------
# GPU phase (library only)
# ---------------------------------------------------------------------------
def gpu_phase(out_dir, only, sets=None):
    import torch
    import rejection_sampling_verify_15_amd as sv
    from parity import to_device, to_device_logits

    os.makedirs(out_dir, exist_ok=True)
    for name, (kind, build, seeds, n_sets) in WORKLOADS.items():
        if only and name not in only:
            continue
        n_sets = sets or n_sets
        for seed in seeds:
            t0 = time.time()
            x = build(seed)
            fp = inputs_fingerprint(kind, x)
            print(f"[gpu] {name} seed={seed} built in {time.time() - t0:.1f}s", flush=True)
            us = uniform_sets(kind, x, seed, n_sets)
            toks, paths, ns = [], [], []
            if kind in ("chain", "filtered", "ragged", "topk"):
                tgt = to_device_logits(x.target, x.dtype)
                drf = to_device_logits(x.draft, x.dtype)
                dt = to_device(x.draft_tokens.astype(np.int32))
                T = to_device(x.temperature.astype(np.float32))
                if kind in ("filtered", "topk"):
                    kd = None if x.top_k is None else to_device(np.asarray(x.top_k, np.int32))
                    pd = None if x.top_p is None else to_device(np.asarray(x.top_p, np.float32))
                if kind == "ragged":
                    gd = to_device(np.asarray(x.gammas, np.int32))
                for (u,) in us:
                    if kind == "filtered":
                        ot, on = sv.verify_chain_filtered(tgt, drf, dt, to_device(u), T, kd, pd)
                    elif kind == "topk":
                        ot, on = sv.verify_chain_topk(tgt, drf, dt, to_device(u), T, kd, top_p=pd)
                    elif kind == "ragged":
                        ot, on, _ = sv.verify_chain_ragged(tgt, drf, dt, to_device(u), T, gd)
                    else:
                        ot, on = sv.verify_chain(tgt, drf, dt, to_device(u), T)
                    toks.append(ot.cpu().numpy())
                    ns.append(on.cpu().numpy())
            else:
                lg = to_device_logits(x.logits, x.dtype)
                tok = to_device(x.node_tokens.astype(np.int32))
                par = to_device(x.parents.astype(np.int32))
                T = to_device(x.temperature.astype(np.float32))
                dl = to_device_logits(x.draft_logits, x.dtype) if kind == "mss" else None
                for u in us:
                    if kind == "mss":
                        ot, op, on = sv.verify_tree_mss(lg, dl, tok, par, to_device(u[0]), to_device(u[1]),
                                                        T, x.max_depth)
                    else:
                        ot, op, on = sv.verify_tree(lg, tok, par, to_device(u[0]), T, x.max_depth)
                    toks.append(ot.cpu().numpy())
                    paths.append(op.cpu().numpy())
                    ns.append(on.cpu().numpy())
            torch.cuda.synchronize()
            arrays = dict(tokens=np.stack(toks), n=np.stack(ns))
            if paths:
                arrays["paths"] = np.stack(paths)
            np.savez_compressed(os.path.join(out_dir, f"{name}__{seed}.npz"), fingerprint=np.array(fp),
                                n_sets=np.array(n_sets), **arrays)
            print(f"[gpu] {name} seed={seed} {n_sets} calls done in {time.time() - t0:.1f}s", flush=True)
            del x
    sv.binding.release_workspaces()


# ---------------------------------------------------------------------------
# compare phase (oracle, CPU)
# ---------------------------------------------------------------------------
_STATE = {}


def _compare_part(requests):
    """Oracle results and tally for a subset of requests over every uniform set
    (runs in a forked worker that inherited _STATE)."""
    import oracle
    from parity import (Tally, compare_chain, compare_filtered, compare_tree, compare_tree_mss, oracle_chain_many,
                        oracle_filtered_many)

    kind, x, us, gpu = _STATE["kind"], _STATE["x"], _STATE["us"], _STATE["gpu"]
    tally = Tally()
    if kind == "ragged":
        for s, u in enumerate(us):
            r = oracle.verify_chain_ragged(x.target, x.draft, x.draft_tokens, u[0], x.temperature, x.gammas,
                                           x.dtype, requests=requests)
            tally.add(compare_chain(r, gpu["tokens"][s], gpu["n"][s], requests=requests))
        return tally
    if kind == "topk":
        for s, u in enumerate(us):
            r = oracle.verify_chain_topk(x.target, x.draft, x.draft_tokens, u[0], x.temperature, x.top_k,
                                         x.dtype, requests=requests, top_p=x.top_p)
            tally.add(compare_chain(r, gpu["tokens"][s], gpu["n"][s], requests=requests))
        return tally
    if kind == "filtered":
        refs = oracle_filtered_many(x.ci, [u[0] for u in us], x.top_k, x.top_p, requests=requests)
        for s, r in enumerate(refs):
            tally.add(compare_filtered(r, gpu["tokens"][s], gpu["n"][s], requests=requests))
        return tally
    if kind == "chain":
        refs = oracle_chain_many(x, [u[0] for u in us], requests=requests)
        for s, r in enumerate(refs):
            tally.add(compare_chain(r, gpu["tokens"][s], gpu["n"][s], requests=requests))
        return tally
    cache = {}
    for s, u in enumerate(us):
        if kind == "mss":
            r = oracle.verify_tree_mss(x.logits, x.draft_logits, x.node_tokens, x.parents, u[0], u[1],
                                       x.temperature, x.dtype, x.max_depth, requests=requests,
                                       dist_cache=cache)
            tally.add(compare_tree_mss(r, gpu["tokens"][s], gpu["paths"][s], gpu["n"][s], requests=requests))
        else:
            r = oracle.verify_tree(x.logits, x.node_tokens, x.parents, u[0], x.temperature, x.dtype,
                                   x.max_depth, requests=requests, dist_cache=cache)
            tally.add(compare_tree(r, gpu["tokens"][s], gpu["paths"][s], gpu["n"][s], requests=requests))
    return tally


def compare_phase(in_dir, workers, only):
    from parity import MAX_MISMATCH_RATE, Tally

    ok = True
    for name, (kind, build, seeds, n_sets) in WORKLOADS.items():
        if only and name not in only:
            continue
        total = Tally()
        t0 = time.time()
        used_sets = []
        for seed in seeds:
            path = os.path.join(in_dir, f"{name}__{seed}.npz")
            with np.load(path, allow_pickle=False) as z:
                gpu = {k: z[k] for k in z.files}
            x = build(seed)
            if str(gpu["fingerprint"]) != inputs_fingerprint(kind, x):
                raise SystemExit(f"{name} seed={seed}: inputs differ from the ones the GPU phase used")
            used_sets.append(int(gpu["n_sets"]))
            us = uniform_sets(kind, x, seed, used_sets[-1])
            _STATE.update(kind=kind, x=x, us=us, gpu=gpu)
            parts = [list(range(x.B))[i::workers] for i in range(workers)]
            with mp.get_context("fork").Pool(workers) as pool:
                for t in pool.imap_unordered(_compare_part, parts):
                    total.add(t)
            _STATE.clear()
            del x
            print(f"[compare] {name} seed={seed}: {total} ({time.time() - t0:.0f}s)", flush=True)
        rate = total.mismatches / max(total.decisions, 1)
        passed = not total.hard and rate < MAX_MISMATCH_RATE
        ok &= passed
        print(json.dumps({"workload": name, "logit_seeds": seeds, "uniform_sets_per_seed": used_sets,
                          "decisions": total.decisions, "sampled": total.decisions - total.greedy,
                          "in_window": total.in_window, "boundary_mismatches": total.mismatches,
                          "hard": len(total.hard), "hard_examples": [str(h) for h in total.hard[:5]],
                          "mismatch_rate": rate, "pass": passed}), flush=True)
    return ok


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    sub = ap.add_subparsers(dest="phase", required=True)
    g = sub.add_parser("gpu")
    g.add_argument("--out", required=True)
    g.add_argument("--only", nargs="*", default=[])
    g.add_argument("--sets", type=int, default=None, help="uniform sets per logit seed (a quick run)")
    c = sub.add_parser("compare")
    c.add_argument("--dir", required=True)
    c.add_argument("--workers", type=int, default=min(16, len(os.sched_getaffinity(0))))
    c.add_argument("--only", nargs="*", default=[])
    a = ap.parse_args()
    if a.phase == "gpu":
        gpu_phase(a.out, set(a.only), a.sets)
        return 0
    return 0 if compare_phase(a.dir, a.workers, set(a.only)) else 1


if __name__ == "__main__":
    sys.exit(main())
