"""GPU parity of spec_verify_chain_topk (p and q both filtered to their rows'
top-k logits before verification) against the fp64 oracle, through the C
ABI."""
import numpy as np
import pytest

import oracle
import synth
import rejection_sampling_verify_15_amd as sv
from parity import Tally, assert_shared_workspace_zero, compare_chain, to_device, to_device_logits

pytestmark = pytest.mark.gpu


def run_topk(ci, top_k, u_sets, target=None, draft=None, tokens=None, top_p=None):
    tgt = to_device_logits(ci.target if target is None else target, ci.dtype)
    drf = to_device_logits(ci.draft if draft is None else draft, ci.dtype)
    tok = to_device((ci.draft_tokens if tokens is None else tokens).astype(np.int32))
    T = to_device(ci.temperature.astype(np.float32))
    k = to_device(np.asarray(top_k, np.int32))
    pd = None if top_p is None else to_device(np.asarray(top_p, np.float32))
    outs = []
    for u in u_sets:
        ot, on = sv.verify_chain_topk(tgt, drf, tok, to_device(np.asarray(u, np.float32)), T, k, top_p=pd)
        outs.append((ot.cpu().numpy(), on.cpu().numpy()))
    assert_shared_workspace_zero("chain topk")
    return outs


def topk_parity(ci, top_k, n_sets, label, seed=9, target=None, draft=None, tokens=None, top_p=None):
    u_sets = [ci.uniforms] + [ci.fresh_uniforms(seed * 1000 + s) for s in range(n_sets - 1)]
    print(f"[{label}] B={ci.B} gamma={ci.gamma} V={ci.V} dtype={ci.dtype} sets={n_sets}", flush=True)
    gpu = run_topk(ci, top_k, u_sets, target, draft, tokens, top_p)
    tgt = ci.target if target is None else target
    drf = ci.draft if draft is None else draft
    tok = ci.draft_tokens if tokens is None else tokens
    tally = Tally()
    refs = []
    for (ot, on), u in zip(gpu, u_sets):
        ref = oracle.verify_chain_topk(tgt, drf, tok, u, ci.temperature, np.asarray(top_k), ci.dtype,
                                       top_p=None if top_p is None else np.asarray(top_p, np.float32))
        tally.add(compare_chain(ref, ot, on))
        refs.append(ref)
    print(f"[{label}] {tally}", flush=True)
    tally.check(label)
    return gpu, refs


def filtered_draft_tokens(ci, top_k, seed, top_p=None):
    """Draft tokens drawn from the filtered draft distributions (the
    consistent setting), by Gumbel-max over the kept logits."""
    rng = np.random.default_rng(seed)
    from oracle import specverify_oracle as so
    toks = ci.draft_tokens.copy()
    for b in range(ci.B):
        T = max(float(ci.temperature[b]), 0.0)
        d = so.logits_to_f64(ci.draft[b], ci.dtype)
        for i in range(ci.gamma):
            if T > 0.0:
                # requests with an invalid k draw from a clamped one
                f, _ = oracle.topk_filter(d[i], min(max(int(top_k[b]), 1), oracle.TOPK_MAX))
                if top_p is not None and 0.0 < float(top_p[b]) < 1.0:
                    f, _ = oracle.topp_filter(f, float(np.float32(top_p[b])), T)
                toks[b, i] = int(np.argmax(f / T + rng.gumbel(size=ci.V)))
            else:
                toks[b, i] = int(np.argmax(d[i]))
    return toks


def test_topk_batched_shape():
    """B=64, gamma=4, V=128256 bf16, even requests sampling at T=0.7 with
    k=50 (drafts drawn from the filtered q), odd ones greedy."""
    ci = synth.batched_chain()
    k = np.full(ci.B, 50, np.int32)
    toks = filtered_draft_tokens(ci, k, 15900)
    gpu, refs = topk_parity(ci, k, 3, "topk batched k=50", tokens=toks)
    assert max(int(on.max()) for _, on in gpu) >= 2
    assert all((r.num_accepted >= 0).all() for r in refs)


@pytest.mark.parametrize("dtype,V", [("bf16", 151936), ("f32", 300000)])
def test_topk_long_rows(dtype, V):
    """Rows long enough that the candidate visit reloads by batch of loads:
    bf16 tiles past 32 steps per thread, and fp32 tiles of more than eight
    batches (several batches to a slot)."""
    ci = synth.chain_inputs(15980 + V % 89, B=6, gamma=2, V=V, dtype=dtype, family="gauss",
                            draft_sigma=(0.2, 1.2), temperature=0.8, greedy_odd=True)
    k = np.array([1, 7, 50, 128, 3, 100], np.int32)
    toks = filtered_draft_tokens(ci, k, 15981)
    topk_parity(ci, k, 6, f"topk long rows {dtype} V={V}", tokens=toks)


@pytest.mark.parametrize("dtype,V", [("bf16", 3000), ("f32", 999), ("bf16", 20001)])
def test_topk_small_many_rounds(dtype, V):
    """k varying per request over [1, 128], close and far drafts, odd
    requests greedy; V=999 and V=20001 run the scalar path."""
    ci = synth.chain_inputs(15910 + V % 97, B=40, gamma=6, V=V, dtype=dtype, family="gauss",
                            draft_sigma=(0.1, 1.5), temperature=0.9, greedy_odd=True)
    rng = np.random.default_rng(15911)
    k = rng.integers(1, 129, size=ci.B).astype(np.int32)
    k[:4] = [1, 2, 128, min(V, 128)]
    toks = filtered_draft_tokens(ci, k, 15912)
    topk_parity(ci, k, 15, f"topk {dtype} V={V}", tokens=toks)


def test_topk_ties_at_the_threshold_and_overflow():
    """fp32 logits rounded to 0.25 (many ties straddle the threshold); one row
    with 300 tied maxima (more than 256 kept: the request is invalid)."""
    ci = synth.chain_inputs(15920, B=24, gamma=3, V=4096, dtype="f32", family="gauss",
                            draft_sigma=(0.2, 1.0), temperature=1.0, greedy_odd=True)
    tgt = (np.round(ci.target * 4.0) / 4.0).astype(np.float32)
    drf = (np.round(ci.draft * 4.0) / 4.0).astype(np.float32)
    tgt[2, 1, :300] = 9.0
    ci.target, ci.draft = tgt, drf
    k = np.full(ci.B, 20, np.int32)
    toks = filtered_draft_tokens(ci, k, 15921)
    gpu, refs = topk_parity(ci, k, 8, "topk ties", tokens=toks)
    assert refs[0].num_accepted[2] == -1 and (gpu[0][1][2] == -1)
    assert (refs[0].num_accepted[[0, 4, 6]] >= 0).all()


def test_topk_bisection_fallback():
    """A flat background lets every thread maximum equal it, so far more than
    1024 logits pass the lower bound and the exact bisection runs; the 128
    distinct top logits sit in one contiguous block."""
    B, G, V = 6, 2, 20000
    rng = np.random.default_rng(15930)
    tgt = np.full((B, G + 1, V), -1.0, np.float32)
    drf = np.full((B, G, V), -1.0, np.float32)
    for b in range(B):
        for r in range(G + 1):
            s = int(rng.integers(0, V - 200))
            tgt[b, r, s:s + 200] = np.sort(rng.uniform(2.0, 6.0, 200)).astype(np.float32)
        for r in range(G):
            s = int(rng.integers(0, V - 200))
            drf[b, r, s:s + 200] = rng.uniform(2.0, 6.0, 200).astype(np.float32)
    ci = synth.ChainInputs(tgt, drf, np.zeros((B, G), np.int32), synth.uniforms(rng, (B, G + 1)),
                           np.full(B, 1.0, np.float32), "f32", B, G, V, "flat", "flat background")
    k = np.array([128, 64, 100, 1, 128, 7], np.int32)
    toks = filtered_draft_tokens(ci, k, 15931)
    gpu, refs = topk_parity(ci, k, 8, "topk bisection", tokens=toks)
    assert (refs[0].num_accepted >= 0).all()


def test_topk_invalid_requests():
    ci = synth.chain_inputs(15940, B=10, gamma=3, V=2048, dtype="bf16", family="peaked",
                            draft_sigma=0.5, temperature=1.0)
    k = np.full(ci.B, 16, np.int32)
    k[1], k[2] = 0, 129
    ci.temperature[3] = 0.0
    k[3] = 0                          # greedy: k is ignored
    ci.temperature[4] = -1.0
    toks = filtered_draft_tokens(ci, k, 15941)
    toks[5, 1] = ci.V
    gpu, refs = topk_parity(ci, k, 2, "topk invalid", tokens=toks)
    on = gpu[0][1]
    assert (on[[1, 2, 4, 5]] == -1).all() and (on[[0, 3, 6]] >= 0).all()


def test_top1_with_argmax_drafts_equals_the_greedy_call():
    """k = 1 keeps a row's maximum alone unless it is tied (bf16 rows tie
    now and then): requests whose rows all have a single maximum give the
    greedy call's output, and every request matches the oracle."""
    ci = synth.chain_inputs(15950, B=32, gamma=4, V=30000, dtype="bf16", family="gauss",
                            draft_sigma=(0.05, 0.8), temperature=0.8)
    wide_d = synth.bf16_bits_as_float32(ci.draft)
    wide_t = synth.bf16_bits_as_float32(ci.target)
    toks = np.argmax(wide_d, axis=2).astype(np.int32)
    k = np.ones(ci.B, np.int32)
    gpu, _ = topk_parity(ci, k, 1, "topk k=1", tokens=toks)
    ot, on = gpu[0]
    tgt = to_device_logits(ci.target, ci.dtype)
    gt, gn = sv.verify_chain(tgt, None, to_device(toks), to_device(ci.uniforms),
                             to_device(np.zeros(ci.B, np.float32)))
    gt, gn = gt.cpu().numpy(), gn.cpu().numpy()

    def single_max(rows):
        return ((rows == rows.max(axis=-1, keepdims=True)).sum(axis=-1) == 1).all(axis=-1)
    one = single_max(wide_t) & single_max(wide_d)
    assert one.sum() >= 12
    assert np.array_equal(ot[one], gt[one]) and np.array_equal(on[one], gn[one])
    assert on.max() >= 2


def test_topk_longest_draft_interleaved_with_the_plain_call():
    """gamma = 32 (65 rows per request), and top-k calls alternating with
    plain calls on the one shared workspace: each matches its oracle."""
    ci = synth.chain_inputs(15960, B=6, gamma=32, V=5000, dtype="bf16", family="gauss",
                            draft_sigma=(0.02, 0.3), temperature=1.0, greedy_odd=True)
    k = np.array([128, 1, 40, 7, 99, 3], np.int32)
    toks = filtered_draft_tokens(ci, k, 15961)
    tgt, drf = to_device_logits(ci.target, ci.dtype), to_device_logits(ci.draft, ci.dtype)
    tok, T, kd = to_device(toks), to_device(ci.temperature), to_device(k)
    t_topk, t_plain = Tally(), Tally()
    deepest = 0
    for s in range(6):
        u = ci.uniforms if s == 0 else ci.fresh_uniforms(15962 + s)
        ot, on = sv.verify_chain_topk(tgt, drf, tok, to_device(u), T, kd)
        ref = oracle.verify_chain_topk(ci.target, ci.draft, toks, u, ci.temperature, k, "bf16")
        t_topk.add(compare_chain(ref, ot.cpu().numpy(), on.cpu().numpy()))
        deepest = max(deepest, int(on.max()))
        pt, pn = sv.verify_chain(tgt, drf, tok, to_device(u), T)
        pref = oracle.verify_chain(ci.target, ci.draft, toks, u, ci.temperature, "bf16")
        t_plain.add(compare_chain(pref, pt.cpu().numpy(), pn.cpu().numpy()))
        assert_shared_workspace_zero("topk then plain")
    print(f"[topk gamma=32] {t_topk} deepest={deepest}; [plain] {t_plain}", flush=True)
    t_topk.check("topk gamma=32")
    t_plain.check("plain after topk")
    assert deepest >= 8


def test_topk_graph_capture_replays_match_eager():
    """One top-k call captured in a HIP graph and replayed, with eager calls
    on other uniforms between the replays: every replay gives the eager
    result and the workspace stays zero."""
    import torch
    ci = synth.chain_inputs(15970, B=12, gamma=4, V=20000, dtype="bf16", family="peaked",
                            draft_sigma=(0.3, 2.0), temperature=0.8, greedy_odd=True)
    k = np.full(ci.B, 32, np.int32)
    toks = filtered_draft_tokens(ci, k, 15971)
    dev = torch.device("cuda")
    tgt, drf = to_device_logits(ci.target, ci.dtype), to_device_logits(ci.draft, ci.dtype)
    tok, T, kd, u0 = to_device(toks), to_device(ci.temperature), to_device(k), to_device(ci.uniforms)
    need = sv.lib().sv_chain_topk_workspace_bytes(ci.B, ci.gamma, ci.V, 0)
    ws = torch.zeros(need, dtype=torch.uint8, device=dev)
    want = [x.clone() for x in sv.verify_chain_topk(tgt, drf, tok, u0, T, kd, ws=ws)]
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            got = sv.verify_chain_topk(tgt, drf, tok, u0, T, kd, ws=ws)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    for r in range(4):
        for x in got:
            x.fill_(-7)
        g.replay()
        torch.cuda.synchronize()
        for x, y in zip(got, want):
            assert torch.equal(x, y), f"replay {r}"
        assert int(ws.count_nonzero()) == 0
        sv.verify_chain_topk(tgt, drf, tok, to_device(ci.fresh_uniforms(15972 + r)), T, kd, ws=ws)
        torch.cuda.synchronize()
        assert int(ws.count_nonzero()) == 0


def test_topp_batched_shape():
    """The batched shape with k = 50 and p = 0.9 on every sampling request."""
    ci = synth.batched_chain()
    k = np.full(ci.B, 50, np.int32)
    p = np.full(ci.B, 0.9, np.float32)
    toks = filtered_draft_tokens(ci, k, 15980, top_p=p)
    gpu, refs = topk_parity(ci, k, 3, "topk+topp batched", tokens=toks, top_p=p)
    assert all((r.num_accepted >= 0).all() for r in refs)


@pytest.mark.parametrize("dtype,V", [("bf16", 3000), ("f32", 999), ("bf16", 20001)])
def test_topp_small_many_rounds(dtype, V):
    ci = synth.chain_inputs(15985 + V % 89, B=40, gamma=5, V=V, dtype=dtype, family="gauss",
                            draft_sigma=(0.1, 1.5), temperature=0.8, greedy_odd=True)
    rng = np.random.default_rng(15986)
    k = rng.integers(1, 129, size=ci.B).astype(np.int32)
    p = rng.choice(np.array([0.2, 0.5, 0.8, 0.9, 0.97, 1.0], np.float32), size=ci.B)
    toks = filtered_draft_tokens(ci, k, 15987, top_p=p)
    topk_parity(ci, k, 12, f"topk+topp {dtype} V={V}", tokens=toks, top_p=p)


def test_topp_after_the_bisection_fallback_and_bad_p():
    """Flat rows (the bisection path) with top-p, and p values outside
    (0, 1] (invalid requests)."""
    B, G, V = 8, 2, 20000
    rng = np.random.default_rng(15990)
    tgt = np.full((B, G + 1, V), -1.0, np.float32)
    drf = np.full((B, G, V), -1.0, np.float32)
    for b in range(B):
        for r in range(G + 1):
            s0 = int(rng.integers(0, V - 200))
            tgt[b, r, s0:s0 + 200] = rng.uniform(2.0, 6.0, 200).astype(np.float32)
        for r in range(G):
            s0 = int(rng.integers(0, V - 200))
            drf[b, r, s0:s0 + 200] = rng.uniform(2.0, 6.0, 200).astype(np.float32)
    ci = synth.ChainInputs(tgt, drf, np.zeros((B, G), np.int32), synth.uniforms(rng, (B, G + 1)),
                           np.full(B, 1.0, np.float32), "f32", B, G, V, "flat", "flat background")
    k = np.array([128, 64, 100, 128, 128, 50, 50, 50], np.int32)
    p = np.array([0.5, 0.9, 0.99, 1.0, 0.05, 0.0, 1.5, np.nan], np.float32)
    toks = filtered_draft_tokens(ci, k, 15991, top_p=np.where(np.isfinite(p) & (p > 0) & (p <= 1), p, 1.0))
    gpu, refs = topk_parity(ci, k, 6, "topk+topp bisection", tokens=toks, top_p=p)
    on = gpu[0][1]
    assert (on[:5] >= 0).all() and (on[5:] == -1).all()


def test_tiny_top_p_with_argmax_drafts_equals_the_greedy_call():
    ci = synth.chain_inputs(15995, B=32, gamma=4, V=30000, dtype="f32", family="gauss",
                            draft_sigma=(0.05, 0.8), temperature=0.8)
    toks = np.argmax(ci.draft, axis=2).astype(np.int32)
    k = np.full(ci.B, 64, np.int32)
    p = np.full(ci.B, 1e-6, np.float32)
    gpu, _ = topk_parity(ci, k, 1, "topk+topp tiny p", tokens=toks, top_p=p)
    ot, on = gpu[0]
    gt, gn = sv.verify_chain(to_device_logits(ci.target, ci.dtype), None, to_device(toks), to_device(ci.uniforms),
                             to_device(np.zeros(ci.B, np.float32)))
    assert np.array_equal(ot, gt.cpu().numpy()) and np.array_equal(on, gn.cpu().numpy())
