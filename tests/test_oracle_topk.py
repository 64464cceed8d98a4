"""Pins of the oracle's consistent top-k verification (CPU only).

- The filter's threshold is the k-th largest value with multiplicity: the
  same as the last value torch.topk returns, on rows full of ties.
- The lossless theorem for the filtered target: by exact enumeration, the
  emitted tokens follow p' = softmax(topk-masked target / T), with p' and q'
  built here from torch.topk and torch.softmax, not from the oracle.
- A planted mistake (drafts from the filtered q' tested against the
  unfiltered q) breaks that law.
- k = 1 with drafts sampled from the filtered q (its argmax) is greedy
  verification; k >= V is the unfiltered call.
- The contract limits: k outside [1, 128], or a row keeping more than 256
  logits, makes a sampling request invalid; greedy requests ignore k.
"""
import numpy as np
import torch

import oracle
from oracle import specverify_oracle as so
import synth
from enum_tools import enumerate_round, slot_marginals


def library_topk_mask(row, k):
    x = torch.as_tensor(np.asarray(row, np.float64))
    kk = min(int(k), x.numel())
    thr = torch.topk(x, kk).values[-1]
    return (x >= thr).numpy(), float(thr)


def library_filtered_probs(row, k, T):
    keep, _ = library_topk_mask(row, k)
    x = torch.as_tensor(np.asarray(row, np.float64)) / T
    x = torch.where(torch.as_tensor(keep), x, torch.tensor(-np.inf, dtype=torch.float64))
    return torch.softmax(x, 0).numpy()


def test_threshold_is_the_kth_largest_with_ties():
    rng = np.random.default_rng(15800)
    for trial in range(200):
        V = int(rng.integers(1, 400))
        # few distinct values, so that ties straddle the threshold; -inf too
        vals = rng.choice(np.array([-np.inf, -3.0, -1.0, 0.0, 0.5, 2.0, 2.5, 7.0]), size=V)
        if trial % 3 == 0:
            vals = rng.standard_normal(V)
        for k in (1, 2, 3, 7, V - 1, V, V + 5):
            if k < 1:
                continue
            filt, count = oracle.topk_filter(vals, k)
            keep, thr = library_topk_mask(vals, k)
            assert np.array_equal(np.isfinite(filt) | (vals == -np.inf) & keep, keep)
            assert count == keep.sum() >= min(k, V)
            assert np.array_equal(filt[keep], vals[keep]) and (filt[~keep] == -np.inf).all()
            # the k-th largest value itself is kept, nothing above it is dropped
            assert (vals[vals > thr] == filt[vals > thr]).all()


def test_signed_zeros_tie():
    row = np.array([-0.0, 0.0, -1.0, 0.0, -0.0])
    filt, count = oracle.topk_filter(row, 1)
    assert count == 4 and (filt[[0, 1, 3, 4]] == 0.0).all() and filt[2] == -np.inf


def decider_topk(tgt_rows, drf_rows, k, T):
    """The oracle's batch entry point as a black box on one request."""
    G = drf_rows.shape[0]

    def decide(tokens, u):
        res = oracle.verify_chain_topk(tgt_rows[None].astype(np.float32), drf_rows[None].astype(np.float32),
                                       np.asarray([tokens], np.int32), np.asarray([u], np.float32),
                                       np.array([T], np.float32), np.array([k], np.int32), "f32")
        n = int(res.num_accepted[0])
        return [int(t) for t in res.out_tokens[0, :n + 1]], n
    return decide


def enumerate_topk(seed, V, G, k, T, filter_q=True):
    rng = np.random.default_rng(seed)
    tgt = np.round(rng.standard_normal((G + 1, V)) * 1.5, 2).astype(np.float32)
    drf = (tgt[:G] + np.round(rng.standard_normal((G, V)), 2)).astype(np.float32)
    P = [library_filtered_probs(tgt[i], k, T) for i in range(G + 1)]
    Q = [library_filtered_probs(drf[i], k, T) for i in range(G)]
    Qd = Q if filter_q else [library_filtered_probs(drf[i], V, T) for i in range(G)]
    # drafts come from the (filtered) draft distribution
    law = enumerate_round(P, Qd, decider_topk(tgt, drf, k, T))
    return P, law


def test_emitted_tokens_follow_the_filtered_target():
    for seed, V, G, k, T in ((15810, 5, 2, 3, 0.8), (15811, 6, 2, 2, 1.3), (15812, 5, 1, 4, 0.5)):
        P, law = enumerate_topk(seed, V, G, k, T)
        reach, cond = slot_marginals(law, V, G + 1)
        assert abs(sum(law.values()) - 1.0) < 1e-12
        for s in range(G + 1):
            if reach[s] > 1e-12:
                np.testing.assert_allclose(cond[s], P[s], atol=1e-12)
        # the filtered-out tokens are never emitted
        for seq in law:
            for s, t in enumerate(seq):
                assert P[s][t] > 0.0


def test_planted_mistake_unfiltered_q_in_the_test_is_biased(monkeypatch):
    """Drafts drawn from the filtered q', and an oracle planted to filter only
    the target rows (its accept ratio and residual use the unfiltered q):
    the emitted law is no longer p'.  Drafts from the unfiltered q through
    the real oracle are biased too: the rule must be the same on both sides."""
    real = so.topk_filter
    seed, V, G, k, T = 15820, 5, 1, 2, 1.0
    rng = np.random.default_rng(seed)
    tgt = np.round(rng.standard_normal((G + 1, V)) * 1.5, 2).astype(np.float32)
    drf = (tgt[:G] + np.round(rng.standard_normal((G, V)), 2)).astype(np.float32)
    P = [library_filtered_probs(tgt[i], k, T) for i in range(G + 1)]
    Qf = [library_filtered_probs(drf[i], k, T) for i in range(G)]
    Qfull = [library_filtered_probs(drf[i], V, T) for i in range(G)]
    inner = decider_topk(tgt, drf, k, T)
    calls = {"n": 0}

    def target_only(row, kk):
        # verify_chain_topk filters the G + 1 target rows first, then the draft rows
        calls["n"] += 1
        return real(row, kk if calls["n"] <= G + 1 else 10 ** 9)

    def planted(tokens, u):
        calls["n"] = 0
        return inner(tokens, u)

    def law_of(Qdraws):
        return lambda tup: float(np.prod([Qdraws[i][tup[i]] for i in range(G)]))

    # the enumeration places its uniforms by the verifier's own rule (the
    # second argument) and weighs the draft tuples by the draft law
    monkeypatch.setattr(so, "topk_filter", target_only)
    _, cond = slot_marginals(enumerate_round(P, Qfull, planted, draft_law=law_of(Qf)), V, 1)
    assert np.abs(cond[0] - P[0]).sum() > 1e-2
    monkeypatch.setattr(so, "topk_filter", real)
    _, cond = slot_marginals(enumerate_round(P, Qf, inner, draft_law=law_of(Qfull)), V, 1)
    assert np.abs(cond[0] - P[0]).sum() > 1e-2
    _, cond = slot_marginals(enumerate_round(P, Qf, inner), V, 1)
    np.testing.assert_allclose(cond[0], P[0], atol=1e-12)


def test_top1_with_argmax_drafts_is_greedy():
    ci = synth.chain_inputs(15830, B=40, gamma=4, V=700, dtype="f32", family="gauss",
                            draft_sigma=(0.1, 1.0), temperature=0.9)
    drf = ci.draft.astype(np.float64)
    toks = np.argmax(drf, axis=2).astype(np.int32)       # the filtered q is a point mass there
    toks[::3, 1] = np.argmax(ci.target[::3, 1], axis=1)  # some forced matches deeper in
    assert (ci.uniforms > 0).all()
    got = oracle.verify_chain_topk(ci.target, ci.draft, toks, ci.uniforms, ci.temperature,
                                   np.ones(ci.B, np.int32), "f32")
    ref = oracle.verify_chain(ci.target, ci.draft, toks, ci.uniforms, np.zeros(ci.B, np.float32), "f32")
    assert np.array_equal(got.out_tokens, ref.out_tokens)
    assert np.array_equal(got.num_accepted, ref.num_accepted)
    assert got.num_accepted.max() >= 2


def test_k_at_least_V_is_the_unfiltered_call():
    ci = synth.chain_inputs(15840, B=24, gamma=3, V=90, dtype="bf16", family="peaked",
                            draft_sigma=(0.3, 2.0), temperature=0.8, greedy_odd=True)
    ref = oracle.verify_chain(ci.target, ci.draft, ci.draft_tokens, ci.uniforms, ci.temperature, "bf16")
    for k in (90, 128):
        got = oracle.verify_chain_topk(ci.target, ci.draft, ci.draft_tokens, ci.uniforms, ci.temperature,
                                       np.full(ci.B, k, np.int32), "bf16")
        assert np.array_equal(got.out_tokens, ref.out_tokens)
        assert np.array_equal(got.num_accepted, ref.num_accepted)


def test_contract_limits():
    ci = synth.chain_inputs(15850, B=6, gamma=2, V=400, dtype="f32", family="gauss",
                            draft_sigma=0.5, temperature=1.0)
    tgt = ci.target.copy()
    tgt[1, 1, :300] = 9.0                       # 300 tied maxima: too many kept for any k
    k = np.array([5, 5, 0, 129, 128, 0], np.int32)
    T = ci.temperature.copy()
    T[5] = 0.0                                  # greedy: k is ignored
    got = oracle.verify_chain_topk(tgt, ci.draft, ci.draft_tokens, ci.uniforms, T, k, "f32")
    assert got.num_accepted[0] >= 0 and got.num_accepted[4] >= 0 and got.num_accepted[5] >= 0
    assert (got.num_accepted[1:4] == -1).all() and (got.out_tokens[1:4] == -1).all()
    # 256 tied values are still within the limit
    tgt[1, 1, :300] = 0.0
    tgt[1, 1, :256] = 9.0
    got = oracle.verify_chain_topk(tgt, ci.draft, ci.draft_tokens, ci.uniforms, T, k, "f32")
    assert got.num_accepted[1] >= 0


# ---------------------------------------------------------------------------
# top-p after top-k (R19)
# ---------------------------------------------------------------------------
def library_topp_mask(row, k, p, T):
    """Sort the top-k logits, cumulate their softmax mass in that order and
    cut at the first position reaching p (rows without ties)."""
    keep, _ = library_topk_mask(row, k)
    x = torch.as_tensor(np.asarray(row, np.float64))
    kept_vals = x[torch.as_tensor(keep)]
    srt = torch.sort(kept_vals, descending=True).values
    cum = torch.cumsum(torch.softmax(srt / T, 0), 0)
    cut = int(torch.nonzero(cum >= p)[0]) if p < 1.0 else len(srt) - 1
    return (x >= srt[cut]).numpy() & keep


def library_topkp_probs(row, k, p, T):
    keep = library_topp_mask(row, k, p, T)
    x = torch.as_tensor(np.asarray(row, np.float64)) / T
    x = torch.where(torch.as_tensor(keep), x, torch.tensor(-np.inf, dtype=torch.float64))
    return torch.softmax(x, 0).numpy()


def test_topp_cut_matches_sorted_cumsum():
    rng = np.random.default_rng(15860)
    for _ in range(300):
        V = int(rng.integers(2, 300))
        row = rng.standard_normal(V) * rng.uniform(0.3, 3.0)
        k = int(rng.integers(1, 129))
        p = float(rng.choice([1e-6, 0.1, 0.5, 0.8, 0.9, 0.95, 0.999, 1.0]))
        T = float(rng.uniform(0.3, 2.0))
        fk, _ = oracle.topk_filter(row, k)
        fp, count = oracle.topp_filter(fk, p, T)
        want = library_topp_mask(row, k, p, T)
        assert np.array_equal(np.isfinite(fp), want) and count == want.sum()


def test_topp_keeps_every_tie_at_the_cut():
    row = np.array([5.0, 3.0, 1.0, 3.0, 3.0, -2.0])
    fk, _ = oracle.topk_filter(row, 6)
    r = oracle.softmax_t(fk, 1.0)
    p = r[0] + r[1] / 2.0                      # the cut falls inside the three tied 3.0s
    fp, count = oracle.topp_filter(fk, p, 1.0)
    assert count == 4 and np.isfinite(fp[[0, 1, 3, 4]]).all() and not np.isfinite(fp[[2, 5]]).any()
    fp, count = oracle.topp_filter(fk, r[0] * 0.999, 1.0)
    assert count == 1 and np.isfinite(fp[0])


def decider_topkp(tgt_rows, drf_rows, k, p, T):
    def decide(tokens, u):
        res = oracle.verify_chain_topk(tgt_rows[None].astype(np.float32), drf_rows[None].astype(np.float32),
                                       np.asarray([tokens], np.int32), np.asarray([u], np.float32),
                                       np.array([T], np.float32), np.array([k], np.int32), "f32",
                                       top_p=np.array([p], np.float32))
        n = int(res.num_accepted[0])
        return [int(t) for t in res.out_tokens[0, :n + 1]], n
    return decide


def test_emitted_tokens_follow_the_top_k_top_p_target():
    cut_any = False
    for seed, V, G, k, p, T in ((15870, 6, 2, 5, 0.7, 0.9), (15871, 5, 1, 4, 0.5, 1.2), (15872, 6, 2, 6, 0.9, 0.6)):
        rng = np.random.default_rng(seed)
        tgt = np.round(rng.standard_normal((G + 1, V)) * 1.5, 2).astype(np.float32)
        drf = (tgt[:G] + np.round(rng.standard_normal((G, V)), 2)).astype(np.float32)
        pf = float(np.float32(p))
        P = [library_topkp_probs(tgt[i], k, pf, T) for i in range(G + 1)]
        Q = [library_topkp_probs(drf[i], k, pf, T) for i in range(G)]
        law = enumerate_round(P, Q, decider_topkp(tgt, drf, k, p, T))
        reach, cond = slot_marginals(law, V, G + 1)
        for s in range(G + 1):
            if reach[s] > 1e-12:
                np.testing.assert_allclose(cond[s], P[s], atol=1e-12)
        cut_any = cut_any or (P[0] > 0).sum() < min(k, V)
    assert cut_any                              # top-p cut below the top-k set somewhere


def test_topp_special_cases_and_limits():
    ci = synth.chain_inputs(15880, B=30, gamma=4, V=500, dtype="f32", family="gauss",
                            draft_sigma=(0.1, 1.0), temperature=0.9)
    k = np.full(ci.B, 40, np.int32)
    plain = oracle.verify_chain_topk(ci.target, ci.draft, ci.draft_tokens, ci.uniforms, ci.temperature, k, "f32")
    one = oracle.verify_chain_topk(ci.target, ci.draft, ci.draft_tokens, ci.uniforms, ci.temperature, k, "f32",
                                   top_p=np.ones(ci.B, np.float32))
    assert np.array_equal(plain.out_tokens, one.out_tokens) and np.array_equal(plain.num_accepted, one.num_accepted)
    # a tiny p keeps the maximum alone (no ties in fp32 gaussian rows): greedy
    toks = np.argmax(ci.draft, axis=2).astype(np.int32)
    tiny = oracle.verify_chain_topk(ci.target, ci.draft, toks, ci.uniforms, ci.temperature, k, "f32",
                                    top_p=np.full(ci.B, 1e-6, np.float32))
    greedy = oracle.verify_chain(ci.target, ci.draft, toks, ci.uniforms, np.zeros(ci.B, np.float32), "f32")
    assert np.array_equal(tiny.out_tokens, greedy.out_tokens)
    bad = np.array([0.0, -0.5, 1.5, np.nan] + [0.9] * (ci.B - 4), np.float32)
    got = oracle.verify_chain_topk(ci.target, ci.draft, ci.draft_tokens, ci.uniforms, ci.temperature, k, "f32",
                                   top_p=bad)
    assert (got.num_accepted[:4] == -1).all() and (got.num_accepted[4:] >= 0).all()
