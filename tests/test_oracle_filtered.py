"""Pins of the oracle's general consistent filter, R20 (CPU only).

- The sorted top-p cut keeps exactly what the brute-force definition
  (`topp_filter`: every kept value v, its mass M(v) summed directly) keeps,
  on rows full of ties, signed zeros and -inf, and what a torch
  sort-and-cumsum reference keeps on rows without ties.  Its margin is
  min(M(v*) - p, p - M(v+)) recomputed by brute force.
- Within the top-k path's limits (k <= 128, at most 256 kept logits) the
  general call equals `verify_chain_topk`, with and without top-p; with no
  filter, k >= V or p = 1 it equals `verify_chain`.
- The lossless theorem for top-p alone and for a large k: by exact
  enumeration, the emitted tokens follow the filtered target, built here with
  torch.  A planted mistake (top-p applied to the target rows only) breaks
  that law.
- Invalid k or p make a sampling request invalid; greedy requests ignore both.
"""
import numpy as np
import pytest
import torch

import oracle
from oracle import specverify_oracle as so
import synth
from enum_tools import enumerate_round, slot_marginals


def brute_mass(row, v, T):
    r = oracle.softmax_t(row, T)
    return float(r[np.isfinite(row) & (row >= v)].sum())


def tie_rows(rng, n):
    for i in range(n):
        V = int(rng.integers(1, 200))
        if i % 3 == 0:
            row = rng.standard_normal(V) * rng.uniform(0.3, 3.0)
        else:
            row = rng.choice(np.array([-np.inf, -2.0, -0.0, 0.0, 0.5, 1.0, 2.0, 4.0]), size=V)
        yield row


def test_sorted_cut_equals_the_brute_force_definition():
    rng = np.random.default_rng(16400)
    checked = 0
    for row in tie_rows(rng, 600):
        for p in (1e-7, 0.05, 0.3, 0.5, 0.77, 0.9, 0.999, 1.0):
            T = float(rng.uniform(0.3, 2.0))
            if not np.isfinite(row).any():
                continue
            v, margin = oracle.topp_cut(row, p, T)
            kept_sorted = np.isfinite(row) & (row >= v)
            fp, count = oracle.topp_filter(row, p, T)
            assert np.array_equal(kept_sorted, np.isfinite(fp)), (row, p, T)
            assert count == kept_sorted.sum()
            if p < 1.0:
                M = brute_mass(row, v, T)
                above = np.unique(row[np.isfinite(row) & (row > v)])
                Mp = brute_mass(row, above.min(), T) if above.size else 0.0
                assert M >= p > Mp
                assert abs(margin - min(M - p, p - Mp)) < 1e-12
            else:
                assert v == -np.inf and margin == np.inf
            checked += 1
    assert checked > 3000


def test_sorted_cut_matches_torch_sort_and_cumsum():
    rng = np.random.default_rng(16401)
    for _ in range(300):
        V = int(rng.integers(2, 5000))
        row = rng.standard_normal(V) * rng.uniform(0.3, 3.0)
        p = float(rng.choice([1e-6, 0.1, 0.5, 0.9, 0.95, 0.999]))
        T = float(rng.uniform(0.3, 2.0))
        x = torch.as_tensor(row)
        srt = torch.sort(x, descending=True).values
        cum = torch.cumsum(torch.softmax(srt / T, 0), 0)
        cut = int(torch.nonzero(cum >= p)[0])
        want = (x >= srt[cut]).numpy()
        v, _ = oracle.topp_cut(row, p, T)
        assert np.array_equal(row >= v, want)


def test_signed_zeros_tie_at_the_cut():
    row = np.array([1.0, -0.0, 0.0, -0.0, -3.0])
    r = oracle.softmax_t(row, 1.0)
    v, _ = oracle.topp_cut(row, r[0] + r[1] / 2.0, 1.0)
    assert v == 0.0 and (row >= v).sum() == 4


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_equals_the_topk_call_within_its_limits(dtype):
    ci = synth.chain_inputs(16410, B=24, gamma=3, V=3000, dtype=dtype, family="peaked",
                            draft_sigma=(0.3, 2.0), temperature=0.8, greedy_odd=True)
    rng = np.random.default_rng(16411)
    k = rng.integers(1, 129, size=ci.B).astype(np.int32)
    p = rng.choice(np.array([0.3, 0.8, 0.95, 1.0], np.float32), size=ci.B)
    for top_p in (None, p):
        a = oracle.verify_chain_topk(ci.target, ci.draft, ci.draft_tokens, ci.uniforms, ci.temperature, k, dtype,
                                     top_p=top_p)
        b = oracle.verify_chain_filtered(ci.target, ci.draft, ci.draft_tokens, ci.uniforms, ci.temperature, dtype,
                                         top_k=k, top_p=top_p)
        assert np.array_equal(a.out_tokens, b.out_tokens) and np.array_equal(a.num_accepted, b.num_accepted)
        assert (b.num_accepted >= 0).all()


def test_no_filter_is_the_plain_call():
    ci = synth.chain_inputs(16420, B=20, gamma=4, V=700, dtype="bf16", family="zipf",
                            draft_sigma=0.8, temperature=1.0, greedy_odd=True)
    ref = oracle.verify_chain(ci.target, ci.draft, ci.draft_tokens, ci.uniforms, ci.temperature, "bf16")
    for kw in ({}, {"top_k": np.full(ci.B, 700, np.int32)}, {"top_k": np.full(ci.B, 5000, np.int32)},
               {"top_p": np.ones(ci.B, np.float32)},
               {"top_k": np.full(ci.B, 700, np.int32), "top_p": np.ones(ci.B, np.float32)}):
        got = oracle.verify_chain_filtered(ci.target, ci.draft, ci.draft_tokens, ci.uniforms, ci.temperature,
                                           "bf16", **kw)
        assert np.array_equal(got.out_tokens, ref.out_tokens), kw
        assert np.array_equal(got.num_accepted, ref.num_accepted), kw
        assert np.isinf(got.cut_margin).all()


def library_filtered_probs(row, k, p, T):
    """top-k (torch.topk's k-th value, ties kept), then top-p by torch sort and
    cumsum over what top-k kept (rows without ties), then the softmax."""
    x = torch.as_tensor(np.asarray(row, np.float64))
    keep = torch.ones_like(x, dtype=torch.bool)
    if k is not None:
        thr = torch.topk(x, min(k, x.numel())).values[-1]
        keep = x >= thr
    if p is not None and p < 1.0:
        srt = torch.sort(x[keep], descending=True).values
        cum = torch.cumsum(torch.softmax(srt / T, 0), 0)
        keep = keep & (x >= srt[int(torch.nonzero(cum >= p)[0])])
    y = torch.where(keep, x / T, torch.tensor(-np.inf, dtype=torch.float64))
    return torch.softmax(y, 0).numpy()


def decider(tgt, drf, k, p, T):
    def decide(tokens, u):
        res = oracle.verify_chain_filtered(tgt[None].astype(np.float32), drf[None].astype(np.float32),
                                           np.asarray([tokens], np.int32), np.asarray([u], np.float32),
                                           np.array([T], np.float32), "f32",
                                           top_k=None if k is None else np.array([k], np.int32),
                                           top_p=None if p is None else np.array([p], np.float32))
        n = int(res.num_accepted[0])
        return [int(t) for t in res.out_tokens[0, :n + 1]], n
    return decide


@pytest.mark.parametrize("seed,V,G,k,p,T", [
    (16430, 6, 2, None, 0.7, 0.9),      # top-p alone
    (16431, 5, 1, None, 0.4, 1.2),
    (16432, 7, 2, 6, 0.85, 0.7),        # a large k (6 of 7), then top-p
    (16433, 6, 2, 5, None, 1.0),        # top-k alone, k close to V
])
def test_emitted_tokens_follow_the_filtered_target(seed, V, G, k, p, T):
    rng = np.random.default_rng(seed)
    tgt = np.round(rng.standard_normal((G + 1, V)) * 1.5, 2).astype(np.float32)
    drf = (tgt[:G] + np.round(rng.standard_normal((G, V)), 2)).astype(np.float32)
    pf = None if p is None else float(np.float32(p))
    P = [library_filtered_probs(tgt[i], k, pf, T) for i in range(G + 1)]
    Q = [library_filtered_probs(drf[i], k, pf, T) for i in range(G)]
    law = enumerate_round(P, Q, decider(tgt, drf, k, p, T))
    assert abs(sum(law.values()) - 1.0) < 1e-12
    reach, cond = slot_marginals(law, V, G + 1)
    for s in range(G + 1):
        if reach[s] > 1e-12:
            np.testing.assert_allclose(cond[s], P[s], atol=1e-12)
    assert any((P[s] > 0).sum() < V for s in range(G + 1))      # something was cut


def test_planted_mistake_unfiltered_draft_rows_are_biased(monkeypatch):
    """Drafts drawn from the filtered q', and an oracle planted to cut only
    the target rows (its accept ratio and residual use the unfiltered q): the
    emitted law is no longer p'.  The rule must be the same on both sides."""
    seed, V, G, p, T = 16440, 6, 1, 0.6, 1.0
    rng = np.random.default_rng(seed)
    tgt = np.round(rng.standard_normal((G + 1, V)) * 1.5, 2).astype(np.float32)
    drf = (tgt[:G] + np.round(rng.standard_normal((G, V)), 2)).astype(np.float32)
    pf = float(np.float32(p))
    P = [library_filtered_probs(tgt[i], None, pf, T) for i in range(G + 1)]
    Q = [library_filtered_probs(drf[i], None, pf, T) for i in range(G)]
    real = so.topp_cut
    calls = {"n": 0}

    def target_only(row, pp, TT):
        # the request's target rows are cut first, then its draft rows
        calls["n"] += 1
        return real(row, pp, TT) if calls["n"] <= G + 1 else (-np.inf, np.inf)

    inner = decider(tgt, drf, None, p, T)

    def planted(tokens, u):
        calls["n"] = 0
        return inner(tokens, u)

    assert any((Q[i] > 0).sum() < V for i in range(G))     # the draft rows are cut
    Qfull = [library_filtered_probs(drf[i], None, None, T) for i in range(G)]

    def law_of(Qdraws):
        return lambda tup: float(np.prod([Qdraws[i][tup[i]] for i in range(G)]))

    # the enumeration places its uniforms by the planted verifier's own rule
    # (unfiltered draft rows) and weighs the draft tuples by the filtered law
    monkeypatch.setattr(so, "topp_cut", target_only)
    _, cond = slot_marginals(enumerate_round(P, Qfull, planted, draft_law=law_of(Q)), V, G + 1)
    assert np.abs(cond[0] - P[0]).sum() > 1e-3
    monkeypatch.setattr(so, "topp_cut", real)
    _, cond = slot_marginals(enumerate_round(P, Q, inner), V, G + 1)
    np.testing.assert_allclose(cond[0], P[0], atol=1e-12)


def test_invalid_filters_and_greedy_requests():
    ci = synth.chain_inputs(16450, B=8, gamma=2, V=300, dtype="f32", family="gauss",
                            draft_sigma=0.5, temperature=1.0)
    T = ci.temperature.copy()
    T[7] = 0.0
    k = np.array([0, -3, 5, 5, 5, 5, 5, 0], np.int32)
    p = np.array([0.9, 0.9, 0.0, 1.5, np.nan, -0.1, 0.9, 0.0], np.float32)
    got = oracle.verify_chain_filtered(ci.target, ci.draft, ci.draft_tokens, ci.uniforms, T, "f32",
                                       top_k=k, top_p=p)
    assert (got.num_accepted[:6] == -1).all() and (got.out_tokens[:6] == -1).all()
    assert got.num_accepted[6] >= 0 and got.num_accepted[7] >= 0
    greedy = oracle.verify_chain(ci.target, ci.draft, ci.draft_tokens, ci.uniforms, T, "f32", requests=[7])
    assert np.array_equal(got.out_tokens[7], greedy.out_tokens[7])


def test_cut_margin_is_reported():
    ci = synth.chain_inputs(16460, B=6, gamma=2, V=2000, dtype="bf16", family="peaked",
                            draft_sigma=0.5, temperature=1.0)
    got = oracle.verify_chain_filtered(ci.target, ci.draft, ci.draft_tokens, ci.uniforms, ci.temperature, "bf16",
                                       top_p=np.full(ci.B, 0.9, np.float32))
    assert np.isfinite(got.cut_margin).all() and (got.cut_margin >= 0).all()
