"""Pins of the oracle's ragged chain verification and its acceptance output
(CPU only).

- E[N] per draft length: with one (p, q) pair at every position, requests of
  length g emit (1 - alpha^(g+1)) / (1 - alpha) tokens on average (the
  closed form the pages print values of), for every g in one ragged batch.
- The acceptance output: over x ~ q, tau(x) averages to sum min(p, q), i.e.
  1 minus the residual mass (close-reading notes section 5.1), by exact
  enumeration and by the ragged call's own output.
- A request never reads past its length: garbage there changes nothing.
- A full-length ragged call agrees with the fixed-length call.
"""
import json
import math
import os

import numpy as np
import pytest

import oracle
from oracle import specverify_oracle as so
import synth


def load(golden_dir, name):
    with open(os.path.join(golden_dir, name)) as f:
        return json.load(f)


def rows_from_probs(p):
    return np.log(np.maximum(np.asarray(p, dtype=np.float64), 1e-300)).astype(np.float32)


def test_expected_tokens_per_length_in_one_ragged_batch(golden_dir):
    g = load(golden_dir, "expected_tokens_printed.json")
    pair = g["pairs_with_exact_alpha"]["0.8"]
    p, q = np.array(pair["p"]), np.array(pair["q"])
    a = float(np.minimum(p, q).sum())
    G = 6
    B = 21000
    ci = synth.replicated_pair_chain(synth.SEED_BASE + 111, rows_from_probs(p), rows_from_probs(q),
                                     B=B, gamma=G)
    gam = (np.arange(B) % (G + 1)).astype(np.int32)
    res = oracle.verify_chain_ragged(ci.target, ci.draft, ci.draft_tokens, ci.uniforms, ci.temperature,
                                     gam, "f32")
    assert (res.num_accepted >= 0).all() and (res.num_accepted <= gam).all()
    for length in range(G + 1):
        sel = gam == length
        n_emit = res.num_accepted[sel].astype(np.float64) + 1.0
        closed = (1.0 - a ** (length + 1)) / (1.0 - a)
        se = max(n_emit.std(ddof=1) / math.sqrt(sel.sum()), 1e-12)
        assert abs(n_emit.mean() - closed) < 4 * se + 1e-12, (length, n_emit.mean(), closed, se)
        # padding after the n + 1 emitted tokens
        for b in np.flatnonzero(sel)[:50]:
            n = res.num_accepted[b]
            assert (res.out_tokens[b, n + 1:] == -1).all() and (res.out_tokens[b, :n + 1] >= 0).all()


def test_tau_averages_to_the_acceptance_rate():
    rng = np.random.default_rng(15500)
    for _ in range(20):
        p = rng.dirichlet(np.full(7, 0.7))
        q = rng.dirichlet(np.full(7, 0.7))
        mean_tau = sum(q[x] * oracle.accept_threshold(p[x], q[x]) for x in range(7))
        assert abs(mean_tau - np.minimum(p, q).sum()) < 1e-15
        assert abs(mean_tau - (1.0 - so.residual_weights(p, q).sum())) < 1e-15


def test_accept_prob_output_estimates_alpha(golden_dir):
    g = load(golden_dir, "expected_tokens_printed.json")
    pair = g["pairs_with_exact_alpha"]["0.75"]
    p, q = np.array(pair["p"]), np.array(pair["q"])
    a = float(np.minimum(p, q).sum())
    B, G = 20000, 3
    ci = synth.replicated_pair_chain(synth.SEED_BASE + 112, rows_from_probs(p), rows_from_probs(q),
                                     B=B, gamma=G)
    res = oracle.verify_chain_ragged(ci.target, ci.draft, ci.draft_tokens, ci.uniforms, ci.temperature,
                                     np.full(B, G, np.int32), "f32")
    # the first test is always taken, with x ~ q: its tau is an unbiased estimate of alpha
    t0 = res.accept_prob[:, 0]
    se = t0.std(ddof=1) / math.sqrt(B)
    assert abs(t0.mean() - a) < 4 * se
    # a test is taken exactly up to the first rejection
    for b in range(200):
        n = res.num_accepted[b]
        taken = res.accept_prob[b] >= 0
        assert taken.sum() == min(n + 1, G)


def test_nothing_past_the_length_is_read():
    ci = synth.chain_inputs(15510, 24, 5, 300, dtype="f32", family="gauss", draft_sigma=(0.2, 1.5),
                            temperature=0.9, greedy_odd=True, name="ragged")
    gam = np.array([b % 6 for b in range(24)], np.int32)
    ref = oracle.verify_chain_ragged(ci.target, ci.draft, ci.draft_tokens, ci.uniforms, ci.temperature,
                                     gam, "f32")
    tgt, drf, tok, u = ci.target.copy(), ci.draft.copy(), ci.draft_tokens.copy(), ci.uniforms.copy()
    for b in range(24):
        g = gam[b]
        tgt[b, g + 1:] = np.nan
        drf[b, g:] = np.nan
        tok[b, g:] = -7
        u[b, g + 1:] = 5.0
    got = oracle.verify_chain_ragged(tgt, drf, tok, u, ci.temperature, gam, "f32")
    assert np.array_equal(got.out_tokens, ref.out_tokens)
    assert np.array_equal(got.num_accepted, ref.num_accepted)
    assert np.array_equal(got.accept_prob, ref.accept_prob)
    assert (ref.num_accepted >= 0).all()


def test_full_length_matches_the_fixed_call_and_bad_lengths_are_invalid():
    ci = synth.chain_inputs(15520, 16, 4, 200, dtype="bf16", family="peaked", draft_sigma=(0.3, 2.0),
                            temperature=0.7, greedy_odd=True, name="ragged-full")
    fixed = oracle.verify_chain(ci.target, ci.draft, ci.draft_tokens, ci.uniforms, ci.temperature, "bf16")
    gam = np.full(16, 4, np.int32)
    gam[3], gam[8] = -1, 5
    rag = oracle.verify_chain_ragged(ci.target, ci.draft, ci.draft_tokens, ci.uniforms, ci.temperature,
                                     gam, "bf16")
    ok = np.ones(16, bool)
    ok[[3, 8]] = False
    assert np.array_equal(rag.out_tokens[ok], fixed.out_tokens[ok])
    assert np.array_equal(rag.num_accepted[ok], fixed.num_accepted[ok])
    assert (rag.num_accepted[~ok] == -1).all() and (rag.out_tokens[~ok] == -1).all()
    for b in np.flatnonzero(ok):
        taus = [d.threshold for d in fixed.decisions[b] if d.kind == "accept"]
        assert np.allclose(rag.accept_prob[b, :len(taus)], taus)
