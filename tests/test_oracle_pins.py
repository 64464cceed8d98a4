"""Pins of the fp64 oracle's chain verification against what the pages fix.

Worked examples with printed values, closed forms, the lossless theorem by
exact enumeration, Monte-Carlo checks and planted mistakes that the
enumeration must catch.  CPU only.
"""
import json
import math
import os

import numpy as np
import pytest

import oracle
from oracle import specverify_oracle as so
import synth
from enum_tools import (enumerate_round, slot_marginals, expected_emitted,
                        total_variation, breakpoints_accept)


def load(golden_dir, name):
    with open(os.path.join(golden_dir, name)) as f:
        return json.load(f)


def rows_from_probs(p):
    """logits whose T=1 softmax is p (log p; zero probabilities -> -inf)."""
    p = np.asarray(p, dtype=np.float64)
    with np.errstate(divide="ignore"):
        return np.log(p)


def oracle_decider(P, Q, T=1.0):
    """Black-box verifier over fixed probability rows."""
    def decide(tokens, u):
        emitted, n, _ = oracle.chain_decide_request(P, Q, None, np.asarray(tokens), u, T)
        return emitted, n
    return decide


def f32_chain(p_rows, q_rows, tokens, u):
    """Single-request float32 verify_chain call from probability rows."""
    tgt = np.asarray([rows_from_probs(p) for p in p_rows], dtype=np.float32)[None]
    drf = np.asarray([rows_from_probs(q) for q in q_rows], dtype=np.float32)[None]
    toks = np.asarray(tokens, dtype=np.int32)[None]
    uu = np.asarray(u, dtype=np.float32)[None]
    return oracle.verify_chain(tgt, drf, toks, uu, np.ones(1, np.float32), "f32")


# ---------------------------------------------------------------------------
# worked examples
# ---------------------------------------------------------------------------
def test_close_reading_worked_round(golden_dir):
    g = load(golden_dir, "close_reading_worked_round.json")
    p, q = np.array(g["p"]), np.array(g["q"])
    K = g["K"]
    P = [oracle.softmax_t(rows_from_probs(p), 1.0)] * (K + 1)
    Q = [oracle.softmax_t(rows_from_probs(q), 1.0)] * K
    np.testing.assert_allclose(P[0], p, rtol=0, atol=1e-15)
    # alpha, beta, residual
    pr = oracle.probs_debug(np.asarray([[rows_from_probs(p)] * (K + 1)], np.float32),
                            np.asarray([[rows_from_probs(q)] * K], np.float32),
                            np.asarray([g["drafts"]], np.int32), np.ones(1, np.float32), "f32")
    assert abs(pr.residual_mass[0, 0] - g["beta"]) < 1e-7       # float32 logits
    assert abs(1.0 - pr.residual_mass[0, 0] - g["alpha"]) < 1e-7
    w = so.residual_weights(P[0], Q[0])
    np.testing.assert_allclose(w / w.sum(), g["residual"], atol=1e-14)
    for i, x in enumerate(g["drafts"]):
        assert abs(oracle.accept_threshold(P[i][x], Q[i][x]) - g["accept_probability"][str(i + 1)]) < 1e-14
    # the traced round: r1 = 0.35 accepts A, B is accepted outright, r3 = 0.80 rejects
    # A; the residual draw lands on B for u_final < 0.75 and on C above it.
    for u_final, third in ((0.10, 1), (0.7499, 1), (0.7501, 2), (0.99, 2)):
        u = np.array([g["r"]["1"], 0.5, g["r"]["3"], u_final])
        emitted, n, dec = oracle.chain_decide_request(P, Q, None, np.array(g["drafts"]), u, 1.0)
        assert emitted == [0, 1, third] and n == 2
        assert [d.kind for d in dec] == ["accept", "accept", "accept", "draw"]
    # same trace through the batch entry point on float32 logits
    res = f32_chain([p] * 4, [q] * 3, g["drafts"], [0.35, 0.5, 0.80, 0.3])
    assert res.out_tokens[0].tolist() == g["emitted_when_residual_draw_is_B"] + [-1]
    assert res.num_accepted[0] == 2


def test_close_reading_exercise2(golden_dir):
    g = load(golden_dir, "close_reading_exercise2.json")
    p, q = np.array(g["p"]), np.array(g["q"])
    P = [oracle.softmax_t(rows_from_probs(p), 1.0)] * 4
    Q = [oracle.softmax_t(rows_from_probs(q), 1.0)] * 3
    assert abs(oracle.accept_threshold(P[0][0], Q[0][0]) - g["accept_probability_A"]) < 1e-14
    w = so.residual_weights(P[0], Q[0])
    np.testing.assert_allclose(w / w.sum(), g["residual"], atol=1e-14)
    assert abs(w.sum() - g["beta"]) < 1e-14
    for u3 in (0.67, 0.8, 0.999):
        for uf in (0.0, 0.4, 0.99):
            emitted, n, _ = oracle.chain_decide_request(
                P, Q, None, np.array(g["drafts"]), np.array([g["r1"], 0.9, u3, uf]), 1.0)
            assert emitted == g["emitted_if_r3_above_threshold"] and n == 2
    law = enumerate_round(P, Q, oracle_decider(P, Q))
    assert abs(expected_emitted(law) - g["expected_tokens_per_round"]) < 1e-12


def test_lecture_exercise3_output_equals_p(golden_dir):
    g = load(golden_dir, "lecture17_exercises.json")["exercise3"]
    p, q = np.array(g["p"]), np.array(g["q"])
    P = [oracle.softmax_t(rows_from_probs(p), 1.0)] * 2
    Q = [oracle.softmax_t(rows_from_probs(q), 1.0)]
    w = so.residual_weights(P[0], Q[0])
    np.testing.assert_allclose(w / w.sum(), g["residual"], atol=1e-15)
    assert abs(1.0 - w.sum() - g["alpha"]) < 1e-15
    law = enumerate_round(P, Q, oracle_decider(P, Q))
    _, cond = slot_marginals(law, 2, 1)
    np.testing.assert_allclose(cond[0], g["output"], atol=1e-15)


def test_lecture_exercise3_greedy_rule_is_biased(golden_dir, monkeypatch):
    """Planted mistake: the greedy rule under sampling (accept iff the draft is
    argmax p, otherwise sample from p) must reproduce the page's biased law."""
    g = load(golden_dir, "lecture17_exercises.json")["exercise3"]
    p, q = np.array(g["p"]), np.array(g["q"])
    P = [oracle.softmax_t(rows_from_probs(p), 1.0)] * 2
    Q = [oracle.softmax_t(rows_from_probs(q), 1.0)]
    pmax = P[0].max()
    greedy_rule = lambda px, qx: 1.0 if px == pmax else 0.0
    from_p = lambda pp, qq: np.asarray(pp)
    monkeypatch.setattr(so, "accept_threshold", greedy_rule)
    monkeypatch.setattr(so, "residual_weights", from_p)
    law = enumerate_round(P, Q, oracle_decider(P, Q), accept_fn=greedy_rule, residual_fn=from_p)
    _, cond = slot_marginals(law, 2, 1)
    np.testing.assert_allclose(cond[0], g["greedy_rule_under_sampling_output"], atol=1e-15)


def test_lecture_exercise7_deterministic_top1(golden_dir):
    """A draft that always proposes token 0 (not sampled from q) gives the
    page's biased law through the unmodified verifier."""
    g = load(golden_dir, "lecture17_exercises.json")["exercise7"]
    p, q = np.array(g["p"]), np.array(g["q"])
    P = [oracle.softmax_t(rows_from_probs(p), 1.0)] * 2
    Q = [oracle.softmax_t(rows_from_probs(q), 1.0)]
    law = enumerate_round(P, Q, oracle_decider(P, Q),
                          draft_law=lambda tup: 1.0 if tup == (0,) else 0.0)
    _, cond = slot_marginals(law, 2, 1)
    np.testing.assert_allclose(cond[0], g["deterministic_top1_output"], atol=1e-15)


# ---------------------------------------------------------------------------
# expected tokens per round (closed form and printed values)
# ---------------------------------------------------------------------------
def test_expected_tokens_printed_values(golden_dir):
    g = load(golden_dir, "expected_tokens_printed.json")
    for case in g["cases"]:
        a, gam = case["alpha"], case["gamma"]
        pair = g["pairs_with_exact_alpha"][repr(a) if repr(a) in g["pairs_with_exact_alpha"] else str(a)]
        p, q = np.array(pair["p"]), np.array(pair["q"])
        assert abs(np.minimum(p, q).sum() - a) < 1e-15
        if len(p) ** gam > 5000:
            continue  # covered by the closed-form Monte-Carlo test below
        P = [oracle.softmax_t(rows_from_probs(p), 1.0)] * (gam + 1)
        Q = [oracle.softmax_t(rows_from_probs(q), 1.0)] * gam
        e = expected_emitted(enumerate_round(P, Q, oracle_decider(P, Q)))
        closed = (1.0 - a ** (gam + 1)) / (1.0 - a)
        assert abs(e - closed) < 1e-12, (case, e, closed)
        assert round(e, case["decimals"]) == pytest.approx(case["printed"], abs=10 ** -case["decimals"] / 2 + 1e-12), case


def test_expected_tokens_monte_carlo_replicated_pair(golden_dir):
    """Seeded Monte-Carlo with one (p, q) pair at every position: mean emitted
    tokens within 4 standard errors of (1 - alpha^(gamma+1)) / (1 - alpha)."""
    g = load(golden_dir, "expected_tokens_printed.json")
    for a_key, gam in (("0.8", 4), ("0.9", 6), ("0.5", 4), ("0.75", 4)):
        pair = g["pairs_with_exact_alpha"][a_key]
        p, q = np.array(pair["p"]), np.array(pair["q"])
        a = float(np.minimum(p, q).sum())
        ci = synth.replicated_pair_chain(synth.SEED_BASE + 101, rows_from_probs(p),
                                         rows_from_probs(q), B=20000, gamma=gam)
        res = oracle.verify_chain(ci.target, ci.draft, ci.draft_tokens, ci.uniforms,
                                  ci.temperature, "f32")
        n_emit = res.num_accepted.astype(np.float64) + 1.0
        closed = (1.0 - a ** (gam + 1)) / (1.0 - a)
        se = n_emit.std(ddof=1) / math.sqrt(len(n_emit))
        assert abs(n_emit.mean() - closed) < 4 * se, (a_key, n_emit.mean(), closed, se)


# ---------------------------------------------------------------------------
# lossless theorem by exact enumeration
# ---------------------------------------------------------------------------
def random_rows(rng, n, V, zero_frac=0.0):
    rows = []
    for _ in range(n):
        x = rng.dirichlet(np.ones(V))
        if zero_frac:
            x[rng.random(V) < zero_frac] = 0.0
            if x.sum() == 0:
                x[0] = 1.0
            x = x / x.sum()
        rows.append(x)
    return rows


@pytest.mark.parametrize("gamma", [0, 1, 2, 3, 4])
def test_single_round_slot_marginals_equal_target(gamma):
    rng = np.random.default_rng(7 + gamma)
    V = 5
    P = random_rows(rng, gamma + 1, V)
    Q = random_rows(rng, gamma, V)
    law = enumerate_round(P, Q, oracle_decider(P, Q))
    assert abs(sum(law.values()) - 1.0) < 1e-14
    reach, cond = slot_marginals(law, V, gamma + 1)
    for s in range(gamma + 1):
        np.testing.assert_allclose(cond[s], P[s], atol=1e-14)
        alpha_prod = np.prod([np.minimum(P[i], Q[i]).sum() for i in range(s)])
        assert abs(reach[s] - alpha_prod) < 1e-14


def test_single_round_with_zero_probabilities():
    """Masked tokens (probability 0 in p or q) keep the law exact."""
    rng = np.random.default_rng(99)
    V, gamma = 5, 3
    P = random_rows(rng, gamma + 1, V, zero_frac=0.3)
    Q = random_rows(rng, gamma, V, zero_frac=0.3)
    law = enumerate_round(P, Q, oracle_decider(P, Q))
    _, cond = slot_marginals(law, V, gamma + 1)
    for s in range(gamma + 1):
        np.testing.assert_allclose(cond[s], P[s], atol=1e-14)


class ToyLM:
    """Five-token toy language model whose next-token law depends on the last
    two tokens, with a noisy draft q = softmax(log p + noise) -- the setting of
    the lecture 17 exact-enumeration experiment (section 2.3)."""

    def __init__(self, seed, V=5, noise=1.0):
        rng = np.random.default_rng(seed)
        self.V = V
        self.p = rng.dirichlet(np.ones(V), size=(V, V))
        z = np.log(self.p) + rng.standard_normal((V, V, V)) * noise
        z -= z.max(axis=-1, keepdims=True)
        self.q = np.exp(z) / np.exp(z).sum(-1, keepdims=True)

    def target_law(self, prefix, L):
        law = {(): 1.0}
        for _ in range(L):
            nxt = {}
            for seq, pr in law.items():
                ctx = (tuple(prefix) + seq)[-2:]
                for x in range(self.V):
                    nxt[seq + (x,)] = pr * self.p[ctx][x]
            law = nxt
        return law


def speculative_law(lm, prefix, L, gamma, decide_factory):
    """Exact law of the first L emitted tokens under repeated rounds."""
    import itertools
    done = {}
    frontier = {(): 1.0}
    while frontier:
        new_frontier = {}
        for seq, pr in frontier.items():
            ctx = tuple(prefix) + seq
            for tup in itertools.product(range(lm.V), repeat=gamma):
                c = list(ctx)
                P, Q = [], []
                w = 1.0
                for x in tup:
                    P.append(lm.p[tuple(c[-2:])])
                    Q.append(lm.q[tuple(c[-2:])])
                    w *= Q[-1][x]
                    c.append(x)
                P.append(lm.p[tuple(c[-2:])])
                if w == 0.0:
                    continue
                sub = enumerate_round(P, Q, decide_factory(P, Q),
                                      draft_law=lambda t, tup=tup, w=w: w if t == tup else 0.0)
                for em, pe in sub.items():
                    s2 = seq + em
                    if len(s2) >= L:
                        done[s2[:L]] = done.get(s2[:L], 0.0) + pr * pe
                    else:
                        new_frontier[s2] = new_frontier.get(s2, 0.0) + pr * pe
        frontier = new_frontier
    return done


@pytest.mark.parametrize("gamma,L", [(1, 4), (2, 4), (3, 3)])
def test_multi_round_sequence_law_exact(gamma, L):
    lm = ToyLM(seed=2024)
    prefix = (0, 1)
    spec = speculative_law(lm, prefix, L, gamma, lambda P, Q: oracle_decider(P, Q))
    ref = lm.target_law(prefix, L)
    assert len(ref) == lm.V ** L
    assert total_variation(spec, ref) < 1e-14


# ---------------------------------------------------------------------------
# planted mistakes must be caught by the enumeration
# ---------------------------------------------------------------------------
WRONG_VARIANTS = {
    "swapped_ratio": ("accept_threshold", lambda px, qx: 1.0 if px <= qx else qx / px),
    "always_accept": ("accept_threshold", lambda px, qx: 1.0),
    "resample_from_p": ("residual_weights", lambda p, q: np.asarray(p)),
    "resample_from_q": ("residual_weights", lambda p, q: np.asarray(q)),
    "no_clipping": ("residual_weights", lambda p, q: np.abs(p - q)),
}


@pytest.mark.parametrize("variant", sorted(WRONG_VARIANTS))
def test_planted_mistakes_are_detected(variant, monkeypatch):
    name, fn = WRONG_VARIANTS[variant]
    monkeypatch.setattr(so, name, fn)
    lm = ToyLM(seed=2024)
    spec = speculative_law(lm, (0, 1), 3, 2, lambda P, Q: oracle_decider(P, Q))
    ref = lm.target_law((0, 1), 3)
    assert total_variation(spec, ref) > 1e-3, variant


def test_planted_off_by_one_draw_is_detected(monkeypatch):
    real = so.inverse_cdf_draw

    def shifted(w, u):
        k, m = real(w, u)
        return (k + 1) % len(w), m
    monkeypatch.setattr(so, "inverse_cdf_draw", shifted)
    rng = np.random.default_rng(5)
    P = random_rows(rng, 3, 5)
    Q = random_rows(rng, 2, 5)
    law = enumerate_round(P, Q, oracle_decider(P, Q))
    _, cond = slot_marginals(law, 5, 3)
    assert np.abs(cond[0] - P[0]).max() > 1e-3


# ---------------------------------------------------------------------------
# identities and special cases
# ---------------------------------------------------------------------------
def test_residual_mass_identity_bf16():
    """sum_k max(0, p-q) = 1 - sum_k min(p, q) (close-reading notes 5.1)."""
    ci = synth.chain_inputs(11, B=6, gamma=3, V=3000, dtype="bf16", family="peaked",
                            draft_sigma=(0.3, 2.0), temperature=0.7)
    pr = oracle.probs_debug(ci.target, ci.draft, ci.draft_tokens, ci.temperature, "bf16")
    for b in range(ci.B):
        t = float(ci.temperature[b])
        tgt = so.logits_to_f64(ci.target[b], "bf16")
        drf = so.logits_to_f64(ci.draft[b], "bf16")
        for i in range(ci.gamma):
            zp = tgt[i] / t
            zq = drf[i] / t
            p = np.exp(zp - zp.max()); p /= p.sum()
            q = np.exp(zq - zq.max()); q /= q.sum()
            assert abs(pr.residual_mass[b, i] + np.minimum(p, q).sum() - 1.0) < 1e-14
            x = ci.draft_tokens[b, i]
            assert abs(pr.p_at_draft[b, i] - p[x]) <= 1e-13 * p[x]
            assert abs(pr.q_at_draft[b, i] - q[x]) <= 1e-13 * q[x]
        for i in range(ci.gamma + 1):
            z = tgt[i] / t
            assert abs(pr.target_lse[b, i] - np.log(np.exp(z).sum())) < 1e-12


def test_gamma0_draw_law_on_a_uniform_grid():
    """With gamma = 0 the round is one inverse-CDF draw from p_1: on a fine grid
    of uniforms, token frequencies equal p up to the grid spacing."""
    rng = np.random.default_rng(3)
    V = 7
    logits = rng.standard_normal(V)
    p = np.exp(logits - logits.max()); p /= p.sum()
    n = 200000
    counts = np.zeros(V)
    P = [oracle.softmax_t(logits, 1.0)]
    for j in range(n):
        u = np.array([(j + 0.5) / n])
        emitted, nacc, _ = oracle.chain_decide_request(P, [], None, np.zeros(0, np.int64), u, 1.0)
        assert nacc == 0
        counts[emitted[0]] += 1
    np.testing.assert_allclose(counts / n, p, atol=1.5 / n)


def test_draw_never_picks_zero_weight():
    w = np.array([0.0, 0.0, 0.3, 0.0, 0.7, 0.0])
    assert oracle.inverse_cdf_draw(w, 0.0)[0] == 2
    assert oracle.inverse_cdf_draw(w, 0.2999999)[0] == 2
    assert oracle.inverse_cdf_draw(w, 0.3)[0] == 4      # C_k > u*W is strict
    assert oracle.inverse_cdf_draw(w, 0.9999999)[0] == 4
    for u in np.linspace(0, 1, 1001, endpoint=False):
        assert w[oracle.inverse_cdf_draw(w, u)[0]] > 0


def test_greedy_chain_equals_argmax_chain():
    ci = synth.chain_inputs(21, B=8, gamma=5, V=4000, dtype="bf16", family="peaked",
                            temperature=0.0)
    tgt = np.stack([so.logits_to_f64(ci.target[b], "bf16") for b in range(ci.B)])
    amax = np.argmax(tgt, axis=-1)                 # lowest index on ties
    toks = ci.draft_tokens.copy()
    for b in range(ci.B):
        k = b % (ci.gamma + 1)                     # first k drafts match the argmax chain
        toks[b, :k] = amax[b, :k]
        if k < ci.gamma:
            toks[b, k] = (amax[b, k] + 1) % ci.V
    res = oracle.verify_chain(ci.target, None, toks, ci.uniforms, ci.temperature, "bf16")
    for b in range(ci.B):
        k = b % (ci.gamma + 1)
        assert res.num_accepted[b] == k
        assert res.out_tokens[b, :k + 1].tolist() == amax[b, :k + 1].tolist()
        assert (res.out_tokens[b, k + 1:] == -1).all()


def test_greedy_ties_take_lowest_index():
    V = 16
    row = np.full(V, -1.0, dtype=np.float32)
    row[[5, 9, 12]] = 3.0
    tgt = np.stack([row, row])[None]
    res = oracle.verify_chain(tgt, None, np.array([[9]], np.int32), np.zeros((1, 2), np.float32),
                              np.zeros(1, np.float32), "f32")
    assert res.num_accepted[0] == 0 and res.out_tokens[0].tolist() == [5, -1]
    res = oracle.verify_chain(tgt, None, np.array([[5]], np.int32), np.zeros((1, 2), np.float32),
                              np.zeros(1, np.float32), "f32")
    assert res.num_accepted[0] == 1 and res.out_tokens[0].tolist() == [5, 5]


def test_invalid_requests_get_sentinels():
    ci = synth.chain_inputs(31, B=8, gamma=3, V=50, dtype="f32", family="gauss", temperature=1.0)
    toks = ci.draft_tokens.copy()
    u = ci.uniforms.copy()
    T = ci.temperature.copy()
    toks[0, 1] = 50                 # token out of range
    toks[1, 0] = -1
    T[2] = -0.5                     # negative temperature
    T[3] = np.nan
    u[4, 3] = 1.0                   # uniform outside [0, 1)
    u[5, 0] = np.nan
    T[6] = 0.0                      # greedy: uniforms are not read
    u[6, :] = 7.0
    res = oracle.verify_chain(ci.target, ci.draft, toks, u, T, "f32")
    for b in range(6):
        assert res.num_accepted[b] == -1 and (res.out_tokens[b] == -1).all()
    assert res.num_accepted[6] >= 0 and res.num_accepted[7] >= 0


def test_toy_config_monte_carlo_first_slot():
    """Seeded Monte-Carlo on the V=5 toy batch (4096 independent rounds): the
    count of each first emitted token is within 4.5 standard deviations of
    sum_b p_b1(token) (lecture 17 notes section 2.3: Monte-Carlo check)."""
    ci = synth.toy_chain()
    res = oracle.verify_chain(ci.target, ci.draft, ci.draft_tokens, ci.uniforms,
                              ci.temperature, "f32")
    tgt = np.stack([so.logits_to_f64(ci.target[b], "f32") for b in range(ci.B)])
    e = np.exp(tgt[:, 0, :] - tgt[:, 0, :].max(-1, keepdims=True))
    p1 = e / e.sum(-1, keepdims=True)
    for k in range(ci.V):
        obs = (res.out_tokens[:, 0] == k).sum()
        exp = p1[:, k].sum()
        sd = math.sqrt((p1[:, k] * (1 - p1[:, k])).sum())
        assert abs(obs - exp) < 4.5 * sd, (k, obs, exp, sd)
