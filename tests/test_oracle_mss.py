"""Pins of the fp64 oracle's multi-step speculative sampling (CPU only).

Lecture 17 notes section 4.5 and exercises 6 and 7: the printed thresholds,
residuals and acceptance rates of the slides' four-token example and of
exercise 6; the bias of a deterministic top-1 draft (exercise 7's printed
output).  Theorem 4.2 (MSS emits exactly the target distribution) and theorem
4.3 (MSS rejects no more often than naive sampling) by exact enumeration over
the children's draws on V = 5, with a negative control that drops the
renormalisation of q_j.  A chain-shaped tree reduces to the chain
verification, and greedy trees to the greedy tree verification.
"""
import itertools
import json
import os

import numpy as np
import pytest

import oracle
import synth


def load(golden_dir, name):
    with open(os.path.join(golden_dir, name)) as f:
        return json.load(f)


def naive_acceptance_on_grid(llm, child_tokens, n=4000):
    """Fraction of a midpoint grid of uniforms for which naive sampling on a
    root with these children accepts one (the tree oracle of section 4.5)."""
    logits = np.log(np.maximum(np.asarray(llm, dtype=np.float64), 1e-300)).astype(np.float32)
    rows = np.stack([logits] * (1 + len(child_tokens)))[None]
    tokens = np.asarray([[0] + list(child_tokens)], np.int32)
    parents = np.asarray([[-1] + [0] * len(child_tokens)], np.int32)
    acc = 0
    for j in range(n):
        u = np.full((1, 1 + len(child_tokens)), 0.5, np.float32)
        u[0, 0] = (j + 0.5) / n
        r = oracle.verify_tree(rows, tokens, parents, u, np.asarray([1.0], np.float32), "f32", 1)
        acc += int(r.num_accepted[0] >= 1)
    return acc / n


def mss_acceptance(taus):
    rej = 1.0
    for t in taus:
        rej *= 1.0 - t
    return 1.0 - rej


def test_slide_example(golden_dir):
    g = load(golden_dir, "lecture17_mss.json")["slide_example"]
    p = np.array(g["llm"])
    taus, res = oracle.mss_thresholds(p, [(g["ssm1_token"], np.array(g["ssm1"])),
                                          (g["ssm2_token"], np.array(g["ssm2"]))])
    assert taus[0] == pytest.approx(g["first_accept"], abs=1e-15)
    assert np.allclose(res[0], g["residual_after_first"], atol=1e-15)
    assert taus[1] == pytest.approx(g["second_accept"], abs=1e-15)
    assert mss_acceptance(taus) == pytest.approx(g["mss_acceptance_this_draw"], abs=1e-15)
    assert naive_acceptance_on_grid(g["llm"], [g["ssm1_token"], g["ssm2_token"]]) == \
        pytest.approx(g["naive_acceptance_this_draw"], abs=1e-12)
    # averaged over the second draft's draws (the first draft always gives t1)
    q2 = np.array(g["ssm2"])
    mss = naive = 0.0
    for t in range(4):
        taus, _ = oracle.mss_thresholds(p, [(g["ssm1_token"], np.array(g["ssm1"])), (t, q2)])
        mss += q2[t] * mss_acceptance(taus)
        naive += q2[t] * p[sorted({g["ssm1_token"], t})].sum()
    assert mss == pytest.approx(g["mss_acceptance_averaged"], abs=1e-15)
    assert naive == pytest.approx(g["naive_acceptance_averaged"], abs=1e-15)


def test_exercise6(golden_dir):
    g = load(golden_dir, "lecture17_mss.json")["exercise6"]
    p = np.array(g["llm"])
    taus, res = oracle.mss_thresholds(p, [(g["ssm1_token"], np.array(g["ssm1"])),
                                          (g["ssm2_token"], np.array(g["ssm2"]))])
    assert taus[0] == pytest.approx(g["first_accept"], abs=1e-15)
    assert np.allclose(res[0], g["residual_after_first"], atol=1e-15)
    assert taus[1] == pytest.approx(g["second_accept"], abs=1e-15)
    assert mss_acceptance(taus) == pytest.approx(g["mss_acceptance"], abs=1e-15)
    assert naive_acceptance_on_grid(g["llm"], [g["ssm1_token"], g["ssm2_token"]]) == \
        pytest.approx(g["naive_acceptance"], abs=1e-12)
    # the same decisions through mss_node with uniforms: accepted on the whole grid
    n = 200
    for i in range(n):
        for u2 in (0.0, 0.5, 0.999):
            j, _, _ = oracle.mss_node(p, [(g["ssm1_token"], np.array(g["ssm1"])),
                                          (g["ssm2_token"], np.array(g["ssm2"]))],
                                      [(i + 0.5) / n, u2], 0.5)
            assert j == (0 if (i + 0.5) / n <= 0.5 else 1)


def test_exercise7_deterministic_top1_is_biased(golden_dir):
    g = load(golden_dir, "lecture17_exercises.json")["exercise7"]
    p, q = np.array(g["p"]), np.array(g["q"])
    # the draft always proposes argmax q: integrate mss_node over both uniforms
    n = 600
    out = np.zeros(2)
    for i in range(n):
        for k in range(n):
            _, tok, _ = oracle.mss_node(p, [(int(np.argmax(q)), q)], [(i + 0.5) / n], (k + 0.5) / n)
            out[tok] += 1.0 / (n * n)
    assert np.allclose(out, g["deterministic_top1_output"], atol=2e-3)
    # proposals drawn from q instead: exactly p
    exact = np.zeros(2)
    for x in range(2):
        taus, res = oracle.mss_thresholds(p, [(x, q)])
        exact[x] += q[x] * taus[0]
        if taus[0] < 1.0:
            exact += q[x] * (1.0 - taus[0]) * res[0]
    assert np.allclose(exact, p, atol=1e-15)


def emitted_distribution(p, props):
    """Exact law of the token emitted at a node for fixed proposals: sum over
    the first acceptance, plus the residual draw if all are rejected."""
    taus, res = oracle.mss_thresholds(p, props)
    out = np.zeros_like(p)
    alive = 1.0
    for j, t in enumerate(taus):
        out[props[j][0]] += alive * t
        alive *= 1.0 - t
    if alive > 0.0:
        last = res[-1] if res and res[-1] is not None else p
        out += alive * last
    return out, 1.0 - alive


def children_law(q, k, replacement):
    """Ordered child tuples of k draws from q with their probabilities."""
    V = len(q)
    for tup in itertools.product(range(V), repeat=k):
        if not replacement and len(set(tup)) < k:
            continue
        pr, left = 1.0, 1.0
        for x in tup:
            if q[x] == 0.0:
                pr = 0.0
                break
            pr *= q[x] / left
            if not replacement:
                left -= q[x]
        if pr > 0.0:
            yield tup, pr


def random_pair(rng, V=5, sharp=1.5):
    p = rng.dirichlet(np.full(V, sharp))
    q = rng.dirichlet(np.full(V, sharp))
    return p, q


@pytest.mark.parametrize("k", [1, 2, 3, 4])
def test_theorems_4_2_and_4_3_by_enumeration(k):
    rng = np.random.default_rng(15300 + k)
    for _ in range(12):
        p, q = random_pair(rng)
        law = np.zeros(5)
        law_iid = np.zeros(5)
        acc_mss = acc_naive = 0.0
        for tup, pr in children_law(q, k, replacement=False):
            props = oracle.mss_proposals(q, list(tup))
            dist, acc = emitted_distribution(p, props)
            law += pr * dist
            acc_mss += pr * acc
            acc_naive += pr * p[list(set(tup))].sum()
        for tup, pr in children_law(q, k, replacement=True):
            dist, _ = emitted_distribution(p, [(x, q) for x in tup])
            law_iid += pr * dist
        assert np.allclose(law, p, atol=1e-14, rtol=0)          # theorem 4.2, without replacement
        assert np.allclose(law_iid, p, atol=1e-14, rtol=0)      # and with independent drafts
        assert acc_mss >= acc_naive - 1e-15                     # theorem 4.3


def test_unrenormalised_q_is_biased():
    """Children drawn without replacement but each tested against the plain q
    (no removal and renormalisation): the emitted law moves off p."""
    rng = np.random.default_rng(15310)
    worst = 0.0
    for _ in range(12):
        p, q = random_pair(rng)
        law = np.zeros(5)
        for tup, pr in children_law(q, 3, replacement=False):
            dist, _ = emitted_distribution(p, [(x, q) for x in tup])
            law += pr * dist
        worst = max(worst, 0.5 * np.abs(law - p).sum())
    assert worst > 1e-3


def test_chain_shaped_tree_equals_chain():
    """A tree in which every node has one child is a chain: MSS at each node is
    the single-draft test, and the residual / bonus draw is the chain's."""
    B, G, V = 48, 4, 60
    ci = synth.chain_inputs(15320, B, G, V, dtype="f32", family="gauss", draft_sigma=(0.2, 1.0),
                            temperature=0.9, greedy_odd=True, name="chain-as-tree")
    ref = oracle.verify_chain(ci.target, ci.draft, ci.draft_tokens, ci.uniforms, ci.temperature, "f32")
    N = G + 1
    parents = np.tile(np.arange(-1, N - 1, dtype=np.int32), (B, 1))
    tokens = np.concatenate([np.zeros((B, 1), np.int32), ci.draft_tokens.astype(np.int32)], axis=1)
    draft = np.concatenate([ci.draft, ci.draft[:, :1]], axis=1)   # the leaf's row is never read
    acc_u = np.concatenate([np.zeros((B, 1), np.float32), ci.uniforms[:, :G]], axis=1)
    draw_u = np.repeat(ci.uniforms[:, G:G + 1], N, axis=1)
    got = oracle.verify_tree_mss(ci.target, draft, tokens, parents, acc_u, draw_u, ci.temperature,
                                 "f32", max_depth=G)
    assert np.array_equal(got.num_accepted, ref.num_accepted)
    assert np.array_equal(got.out_tokens, ref.out_tokens)
    assert (ref.num_accepted[0::2] < G).any() and (ref.num_accepted[0::2] > 0).any()


def test_greedy_trees_match_the_greedy_tree_verify():
    ti = synth.tree_inputs(seed=15330, B=12, N=30, V=500, max_depth=6, temperature=0.0,
                           family="gauss", draft_sigma=0.3)
    a = oracle.verify_tree(ti.logits, ti.node_tokens, ti.parents, ti.uniforms, ti.temperature,
                           ti.dtype, ti.max_depth)
    b = oracle.verify_tree_mss(ti.logits, ti.logits, ti.node_tokens, ti.parents, ti.uniforms,
                               ti.uniforms, ti.temperature, ti.dtype, ti.max_depth)
    assert np.array_equal(a.out_tokens, b.out_tokens)
    assert np.array_equal(a.out_path, b.out_path)
    assert np.array_equal(a.num_accepted, b.num_accepted)


def test_duplicate_children_are_skipped():
    V = 6
    rng = np.random.default_rng(15340)
    tl = rng.standard_normal((1, 4, V)).astype(np.float32)
    dl = rng.standard_normal((1, 4, V)).astype(np.float32)
    parents = np.array([[-1, 0, 0, 0]], np.int32)
    tokens = np.array([[0, 3, 3, 5]], np.int32)     # node 2 repeats node 1's token
    T = np.array([1.0], np.float32)
    p = oracle.softmax_t(tl[0, 0].astype(np.float64), 1.0)
    q = oracle.softmax_t(dl[0, 0].astype(np.float64), 1.0)
    for ua1 in (0.01, 0.5, 0.99):
        for ua3 in (0.01, 0.5, 0.99):
            acc = np.array([[0.5, ua1, 0.0, ua3]], np.float32)
            draw = np.array([[0.37, 0.5, 0.5, 0.5]], np.float32)
            r = oracle.verify_tree_mss(tl, dl, tokens, parents, acc, draw, T, "f32", 1)
            j, c, _ = oracle.mss_node(p, oracle.mss_proposals(q, [3, 5]), [ua1, ua3], 0.37)
            assert r.out_tokens[0, 0] == c
            assert r.num_accepted[0] == (1 if j >= 0 else 0)
            if j >= 0:
                assert r.out_path[0, 0] == [1, 3][j]


def test_mss_invalid_inputs():
    ti = synth.tree_inputs(seed=15350, B=6, N=12, V=100, max_depth=5, temperature=1.0,
                           family="gauss", draft_sigma=0.3)
    acc = ti.uniforms.copy()
    draw = ti.uniforms[:, ::-1].copy()
    acc[0, 0] = 7.0        # never used: still valid
    acc[1, 5] = 1.0        # a used accept uniform out of range
    draw[2, 0] = -0.1      # a draw uniform out of range
    par = ti.parents.copy()
    par[3, 4] = 9          # parent after its child
    T = ti.temperature.copy()
    T[4] = -1.0
    r = oracle.verify_tree_mss(ti.logits, ti.logits, ti.node_tokens, par, acc, draw, T,
                               ti.dtype, ti.max_depth)
    assert r.num_accepted[0] >= 0 and r.num_accepted[5] >= 0
    for b in (1, 2, 3, 4):
        assert r.num_accepted[b] == -1 and (r.out_tokens[b] == -1).all() and (r.out_path[b] == -1).all()
