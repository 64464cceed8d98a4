"""Pins of the fp64 oracle's token-tree verification (CPU only).

Lecture 17 notes: exercise 5 (depth-first order, parents, depths), section
4.5 / exercise 6 (naive sampling accepts with probability sum of the
children's target probabilities, and is unbiased), section 4.4 (greedy tree
verification reproduces the target's own greedy output).
"""
import json
import os

import numpy as np

import oracle
from oracle import specverify_oracle as so
import synth


def load(golden_dir, name):
    with open(os.path.join(golden_dir, name)) as f:
        return json.load(f)


def single_tree(rows, tokens, parents, u, T, max_depth, dtype="f32"):
    logits = np.asarray(rows, dtype=np.float32)[None]
    return oracle.verify_tree(logits, np.asarray([tokens], np.int32),
                              np.asarray([parents], np.int32),
                              np.asarray([u], np.float32), np.asarray([T], np.float32),
                              dtype, max_depth)


def test_exercise5_depths(golden_dir):
    g = load(golden_dir, "lecture17_exercises.json")["exercise5"]
    d = oracle.tree_node_depths(np.array(g["parents"]))
    assert d.tolist() == g["depths"]
    # ancestors of e (node 5) by walking parents
    names = g["dfs_order"]
    anc, n = [], g["parents"][5]
    while n >= 0:
        anc.append(names[n])
        n = g["parents"][n]
    assert sorted(anc) == sorted(g["ancestors_of_e"])


def test_exercise6_naive_acceptance_half(golden_dir):
    """Uniform target over 4 tokens, two children carrying tokens 1 and 2:
    naive sampling accepts a child with probability 1/2."""
    g = load(golden_dir, "lecture17_exercises.json")["exercise6"]
    V = 4
    llm = np.log(np.array(g["llm"]))
    rows = [llm, llm, llm]
    parents = [-1, 0, 0]
    tokens = [0] + g["children_tokens"]
    n = 4000
    acc = 0
    for j in range(n):
        r = single_tree(rows, tokens, parents, [(j + 0.5) / n, 0.5, 0.5], 1.0, 2)
        acc += int(r.num_accepted[0] >= 1)
    assert abs(acc / n - g["naive_acceptance"]) < 1e-12


def test_naive_sampling_is_unbiased_on_a_grid():
    """Slot 1 follows p_root and, given child j was accepted, slot 2 follows p_j."""
    rng = np.random.default_rng(12)
    V = 6
    rows = rng.standard_normal((5, V))
    parents = [-1, 0, 0, 1, 1]
    tokens = [0, 2, 4, 1, 3]
    P = [oracle.softmax_t(r, 1.0) for r in rows]
    n = 300
    slot1 = np.zeros(V)
    slot2_given_child1 = np.zeros(V)
    reach1 = 0
    for i in range(n):
        for j in range(n):
            u = [(i + 0.5) / n, (j + 0.5) / n, 0.5, 0.5, 0.5]
            r = single_tree(rows, tokens, parents, u, 1.0, 3)
            out = r.out_tokens[0]
            slot1[out[0]] += 1
            if r.out_path[0, 0] == 1:
                reach1 += 1
                slot2_given_child1[out[1]] += 1
    np.testing.assert_allclose(slot1 / n ** 2, P[0], atol=2.0 / n)
    assert abs(reach1 / n ** 2 - P[0][2]) < 2.0 / n
    np.testing.assert_allclose(slot2_given_child1 / reach1, P[1], atol=3.0 / n)


def test_greedy_tree_reproduces_target_greedy_chain():
    """A toy target whose next-token law depends on the last token: greedy tree
    verification emits exactly the target's greedy continuation, as far as the
    tree holds it, plus one token."""
    rng = np.random.default_rng(4)
    V = 5
    table = rng.standard_normal((V, V)) * 2.0
    root_tok = 3
    chain = [root_tok]
    for _ in range(6):
        chain.append(int(np.argmax(table[chain[-1]])))
    # tree: root -> (wrong, right) -> right child has (right, wrong) -> ...
    parents, tokens = [-1], [root_tok]
    cur = 0
    depth_ok = 3
    for d in range(1, depth_ok + 1):
        right = chain[d]
        wrong = (right + 1) % V
        parents.append(cur); tokens.append(wrong)          # sibling first (lower index)
        parents.append(cur); tokens.append(right)
        cur = len(tokens) - 1
    rows = [table[t] for t in tokens]
    r = single_tree(rows, tokens, parents, [0.5] * len(tokens), 0.0, 8)
    assert r.num_accepted[0] == depth_ok
    assert r.out_tokens[0, :depth_ok + 1].tolist() == chain[1:depth_ok + 2]


def test_tree_duplicate_children_take_lowest_index():
    V = 4
    rows = np.full((4, V), -5.0)
    rows[0, 2] = 5.0
    parents = [-1, 0, 0, 0]
    tokens = [0, 1, 2, 2]
    r = single_tree(rows, tokens, parents, [0.5] * 4, 0.0, 2)
    assert r.out_path[0, 0] == 2 and r.num_accepted[0] == 1


def test_tree_invalid_inputs():
    V = 4
    rows = np.zeros((4, V))
    good = dict(tokens=[0, 1, 2, 3], parents=[-1, 0, 1, 2], u=[0.5] * 4)
    assert single_tree(rows, good["tokens"], good["parents"], good["u"], 0.0, 3).num_accepted[0] >= 0
    # too deep for max_depth
    assert single_tree(rows, good["tokens"], good["parents"], good["u"], 0.0, 2).num_accepted[0] == -1
    # parent not earlier in the order
    assert single_tree(rows, good["tokens"], [-1, 0, 3, 1], good["u"], 0.0, 3).num_accepted[0] == -1
    # root with a parent
    assert single_tree(rows, good["tokens"], [0, 0, 1, 2], good["u"], 0.0, 3).num_accepted[0] == -1
    # token out of range
    assert single_tree(rows, [0, 1, 9, 3], good["parents"], good["u"], 0.0, 3).num_accepted[0] == -1
    # sampling request with a uniform outside [0, 1)
    assert single_tree(rows, good["tokens"], good["parents"], [0.5, 1.0, 0.5, 0.5], 1.0, 3).num_accepted[0] == -1


def test_generated_trees_satisfy_contract():
    ti = synth.tree_inputs(seed=77, B=6, N=64, V=500, max_depth=8, temperature=1.0)
    for b in range(ti.B):
        d = oracle.tree_node_depths(ti.parents[b])
        assert d is not None and d.max() <= 8
        for n in range(ti.N):
            kids = [j for j in range(ti.N) if ti.parents[b, j] == n]
            toks = [int(ti.node_tokens[b, j]) for j in kids]
            assert len(set(toks)) == len(toks)       # drawn without replacement
            assert len(kids) <= 4
    res = oracle.verify_tree(ti.logits, ti.node_tokens, ti.parents, ti.uniforms,
                             ti.temperature, ti.dtype, ti.max_depth)
    assert (res.num_accepted >= 0).all()
    for b in range(ti.B):
        n = res.num_accepted[b]
        path = res.out_path[b, :n]
        prev = 0
        for j in path:                               # each accepted node is a child of the previous
            assert ti.parents[b, j] == prev
            prev = j
        assert res.out_tokens[b, :n].tolist() == [int(ti.node_tokens[b, j]) for j in path]
