"""Pins of the fp64 oracle's tree attention mask and depth positions (CPU only).

Lecture 17 notes: section 4.2 / 4.3 (the slides' merged tree of three draft
sequences and its printed mask; positions follow depth) and exercise 5
(depth-first order, depths, what node e can see).  Beyond the printed
examples: the mask equals the reflexive-transitive closure of the parent
relation computed by repeated boolean matrix products, and on depth-first
trees a node's ancestors are exactly the nodes whose preorder interval holds
it.
"""
import json
import os

import numpy as np
import pytest

import oracle
import synth


def load(golden_dir, name):
    with open(os.path.join(golden_dir, name)) as f:
        return json.load(f)


def merge_sequences(seqs):
    """Merge draft sequences into a token tree (shared prefixes stored once)
    and linearise it depth-first, children in order of first appearance.
    Returns (names in DFS order, parents, depth of each node as its index in
    a sequence)."""
    children = {(): []}
    for s in seqs:
        for k in range(len(s)):
            key, par = tuple(s[:k + 1]), tuple(s[:k])
            if key not in children:
                children[key] = []
                children[par].append(key)
    order, stack = [], list(reversed(children[()]))
    while stack:
        n = stack.pop()
        order.append(n)
        stack.extend(reversed(children[n]))
    ids = {n: i for i, n in enumerate(order)}
    parents = [ids[n[:-1]] if len(n) > 1 else -1 for n in order]
    return [n[-1] for n in order], parents, [len(n) - 1 for n in order]


def closure_mask(parents):
    """Reflexive-transitive closure of i -> parent(i) by boolean products."""
    N = len(parents)
    A = np.zeros((N, N), dtype=np.int64)
    for i, p in enumerate(parents):
        if p >= 0:
            A[i, p] = 1
    M = np.eye(N, dtype=np.int64)
    while True:
        nxt = ((M + M @ A) > 0).astype(np.int64)
        if np.array_equal(nxt, M):
            return M.astype(bool)
        M = nxt


def test_slides_tree_mask(golden_dir):
    g = load(golden_dir, "lecture17_tree_mask.json")
    names, parents, seq_depth = merge_sequences(g["sequences"])
    assert names == g["dfs_order"]
    r = oracle.tree_attention_mask(np.array([parents]), max_depth=8)
    for i, name in enumerate(names):
        seen = sorted(names[j] for j in range(len(names)) if r.mask[0, i, j])
        assert seen == sorted(g["mask_rows"][name]), name
    for name, hidden in g["hidden_although_earlier"].items():
        i = names.index(name)
        for h in hidden:
            j = names.index(h)
            assert j < i and not r.mask[0, i, j]
    assert r.depth[0].tolist() == seq_depth
    assert r.tree_depth[0] == max(seq_depth)


def test_exercise5_mask(golden_dir):
    g = load(golden_dir, "lecture17_exercises.json")["exercise5"]
    names = g["dfs_order"]
    r = oracle.tree_attention_mask(np.array([g["parents"]]), max_depth=8)
    assert r.depth[0].tolist() == g["depths"]
    e = names.index("e")
    seen = sorted(names[j] for j in range(len(names)) if r.mask[0, e, j])
    assert seen == sorted(g["ancestors_of_e"] + ["e"])
    for hidden in ("c", "f", "g"):      # c precedes e in the order, yet stays hidden
        assert not r.mask[0, e, names.index(hidden)]


@pytest.mark.parametrize("dfs", [True, False])
@pytest.mark.parametrize("N,max_depth,branch", [(1, 0, 1), (2, 1, 1), (13, 4, 3), (64, 8, 4),
                                                (70, 69, 1), (130, 12, 4)])
def test_mask_is_the_closure_of_the_parent_relation(N, max_depth, branch, dfs):
    parents = synth.tree_parent_arrays(15100 + N, 3, N, max_depth, branch, dfs=dfs)
    r = oracle.tree_attention_mask(parents, max_depth)
    for b in range(parents.shape[0]):
        M = closure_mask(parents[b].tolist())
        assert np.array_equal(r.mask[b], M)
        # a row holds the node and its depth-many ancestors
        assert np.array_equal(r.mask[b].sum(axis=1) - 1, r.depth[b])
        for i in range(1, N):
            assert r.depth[b, i] == r.depth[b, parents[b, i]] + 1
        assert r.tree_depth[b] == r.depth[b].max() <= max_depth


def test_dfs_interval_property():
    """Depth-first linearisation: j is an ancestor-or-self of i exactly when
    j <= i < j + size(j) (a subtree is a contiguous run in preorder)."""
    parents = synth.tree_parent_arrays(15120, 4, 64, 8, 4, dfs=True)
    r = oracle.tree_attention_mask(parents, 8)
    for b in range(parents.shape[0]):
        N = parents.shape[1]
        size = np.ones(N, dtype=np.int64)
        for i in range(N - 1, 0, -1):
            size[parents[b, i]] += size[i]
        for i in range(N):
            for j in range(N):
                assert r.mask[b, i, j] == (j <= i < j + size[j])


def test_invalid_requests():
    good = [-1, 0, 1, 0]
    bad = [
        [0, 0, 1, 0],      # root with a parent
        [-1, 0, 2, 0],     # parent not before its child
        [-1, 0, -3, 0],    # negative parent off the root
        [-1, 0, 1, 2],     # depth 3 > max_depth 2
    ]
    parents = np.array([good] + bad + [good], dtype=np.int32)
    r = oracle.tree_attention_mask(parents, max_depth=2)
    for b in (1, 2, 3, 4):
        assert not r.mask[b].any()
        assert (r.depth[b] == -1).all() and r.tree_depth[b] == -1
    for b in (0, 5):
        assert r.depth[b].tolist() == [0, 1, 2, 1] and r.tree_depth[b] == 2
        assert np.array_equal(r.mask[b], closure_mask(good))
