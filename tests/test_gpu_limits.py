"""GPU parity at the shape limits the header declares, through the C ABI:
the longest draft (gamma = SV_MAX_GAMMA), the largest batch
(B = SV_MAX_BATCH, oracle on a sample of requests plus properties on all),
the largest vocabulary (V = SV_MAX_VOCAB), and a token tree of
SV_MAX_TREE_NODES nodes whose accepted path reaches SV_MAX_TREE_DEPTH.  One
past each limit is refused by the library itself."""
import numpy as np
import pytest
import torch

import oracle
import synth
import rejection_sampling_verify_15_amd as sv
from parity import (Tally, assert_shared_workspace_zero, compare_chain, compare_tree, compare_tree_mss,
                    oracle_chain_many, to_device, to_device_logits)

pytestmark = pytest.mark.gpu

MAX_GAMMA = 32
MAX_BATCH = 16384
MAX_VOCAB = 1 << 24
MAX_NODES = 1024
MAX_DEPTH = 64


def chain_gpu(ci, u_sets):
    tgt = to_device_logits(ci.target, ci.dtype)
    drf = to_device_logits(ci.draft, ci.dtype) if ci.gamma > 0 else None
    tok = to_device(ci.draft_tokens.astype(np.int32))
    T = to_device(ci.temperature.astype(np.float32))
    outs = []
    for u in u_sets:
        ot, on = sv.verify_chain(tgt, drf, tok, to_device(np.asarray(u, np.float32)), T)
        outs.append((ot.cpu().numpy(), on.cpu().numpy()))
    del tgt, drf
    assert_shared_workspace_zero("chain limits")
    return outs


def chain_parity(ci, n_sets, label, requests=None, seed=11):
    u_sets = [ci.uniforms] + [ci.fresh_uniforms(seed * 1000 + s) for s in range(n_sets - 1)]
    print(f"[{label}] B={ci.B} gamma={ci.gamma} V={ci.V} dtype={ci.dtype} sets={n_sets}", flush=True)
    gpu = chain_gpu(ci, u_sets)
    ref = oracle_chain_many(ci, u_sets, requests=requests)
    tally = Tally()
    for (ot, on), r in zip(gpu, ref):
        tally.add(compare_chain(r, ot, on, requests=requests))
    print(f"[{label}] {tally}", flush=True)
    tally.check(label)
    return gpu


def test_chain_longest_draft():
    """gamma = 32 with close drafts, so that accepted runs reach deep
    positions; odd requests greedy."""
    ci = synth.chain_inputs(15700, B=12, gamma=MAX_GAMMA, V=4000, dtype="bf16", family="gauss",
                            draft_sigma=(0.02, 0.3), temperature=1.0, greedy_odd=True)
    gpu = chain_parity(ci, 12, "gamma=32")
    assert max(int(on.max()) for _, on in gpu) >= 16


def test_chain_longest_draft_ragged():
    """Request b drafts b tokens, b = 0..32, in one ragged call."""
    ci = synth.chain_inputs(15705, B=MAX_GAMMA + 1, gamma=MAX_GAMMA, V=3000, dtype="bf16", family="gauss",
                            draft_sigma=(0.02, 0.4), temperature=0.9, greedy_odd=True)
    gam = np.arange(ci.B, dtype=np.int32)
    tgt = to_device_logits(ci.target, ci.dtype)
    drf = to_device_logits(ci.draft, ci.dtype)
    tok = to_device(ci.draft_tokens.astype(np.int32))
    T = to_device(ci.temperature)
    tally = Tally()
    for s in range(6):
        u = ci.uniforms if s == 0 else ci.fresh_uniforms(15706 + s)
        ot, on, _ = sv.verify_chain_ragged(tgt, drf, tok, to_device(u), T, to_device(gam))
        ref = oracle.verify_chain_ragged(ci.target, ci.draft, ci.draft_tokens, u, ci.temperature, gam, "bf16")
        tally.add(compare_chain(ref, ot.cpu().numpy(), on.cpu().numpy()))
        assert (on.cpu().numpy() <= gam).all()
    print(f"[ragged gamma<=32] {tally}", flush=True)
    tally.check("ragged gamma<=32")
    assert_shared_workspace_zero("chain ragged limits")


def check_chain_properties(ci, ot, on):
    """What holds for every request of any call: 0 <= n <= gamma, tokens
    [0, n] inside the vocabulary, -1 after them, and the accepted drafts
    copied from the input."""
    G = ci.gamma
    assert ((on >= 0) & (on <= G)).all()
    cols = np.arange(G + 1)[None, :]
    emitted = cols <= on[:, None]
    assert ((ot >= 0) & (ot < ci.V))[emitted].all()
    assert (ot[~emitted] == -1).all()
    acc = cols[:, :G] < on[:, None]
    assert (ot[:, :G][acc] == ci.draft_tokens[acc]).all()


def test_chain_largest_batch():
    """B = 16384 requests (a quarter greedy), gamma = 2, V = 300 fp32: the
    oracle on 600 sampled requests, the output properties on all."""
    ci = synth.chain_inputs(15710, B=MAX_BATCH, gamma=2, V=300, dtype="f32", family="gauss",
                            draft_sigma=(0.2, 1.5), temperature=0.8)
    ci.temperature[::4] = 0.0
    rng = np.random.default_rng(15711)
    sample = np.sort(rng.choice(ci.B, size=600, replace=False))
    sample[:2] = [0, 1]
    sample[-1] = ci.B - 1
    gpu = chain_parity(ci, 3, "B=16384", requests=[int(b) for b in np.unique(sample)])
    for ot, on in gpu:
        check_chain_properties(ci, ot, on)


def test_chain_largest_vocabulary():
    """V = 2^24 bf16, gamma = 2: one sampling request (T = 1) and one greedy;
    each row is 4096 stream chunks and the draw covers 16384 units."""
    ci = synth.chain_inputs(15720, B=2, gamma=2, V=MAX_VOCAB, dtype="bf16", family="peaked",
                            draft_sigma=0.5, temperature=1.0, greedy_odd=True)
    gpu = chain_parity(ci, 4, "V=2^24")
    for ot, on in gpu:
        check_chain_properties(ci, ot, on)


def spine_tree(N, depth, max_kids, spine_first):
    """A root-to-leaf spine of `depth` edges with side leaves hung on the
    spine nodes until the tree has N nodes (each node at most max_kids
    children, the spine child first or last among its siblings);
    depth-first labelled.  Returns the parent array and, for each node,
    whether it lies on the spine."""
    children = [[] for _ in range(N)]
    spine = list(range(depth + 1))
    nxt = depth + 1
    side = N - (depth + 1)
    per = [side // depth + (1 if i < side % depth else 0) for i in range(depth)]
    assert max(per) + 1 <= max_kids
    for i in range(depth):
        if spine_first:
            children[spine[i]].append(spine[i + 1])
        for _ in range(per[i]):
            children[spine[i]].append(nxt)
            nxt += 1
        if not spine_first:
            children[spine[i]].append(spine[i + 1])
    _, new_id = synth.dfs_relabel(children)
    par = np.full(N, -1, np.int32)
    on_spine = np.zeros(N, bool)
    for old in range(N):
        for c in children[old]:
            par[new_id[c]] = new_id[old]
    for s in spine:
        on_spine[new_id[s]] = True
    return par, on_spine


def spine_tree_inputs(seed, B, V, T, spine_first=False, draft_sigma=0.3):
    """B trees of 1024 nodes, a 64-deep spine each.  Node logits are peaked
    bf16 rows; a spine child carries the target argmax of its parent (so the
    greedy descent accepts the whole spine), every other child a distinct
    random token that is not that argmax.  Draft rows are the target rows
    plus N(0, draft_sigma^2) noise."""
    rng = np.random.default_rng(seed)
    logits32 = synth.peaked_logits(rng, B * MAX_NODES, V).reshape(B, MAX_NODES, V)
    tl = synth.bf16_round_bits(logits32)
    wide = synth.bf16_bits_as_float32(tl)
    dl = synth.bf16_round_bits(wide + rng.standard_normal(tl.shape).astype(np.float32) * np.float32(draft_sigma))
    parents = np.empty((B, MAX_NODES), np.int32)
    tokens = np.zeros((B, MAX_NODES), np.int32)
    for b in range(B):
        par, on_spine = spine_tree(MAX_NODES, MAX_DEPTH, 64, spine_first)
        parents[b] = par
        for n in range(MAX_NODES):
            kids = np.flatnonzero(par == n)
            if kids.size == 0:
                continue
            top = int(np.argmax(wide[b, n]))
            others = rng.permutation(np.delete(np.arange(V), top))[:kids.size]
            for j, c in enumerate(kids):
                tokens[b, c] = top if on_spine[c] else int(others[j])
    return synth.TreeInputs(tl, tokens, parents, synth.uniforms(rng, (B, MAX_NODES)),
                            np.full(B, T, np.float32), "bf16", B, MAX_NODES, V, MAX_DEPTH, "spine",
                            f"seed={seed} spine tree", dl, synth.uniforms(rng, (B, MAX_NODES)))


def test_tree_largest_greedy_accepts_the_full_depth():
    ti = spine_tree_inputs(15730, B=3, V=2000, T=0.0)
    lg = to_device_logits(ti.logits, ti.dtype)
    ot, op, on = (x.cpu().numpy() for x in sv.verify_tree(
        lg, to_device(ti.node_tokens), to_device(ti.parents), to_device(ti.uniforms),
        to_device(ti.temperature), ti.max_depth))
    ref = oracle.verify_tree(ti.logits, ti.node_tokens, ti.parents, ti.uniforms, ti.temperature, "bf16", ti.max_depth)
    t = compare_tree(ref, ot, op, on)
    t.check("tree 1024 nodes greedy")
    assert (on == MAX_DEPTH).all() and (ref.num_accepted == MAX_DEPTH).all()
    assert_shared_workspace_zero("tree limits")


def test_tree_largest_sampling_and_mss():
    """Spine-first trees at T = 0.3 with close drafts: naive sampling
    descends the spine while the argmax keeps most of p, and multi-step
    speculative sampling tests the spine child first at every node."""
    ti = spine_tree_inputs(15740, B=3, V=2000, T=0.3, spine_first=True, draft_sigma=0.05)
    lg = to_device_logits(ti.logits, ti.dtype)
    dl = to_device_logits(ti.draft_logits, ti.dtype)
    tok, par, T = to_device(ti.node_tokens), to_device(ti.parents), to_device(ti.temperature)
    rng = np.random.default_rng(15741)
    naive, mss = Tally(), Tally()
    deepest = deepest_mss = 0
    for s in range(6):
        ua = ti.uniforms if s == 0 else synth.uniforms(rng, (ti.B, ti.N))
        ud = ti.draw_uniforms if s == 0 else synth.uniforms(rng, (ti.B, ti.N))
        ot, op, on = (x.cpu().numpy() for x in sv.verify_tree(lg, tok, par, to_device(ua), T, ti.max_depth))
        ref = oracle.verify_tree(ti.logits, ti.node_tokens, ti.parents, ua, ti.temperature, "bf16", ti.max_depth)
        naive.add(compare_tree(ref, ot, op, on))
        deepest = max(deepest, int(on.max()))
        mt, mp, mn = (x.cpu().numpy() for x in sv.verify_tree_mss(lg, dl, tok, par, to_device(ua), to_device(ud),
                                                                   T, ti.max_depth))
        mref = oracle.verify_tree_mss(ti.logits, ti.draft_logits, ti.node_tokens, ti.parents, ua, ud,
                                      ti.temperature, "bf16", ti.max_depth)
        mss.add(compare_tree_mss(mref, mt, mp, mn))
        deepest_mss = max(deepest_mss, int(mn.max()))
    print(f"[tree 1024 nodes naive] {naive} deepest={deepest}", flush=True)
    print(f"[tree 1024 nodes mss] {mss} deepest={deepest_mss}", flush=True)
    naive.check("tree 1024 nodes naive")
    mss.check("tree 1024 nodes mss")
    assert deepest >= 8 and deepest_mss >= 8
    assert_shared_workspace_zero("tree limits")


def test_one_past_each_limit_is_refused():
    dev = torch.device("cuda:0")

    def chain(B, gamma, V):
        tgt = torch.zeros((B, gamma + 1, V), dtype=torch.float32, device=dev)
        drf = torch.zeros((B, gamma, V), dtype=torch.float32, device=dev) if gamma > 0 else None
        return sv.verify_chain(tgt, drf, torch.zeros((B, gamma), dtype=torch.int32, device=dev),
                               torch.zeros((B, gamma + 1), dtype=torch.float32, device=dev),
                               torch.ones(B, dtype=torch.float32, device=dev))

    for shape in ((1, MAX_GAMMA + 1, 4), (MAX_BATCH + 1, 0, 1), (1, 0, MAX_VOCAB + 1)):
        with pytest.raises(sv.SVError):
            chain(*shape)
    # at the limits themselves the calls go through
    for shape in ((1, MAX_GAMMA, 4), (MAX_BATCH, 0, 1)):
        ot, on = chain(*shape)
        torch.cuda.synchronize()

    def tree(N, max_depth):
        z = torch.zeros((1, N), dtype=torch.int32, device=dev)
        z[0, 0] = -1
        return sv.verify_tree(torch.zeros((1, N, 8), dtype=torch.float32, device=dev), torch.zeros_like(z), z,
                              torch.zeros((1, N), dtype=torch.float32, device=dev),
                              torch.zeros(1, dtype=torch.float32, device=dev), max_depth)

    for N, depth in ((MAX_NODES + 1, 4), (4, MAX_DEPTH + 1)):
        with pytest.raises(sv.SVError):
            tree(N, depth)
    # at the limits: 1023 children of the root, all carrying token 0, the
    # greedy argmax of the all-zero rows
    ot, op, on = (x.cpu().numpy() for x in tree(MAX_NODES, MAX_DEPTH))
    par = np.zeros((1, MAX_NODES), np.int32)
    par[0, 0] = -1
    ref = oracle.verify_tree(np.zeros((1, MAX_NODES, 8), np.float32), np.zeros((1, MAX_NODES), np.int32), par,
                             np.zeros((1, MAX_NODES), np.float32), np.zeros(1, np.float32), "f32", MAX_DEPTH)
    compare_tree(ref, ot, op, on).check("root fan-out")
    assert int(on[0]) == 1
    assert_shared_workspace_zero("limits")
