"""GPU parity of spec_verify_tree against the fp64 oracle (through the C ABI)."""
import numpy as np
import pytest
import torch

import oracle
import synth
import rejection_sampling_verify_15_amd as sv
from parity import Tally, assert_shared_workspace_zero, compare_tree, to_device, to_device_logits

pytestmark = pytest.mark.gpu


def run_tree(ti, u_sets):
    lg = to_device_logits(ti.logits, ti.dtype)
    tok = to_device(ti.node_tokens.astype(np.int32))
    par = to_device(ti.parents.astype(np.int32))
    T = to_device(ti.temperature.astype(np.float32))
    outs = []
    for u in u_sets:
        outs.append(sv.verify_tree(lg, tok, par, to_device(np.asarray(u, np.float32)), T, ti.max_depth))
    assert_shared_workspace_zero("tree")
    return [tuple(x.cpu().numpy() for x in o) for o in outs]


def tree_parity(ti, n_sets, label, seed=3):
    rng = np.random.default_rng(seed)
    u_sets = [ti.uniforms] + [synth.uniforms(rng, (ti.B, ti.N)) for _ in range(n_sets - 1)]
    gpu = run_tree(ti, u_sets)
    tally = Tally()
    for (ot, op, on), u in zip(gpu, u_sets):
        ref = oracle.verify_tree(ti.logits, ti.node_tokens, ti.parents, u, ti.temperature,
                                 ti.dtype, ti.max_depth)
        tally.add(compare_tree(ref, ot, op, on))
    print(f"[{label}] {tally}", flush=True)
    tally.check(label)
    return tally, gpu


def test_tree_config_greedy():
    ti = synth.tree_inputs(temperature=0.0)
    tree_parity(ti, 1, "tree greedy")


def test_tree_config_naive_sampling():
    ti = synth.tree_inputs(temperature=1.0)
    tree_parity(ti, 6, "tree sampling")


def test_small_trees_many_rounds():
    for T in (0.0, 0.8):
        ti = synth.tree_inputs(seed=301, B=24, N=40, V=3000, max_depth=6, temperature=T,
                               draft_sigma=0.3)
        t, gpu = tree_parity(ti, 40, f"small trees T={T}")
        assert max(int(on.max()) for _, _, on in gpu) >= 2     # some deep accepts happen


def test_tree_f32_scalar_path_and_mixed_modes():
    ti = synth.tree_inputs(seed=302, B=16, N=30, V=4001, max_depth=8, temperature=1.0,
                           dtype="f32", family="gauss", draft_sigma=0.2)
    ti.temperature[1::2] = 0.0
    tree_parity(ti, 20, "f32 mixed")


def test_root_only_and_chains():
    V = 500
    rng = np.random.default_rng(9)
    B, N = 4, 1
    logits = synth.bf16_round_bits(rng.standard_normal((B, N, V)).astype(np.float32))
    ti = synth.TreeInputs(logits, np.zeros((B, N), np.int32), -np.ones((B, N), np.int32),
                          synth.uniforms(rng, (B, N)), np.array([0, 1, 0.5, 2], np.float32),
                          "bf16", B, N, V, 0)
    _, gpu = tree_parity(ti, 5, "root only")
    assert (gpu[0][2] == 0).all()


def test_invalid_trees_are_flagged():
    ti = synth.tree_inputs(seed=303, B=8, N=16, V=1000, max_depth=8, temperature=1.0)
    ti.parents[0, 5] = 7          # parent after the child
    ti.parents[1, 0] = 0          # root with a parent
    ti.node_tokens[2, 3] = 1000   # token out of range
    ti.uniforms[3, 9] = 1.0       # uniform outside [0, 1)
    ti.temperature[4] = np.nan
    gpu = run_tree(ti, [ti.uniforms])
    ref = oracle.verify_tree(ti.logits, ti.node_tokens, ti.parents, ti.uniforms, ti.temperature,
                             ti.dtype, ti.max_depth)
    for b in range(5):
        assert ref.num_accepted[b] == -1 and gpu[0][2][b] == -1, b
        assert (gpu[0][0][b] == -1).all() and (gpu[0][1][b] == -1).all()
    compare_tree(ref, *gpu[0]).check("invalid trees")


def test_depth_cap_enforced():
    ti = synth.tree_inputs(seed=304, B=4, N=20, V=800, max_depth=8, temperature=0.0)
    ti.max_depth = 2           # the generated trees are deeper than 2
    gpu = run_tree(ti, [ti.uniforms])
    ref = oracle.verify_tree(ti.logits, ti.node_tokens, ti.parents, ti.uniforms, ti.temperature,
                             ti.dtype, 2)
    compare_tree(ref, *gpu[0]).check("depth cap")
    assert (ref.num_accepted == gpu[0][2]).all()


def test_multi_launch_form():
    """The multi-launch form (one step per depth level, used when the single
    launch's grid would be too large) agrees with the oracle."""
    with sv.library_control(sv.SV_HOOK_TREE_SPLIT, 1):
        for T in (0.0, 0.8):
            ti = synth.tree_inputs(seed=305, B=12, N=40, V=3000, max_depth=6, temperature=T, draft_sigma=0.3)
            tree_parity(ti, 10, f"multi-launch T={T}")


def test_graph_capture_replays_match_eager():
    """One tree call captured in a HIP graph and replayed several times, with
    eager calls (on other uniforms) and synchronisations between the replays:
    every replay gives the eager result for the captured inputs, and the
    workspace stays zero (the kernel leaves it so; no memset is captured)."""
    ti = synth.tree_inputs(seed=309, B=12, N=40, V=5000, max_depth=6, temperature=0.9, draft_sigma=0.3)
    ti.temperature[::3] = 0.0
    dev = torch.device("cuda")
    lg = to_device_logits(ti.logits, ti.dtype)
    tok = to_device(ti.node_tokens.astype(np.int32))
    par = to_device(ti.parents.astype(np.int32))
    T = to_device(ti.temperature.astype(np.float32))
    u0 = to_device(ti.uniforms)
    need = sv.lib().sv_tree_workspace_bytes(ti.B, ti.N, ti.V, 0)
    ws = torch.zeros(need, dtype=torch.uint8, device=dev)
    want = [x.clone() for x in sv.verify_tree(lg, tok, par, u0, T, ti.max_depth, ws=ws)]
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            got = sv.verify_tree(lg, tok, par, u0, T, ti.max_depth, ws=ws)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    rng = np.random.default_rng(12)
    for r in range(4):
        for x in got:
            x.fill_(-7)
        g.replay()
        torch.cuda.synchronize()
        for x, y in zip(got, want):
            assert torch.equal(x, y), f"replay {r}"
        assert int(ws.count_nonzero()) == 0
        # eager work on other uniforms between the replays
        sv.verify_tree(lg, tok, par, to_device(synth.uniforms(rng, (ti.B, ti.N))), T, ti.max_depth, ws=ws)
        torch.cuda.synchronize()
        assert int(ws.count_nonzero()) == 0


def test_more_workgroups_than_fit_at_once():
    """2048 small trees: 6144 workgroups of the single launch (a choose and two
    stream workgroups per request), more than the GPU holds at once, so later
    requests start only as earlier ones finish; every request still agrees
    with the oracle and the workspace returns to zero."""
    ti = synth.tree_inputs(seed=308, B=2048, N=16, V=3000, max_depth=5, temperature=0.9, draft_sigma=0.3)
    ti.temperature[::4] = 0.0
    tree_parity(ti, 2, "2048 trees")


def test_single_launch_after_the_other_forms_on_the_shared_workspace():
    """The debug-probabilities call and the multi-launch tree form run on the
    same cached workspace as the single-launch tree kernel, which counts and
    flags through it: each leaves it zero, so sampled tree calls after them
    still agree with the oracle."""
    ci = synth.chain_inputs(207, B=12, gamma=5, V=70000, dtype="bf16", family="peaked",
                            draft_sigma=0.5, temperature=0.9)
    sv.probs_debug(to_device_logits(ci.target, ci.dtype), to_device_logits(ci.draft, ci.dtype),
                   to_device(ci.draft_tokens.astype(np.int32)), to_device(ci.temperature.astype(np.float32)))
    assert_shared_workspace_zero("probs")
    ti = synth.tree_inputs(seed=307, B=20, N=48, V=40000, max_depth=7, temperature=1.0, draft_sigma=0.3)
    with sv.library_control(sv.SV_HOOK_TREE_SPLIT, 1):
        tree_parity(ti, 3, "multi-launch before single")
    tree_parity(ti, 6, "single after multi-launch", seed=4)


def test_single_launch_returns_workspace_to_zero():
    """Calls on one explicit workspace with invalid requests, early stops, deep
    accepts and mixed modes: the oracle agrees each time and every workspace
    word is zero again after each call."""
    ti = synth.tree_inputs(seed=306, B=10, N=48, V=5000, max_depth=7, temperature=0.9, draft_sigma=0.3)
    ti.temperature[::3] = 0.0
    ti.parents[4, 6] = 9          # invalid: parent after the child
    dev = torch.device("cuda")
    need = sv.lib().sv_tree_workspace_bytes(ti.B, ti.N, ti.V, 0)
    ws = torch.zeros(need, dtype=torch.uint8, device=dev)
    lg = to_device_logits(ti.logits, ti.dtype)
    tok = to_device(ti.node_tokens.astype(np.int32))
    par = to_device(ti.parents.astype(np.int32))
    T = to_device(ti.temperature.astype(np.float32))
    rng = np.random.default_rng(11)
    tally = Tally()
    for r in range(6):
        u = ti.uniforms if r == 0 else synth.uniforms(rng, (ti.B, ti.N))
        ot, op, on = sv.verify_tree(lg, tok, par, to_device(u), T, ti.max_depth, ws=ws)
        torch.cuda.synchronize()
        assert int(ws.count_nonzero()) == 0, f"call {r}"
        ref = oracle.verify_tree(ti.logits, ti.node_tokens, ti.parents, u, ti.temperature, ti.dtype, ti.max_depth)
        tally.add(compare_tree(ref, ot.cpu().numpy(), op.cpu().numpy(), on.cpu().numpy()))
    print(f"[tree workspace] {tally}", flush=True)
    tally.check("tree workspace")


@pytest.mark.parametrize("T", [0.0, 1.0])
def test_all_nodes_design_matches(T):
    """The all-nodes statistics form (SV_HOOK_TREE_ALL_NODES: every node's row
    reduced up front, then the descent) gives path descent's results: parity
    with the oracle at the token-tree shape, on small deep trees with mixed
    modes and an invalid request, and the workspace left zero."""
    with sv.library_control(sv.SV_HOOK_TREE_ALL_NODES, 1):
        ti = synth.tree_inputs(temperature=T)
        tree_parity(ti, 1 if T == 0.0 else 4, f"all-nodes T={T}")
        small = synth.tree_inputs(seed=311, B=16, N=40, V=3001, max_depth=6, temperature=max(T, 0.7),
                                  draft_sigma=0.3, dtype="f32", family="gauss")
        small.temperature[::3] = 0.0
        small.parents[5, 0] = 0    # an invalid request among valid ones
        tree_parity(small, 10, f"all-nodes small T={T}")
