"""GPU parity of spec_verify_chain against the fp64 oracle (through the C ABI)."""
import numpy as np
import pytest
import torch

import oracle
import synth
import rejection_sampling_verify_15_amd as sv
from parity import (Tally, assert_shared_workspace_zero, compare_chain, oracle_chain_many, to_device,
                    to_device_logits)

pytestmark = pytest.mark.gpu


def run_gpu(ci, u_sets, draft_on_device=True):
    """One library call per uniform set; returns [(tokens, n)] as numpy."""
    tgt = to_device_logits(ci.target, ci.dtype)
    drf = to_device_logits(ci.draft, ci.dtype) if (draft_on_device and ci.gamma > 0) else None
    tok = to_device(ci.draft_tokens.astype(np.int32))
    T = to_device(ci.temperature.astype(np.float32))
    outs = []
    for u in u_sets:
        ud = to_device(np.asarray(u, dtype=np.float32))
        ot, on = sv.verify_chain(tgt, drf, tok, ud, T)
        outs.append((ot, on))
    assert_shared_workspace_zero("chain")
    return [(ot.cpu().numpy(), on.cpu().numpy()) for ot, on in outs]


def parity(ci, n_sets, seed=1, label=""):
    u_sets = [ci.uniforms] + [ci.fresh_uniforms(seed * 1000 + s) for s in range(n_sets - 1)]
    gpu = run_gpu(ci, u_sets)
    ref = oracle_chain_many(ci, u_sets)
    tally = Tally()
    for (ot, on), r in zip(gpu, ref):
        tally.add(compare_chain(r, ot, on))
    print(f"[{label}] {tally}", flush=True)
    tally.check(label)
    return tally, gpu, ref


def test_small_mixed_vector_path():
    ci = synth.chain_inputs(101, B=16, gamma=4, V=20000, dtype="bf16", family="peaked",
                            draft_sigma=(0.3, 2.0), temperature=0.7, greedy_odd=True)
    t, _, _ = parity(ci, 60, label="bf16 V=20000 mixed")
    assert t.decisions > 1000


@pytest.mark.parametrize("dtype,V", [("bf16", 20001), ("f32", 9999), ("f32", 16384)])
def test_scalar_and_f32_paths(dtype, V):
    ci = synth.chain_inputs(102, B=12, gamma=3, V=V, dtype=dtype, family="gauss",
                            draft_sigma=(0.3, 1.5), temperature=1.0, greedy_odd=True)
    parity(ci, 20, label=f"{dtype} V={V}")


def test_toy_config_full():
    """V=5 fp32, B=4096: parity plus the Monte-Carlo first-slot law on the GPU's outputs."""
    ci = synth.toy_chain()
    _, gpu, _ = parity(ci, 4, label="toy")
    from oracle import specverify_oracle as so
    tgt = np.stack([so.logits_to_f64(ci.target[b], "f32") for b in range(ci.B)])
    e = np.exp(tgt[:, 0, :] - tgt[:, 0, :].max(-1, keepdims=True))
    p1 = e / e.sum(-1, keepdims=True)
    first = np.concatenate([ot[:, 0] for ot, _ in gpu])
    p1r = np.concatenate([p1] * len(gpu))
    for k in range(ci.V):
        obs = (first == k).sum()
        exp = p1r[:, k].sum()
        sd = np.sqrt((p1r[:, k] * (1 - p1r[:, k])).sum())
        assert abs(obs - exp) < 4.5 * sd


def test_single_request_config_many_rounds():
    ci = synth.single_chain()
    t, _, _ = parity(ci, 1500, label="single B=1 V=32000")
    assert t.decisions > 3000


@pytest.fixture(scope="module")
def batched():
    return synth.batched_chain()


def test_batched_config_full(batched):
    t, _, _ = parity(batched, 300, label="batched B=64 V=128256")
    assert t.decisions > 30000


def test_deep_config_full():
    ci = synth.deep_chain()
    t, _, _ = parity(ci, 24, label="deep B=256 gamma=8 V=151936")
    assert t.decisions > 20000


def test_gamma_zero_is_a_plain_draw():
    ci = synth.chain_inputs(103, B=8, gamma=0, V=3000, dtype="bf16", family="peaked",
                            temperature=1.0, greedy_odd=True)
    parity(ci, 50, label="gamma=0")


def test_vocab_of_one_and_tiny():
    for V in (1, 2, 8):
        ci = synth.chain_inputs(104, B=6, gamma=3, V=V, dtype="f32", family="gauss",
                                temperature=1.0, greedy_odd=True)
        parity(ci, 10, label=f"V={V}")


def test_all_greedy_without_draft_logits():
    ci = synth.chain_inputs(105, B=10, gamma=5, V=5000, dtype="bf16", family="peaked",
                            temperature=0.0)
    # let half the requests match their first drafts to exercise long accepts
    from oracle import specverify_oracle as so
    for b in range(0, ci.B, 2):
        for i in range(ci.gamma):
            ci.draft_tokens[b, i] = int(np.argmax(so.logits_to_f64(ci.target[b, i], "bf16")))
    u = [ci.uniforms]
    gpu = run_gpu(ci, u, draft_on_device=False)
    ref = oracle_chain_many(ci, u)
    t = compare_chain(ref[0], *gpu[0])
    t.check("all greedy, no draft")
    assert (gpu[0][1][0::2] == ci.gamma).all()


def test_invalid_requests_are_flagged():
    ci = synth.chain_inputs(106, B=12, gamma=3, V=4000, dtype="bf16", family="gauss",
                            temperature=1.0)
    ci.draft_tokens[0, 1] = 4000
    ci.draft_tokens[1, 0] = -3
    ci.temperature[2] = -1.0
    ci.temperature[3] = np.nan
    ci.temperature[4] = np.inf
    ci.temperature[5] = 1e-40          # positive but not a normal float
    ci.uniforms[6, 3] = 1.0
    ci.uniforms[7, 0] = -0.25
    ci.temperature[8] = 0.0            # greedy: uniforms ignored
    ci.uniforms[8, :] = 5.0
    gpu = run_gpu(ci, [ci.uniforms])
    ref = oracle.verify_chain(ci.target, ci.draft, ci.draft_tokens, ci.uniforms, ci.temperature,
                              ci.dtype)
    for b in range(8):
        assert gpu[0][1][b] == -1 and (gpu[0][0][b] == -1).all(), b
        assert ref.num_accepted[b] == -1
    compare_chain(ref, *gpu[0]).check("invalid")


def test_masked_logits():
    """-inf (masked) entries, including draft tokens the target masks."""
    ci = synth.chain_inputs(107, B=16, gamma=4, V=6000, dtype="bf16", family="peaked",
                            temperature=1.0, greedy_odd=True)
    rng = np.random.default_rng(0)
    neg_inf_bf16 = np.uint16(0xFF80)
    for arr in (ci.target, ci.draft):
        mask = rng.random(arr.shape) < 0.3
        arr[mask] = neg_inf_bf16
    # make sure some draft tokens are masked in the target (p = 0)
    for b in range(0, ci.B, 3):
        ci.target[b, 0, ci.draft_tokens[b, 0]] = neg_inf_bf16
    # each row keeps a finite entry
    ci.target[:, :, 0] = 0
    ci.draft[:, :, 0] = 0
    parity(ci, 30, label="masked")


@pytest.mark.parametrize("T", [1e-3, 0.05, 3.0, 50.0])
def test_temperature_extremes(T):
    ci = synth.chain_inputs(108, B=8, gamma=3, V=7000, dtype="bf16", family="peaked",
                            temperature=T)
    parity(ci, 20, label=f"T={T}")


def test_repeat_calls_are_deterministic(batched):
    u = [batched.uniforms] * 3
    gpu = run_gpu(batched, u)
    for ot, on in gpu[1:]:
        assert np.array_equal(ot, gpu[0][0]) and np.array_equal(on, gpu[0][1])


def test_workspace_is_left_zeroed_across_shapes():
    """One workspace serves calls of different shapes in a row: every completed
    call returns it to all-zero, and each call stays correct."""
    dev = torch.device("cuda")
    L = sv.lib()
    shapes = [(16, 4, 20000, "bf16"), (12, 3, 20001, "bf16"), (40, 2, 3000, "f32"),
              (3, 6, 50000, "bf16"), (16, 4, 20000, "bf16")]
    need = max(L.sv_chain_workspace_bytes(B, g, V, 0) for B, g, V, _ in shapes)
    ws = torch.zeros(need, dtype=torch.uint8, device=dev)
    for i, (B, g, V, dt) in enumerate(shapes):
        ci = synth.chain_inputs(400 + i, B=B, gamma=g, V=V, dtype=dt, family="peaked",
                                draft_sigma=(0.3, 2.0), temperature=0.9, greedy_odd=True)
        ot, on = sv.verify_chain(to_device_logits(ci.target, dt), to_device_logits(ci.draft, dt),
                                 to_device(ci.draft_tokens.astype(np.int32)),
                                 to_device(ci.uniforms), to_device(ci.temperature), ws=ws)
        torch.cuda.synchronize()
        assert int(ws.count_nonzero()) == 0, f"workspace not zero after call {i}"
        ref = oracle.verify_chain(ci.target, ci.draft, ci.draft_tokens, ci.uniforms,
                                  ci.temperature, dt)
        compare_chain(ref, ot.cpu().numpy(), on.cpu().numpy()).check(f"shape {i}")


def test_kernel_timer_counts_every_launch(batched):
    """Events attached to the dispatches time each of the chain kernels, and
    timing does not change the results."""
    tgt = to_device_logits(batched.target, batched.dtype)
    drf = to_device_logits(batched.draft, batched.dtype)
    tok = to_device(batched.draft_tokens.astype(np.int32))
    u = to_device(batched.uniforms)
    T = to_device(batched.temperature)
    plain = [t.cpu() for t in sv.verify_chain(tgt, drf, tok, u, T)]
    with sv.KernelTimer(64) as timer:
        for _ in range(4):
            timed = sv.verify_chain(tgt, drf, tok, u, T)
    assert timer.launches["chain_verify"] == 4 and len(timer.launches) == 1
    assert 0.0 < timer.mean_us("chain_verify") < 1e5
    assert torch.equal(plain[0], timed[0].cpu()) and torch.equal(plain[1], timed[1].cpu())


def test_single_launch_returns_workspace_to_zero(batched):
    """After the one-launch form every workspace word it used is zero again, so
    the next call (on the same workspace) starts clean; three calls in a row
    with fresh uniforms agree with the oracle."""
    ci = batched
    need = sv.lib().sv_chain_workspace_bytes(ci.B, ci.gamma, ci.V, 0)
    ws = torch.zeros(need, dtype=torch.uint8, device=torch.device("cuda"))
    tgt = to_device_logits(ci.target, ci.dtype)
    drf = to_device_logits(ci.draft, ci.dtype)
    tok = to_device(ci.draft_tokens.astype(np.int32))
    T = to_device(ci.temperature)
    u_sets = [ci.fresh_uniforms(900 + s) for s in range(3)]
    refs = oracle_chain_many(ci, u_sets)
    tally = Tally()
    for u, ref in zip(u_sets, refs):
        ot, on = sv.verify_chain(tgt, drf, tok, to_device(u), T, ws=ws)
        torch.cuda.synchronize()
        assert int(ws.count_nonzero()) == 0
        tally.add(compare_chain(ref, ot.cpu().numpy(), on.cpu().numpy()))
    tally.check("single launch, shared workspace")


@pytest.mark.parametrize("cap", [37, 1000])
def test_split_form_with_striding_workgroups(cap):
    """The split form (decisions and draw units in launches of their own, used
    when one grid would be too large) with a small workgroup cap, so that
    every workgroup strides over several items; it must agree with the oracle
    and leave the workspace zeroed."""
    ci = synth.chain_inputs(131, B=24, gamma=3, V=40000, dtype="bf16", family="peaked",
                            draft_sigma=(0.3, 2.0), temperature=0.8, greedy_odd=True)
    dev = torch.device("cuda")
    need = sv.lib().sv_chain_workspace_bytes(ci.B, ci.gamma, ci.V, 0)
    ws = torch.zeros(need, dtype=torch.uint8, device=dev)
    tgt = to_device_logits(ci.target, ci.dtype)
    drf = to_device_logits(ci.draft, ci.dtype)
    tok = to_device(ci.draft_tokens.astype(np.int32))
    T = to_device(ci.temperature)
    u_sets = [ci.uniforms] + [ci.fresh_uniforms(700 + s) for s in range(7)]
    refs = oracle_chain_many(ci, u_sets)
    tally = Tally()
    for u, ref in zip(u_sets, refs):
        with sv.library_control(sv.SV_HOOK_CHAIN_GRID_CAP, cap), sv.KernelTimer(8) as timer:
            ot, on = sv.verify_chain(tgt, drf, tok, to_device(u), T, ws=ws)
            torch.cuda.synchronize()
        for name in ("chain_stream", "chain_decide", "chain_units"):
            assert timer.launches.get(name) == 1, name
        assert int(ws.count_nonzero()) == 0
        tally.add(compare_chain(ref, ot.cpu().numpy(), on.cpu().numpy()))
    tally.check(f"split form cap={cap}")


def test_three_launch_form_batched(batched):
    """The three-launch form (persistent, prefetching streaming launch, then
    decisions, then draw units) agrees with the oracle on the batched
    workload."""
    with sv.library_control(sv.SV_HOOK_CHAIN_SPLIT, 1):
        parity(batched, 20, label="three launches, batched")


def test_graph_capture_replays_match_eager():
    """One call captured in a HIP graph and replayed several times, with eager
    calls (on other uniforms) and synchronisations between the replays: every
    replay gives the eager result for the captured inputs, and the shared
    workspace stays zero."""
    ci = synth.single_chain()
    dev = torch.device("cuda")
    tgt = to_device_logits(ci.target, ci.dtype)
    drf = to_device_logits(ci.draft, ci.dtype)
    tok = to_device(ci.draft_tokens.astype(np.int32))
    T = to_device(ci.temperature)
    u0 = to_device(ci.uniforms)
    need = sv.lib().sv_chain_workspace_bytes(ci.B, ci.gamma, ci.V, 0)
    ws = torch.zeros(need, dtype=torch.uint8, device=dev)
    out_t = torch.empty((ci.B, ci.gamma + 1), dtype=torch.int32, device=dev)
    out_n = torch.empty((ci.B,), dtype=torch.int32, device=dev)
    sv.verify_chain(tgt, drf, tok, u0, T, out_tokens=out_t, out_num_accepted=out_n, ws=ws)
    torch.cuda.synchronize()
    want_t, want_n = out_t.clone(), out_n.clone()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            sv.verify_chain(tgt, drf, tok, u0, T, out_tokens=out_t, out_num_accepted=out_n, ws=ws)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    for r in range(4):
        out_t.fill_(-7)
        out_n.fill_(-7)
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out_t, want_t) and torch.equal(out_n, want_n), f"replay {r}"
        assert int(ws.count_nonzero()) == 0
        # eager work on other uniforms between the replays
        other_t, other_n = sv.verify_chain(tgt, drf, tok, to_device(ci.fresh_uniforms(4242 + r)), T, ws=ws)
        torch.cuda.synchronize()
        assert int(other_n.item()) >= 0


def test_prepared_call_matches_the_checked_call():
    """prepare_chain: the same outputs as verify_chain, call after call, with
    new uniforms written into the same buffer; and the status of a failing
    call raised."""
    ci = synth.chain_inputs(16601, B=12, gamma=3, V=20000, dtype="bf16", family="peaked",
                            draft_sigma=0.6, temperature=0.9, greedy_odd=True)
    tgt = to_device_logits(ci.target, ci.dtype)
    drf = to_device_logits(ci.draft, ci.dtype)
    tok = to_device(ci.draft_tokens.astype(np.int32))
    T = to_device(ci.temperature.astype(np.float32))
    u = to_device(ci.uniforms)
    for hint in (None, ci.temperature > 0):
        call = sv.prepare_chain(tgt, drf, tok, u, T, sampling_hint=hint)
        for s in range(4):
            u.copy_(to_device(ci.fresh_uniforms(16602 + s)))
            ot, on = call()
            et, en = sv.verify_chain(tgt, drf, tok, u, T)
            assert torch.equal(ot, et) and torch.equal(on, en)
    bad = sv.prepare_chain(tgt, drf, tok, u, T, ws=torch.zeros(256, dtype=torch.uint8, device="cuda"))
    with pytest.raises(sv.SVError):
        bad()
