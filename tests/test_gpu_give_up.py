"""Bounded waits that give up, forced from the host with the SV_HOOK_SPIN_LIMIT
control (every kernel still runs to its end): each request then either
reports SV_GAVE_UP (-2) or carries exactly the oracle's result, recover()
zero-fills the workspace when a request gave up, and the next call without
the control is exact and leaves the workspace zero."""
import ctypes

import numpy as np
import pytest
import torch

import oracle
import synth
import rejection_sampling_verify_15_amd as sv
from parity import (Tally, compare_chain, compare_tree, compare_tree_mss, oracle_chain_many, to_device,
                    to_device_logits)

pytestmark = pytest.mark.gpu

SPINS = (1, 64)


def chain_case(label, ci, ws, u_sets, hooks=()):
    """Calls under each spin limit (and extra controls), then one plain call;
    returns how many requests gave up."""
    tgt = to_device_logits(ci.target, ci.dtype)
    drf = to_device_logits(ci.draft, ci.dtype)
    tok = to_device(ci.draft_tokens.astype(np.int32))
    T = to_device(ci.temperature.astype(np.float32))
    refs = oracle_chain_many(ci, u_sets)
    gave_up = 0
    tally = Tally()
    for spin in SPINS:
        for u, ref in zip(u_sets, refs):
            print(f"[{label}] spin={spin} B={ci.B} V={ci.V}", flush=True)
            with sv.library_control(sv.SV_HOOK_SPIN_LIMIT, spin):
                for h, v in hooks:
                    sv.lib().sv_set_test_hook(h, v)
                try:
                    ot, on = sv.verify_chain(tgt, drf, tok, to_device(u), T, ws=ws)
                    torch.cuda.synchronize()
                finally:
                    for h, _ in hooks:
                        sv.lib().sv_set_test_hook(h, 0)
            n = on.cpu().numpy()
            assert ((n >= -2) & (n <= ci.gamma)).all(), label
            kept = [b for b in range(ci.B) if n[b] != sv.SV_GAVE_UP]
            gave_up += ci.B - len(kept)
            tally.add(compare_chain(ref, ot.cpu().numpy(), n, requests=kept))
            assert sv.recover(on, ws) == (len(kept) < ci.B)
            torch.cuda.synchronize()
            assert int(ws.count_nonzero()) == 0, label
    tally.check(f"{label}, requests that did not give up")
    # the same workspace, no control: exact, and zero afterwards
    ot, on = sv.verify_chain(tgt, drf, tok, to_device(u_sets[0]), T, ws=ws)
    torch.cuda.synchronize()
    t = compare_chain(refs[0], ot.cpu().numpy(), on.cpu().numpy())
    t.check(f"{label}, plain call after give-ups")
    assert int(ws.count_nonzero()) == 0
    print(f"[{label}] gave up {gave_up}; {tally}", flush=True)
    return gave_up


def zeroed_workspace(ci):
    need = sv.lib().sv_chain_workspace_bytes(ci.B, ci.gamma, ci.V, sv.SV_BF16)
    return torch.zeros(need, dtype=torch.uint8, device="cuda")


def test_chain_single_launch_decide_draws():
    """B <= 256: the decide item draws, so it alone writes a drawing request's count."""
    ci = synth.chain_inputs(16101, B=24, gamma=3, V=40000, dtype="bf16", family="peaked",
                            draft_sigma=(0.3, 2.0), temperature=0.8, greedy_odd=True)
    u_sets = [ci.uniforms] + [ci.fresh_uniforms(16110 + s) for s in range(2)]
    assert chain_case("chain single launch", ci, zeroed_workspace(ci), u_sets) > 0


def test_chain_single_launch_counted_units():
    """B > 256: the last unit of a request to count itself in draws and writes the count."""
    ci = synth.chain_inputs(16102, B=300, gamma=2, V=6000, dtype="bf16", family="gauss",
                            draft_sigma=(0.3, 1.5), temperature=1.0, greedy_odd=True)
    u_sets = [ci.uniforms, ci.fresh_uniforms(16120)]
    assert chain_case("chain counted units", ci, zeroed_workspace(ci), u_sets) > 0


def test_chain_three_launch_form():
    """The three-launch form: its waits are on earlier launches, so few or no
    requests give up; every result is still exact or SV_GAVE_UP."""
    ci = synth.chain_inputs(16103, B=20, gamma=4, V=30000, dtype="bf16", family="zipf",
                            draft_sigma=0.8, temperature=1.0)
    chain_case("chain three launches", ci, zeroed_workspace(ci), [ci.uniforms],
               hooks=((sv.SV_HOOK_CHAIN_SPLIT, 1),))


def test_chain_noalloc_reset_after_give_up():
    """The allocation-free entry: after a call with requests that gave up, a
    call with B == 0 zero-fills the static array, and the next call is exact."""
    ci = synth.chain_inputs(16104, B=16, gamma=3, V=20000, dtype="bf16", family="peaked",
                            draft_sigma=0.5, temperature=0.9)
    tgt = to_device_logits(ci.target, ci.dtype)
    drf = to_device_logits(ci.draft, ci.dtype)
    tok = to_device(ci.draft_tokens.astype(np.int32))
    T = to_device(ci.temperature.astype(np.float32))
    u = to_device(ci.uniforms)
    ot = torch.empty((ci.B, ci.gamma + 1), dtype=torch.int32, device="cuda")
    on = torch.empty((ci.B,), dtype=torch.int32, device="cuda")
    ref = oracle.verify_chain(ci.target, ci.draft, ci.draft_tokens, ci.uniforms, ci.temperature, ci.dtype)
    print("[noalloc give-up] spin=1", flush=True)
    with sv.library_control(sv.SV_HOOK_SPIN_LIMIT, 1):
        sv.verify_chain_noalloc(tgt, drf, tok, u, T, ot, on)
        torch.cuda.synchronize()
    n = on.cpu().numpy()
    kept = [b for b in range(ci.B) if n[b] != sv.SV_GAVE_UP]
    compare_chain(ref, ot.cpu().numpy(), n, requests=kept).check("noalloc, requests that did not give up")
    assert len(kept) < ci.B
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    st = sv.lib().spec_verify_chain_noalloc(None, None, None, None, None, 0, ci.gamma, ci.V, sv.SV_BF16,
                                            None, None, stream)
    assert st == sv.SV_OK
    sv.verify_chain_noalloc(tgt, drf, tok, u, T, ot, on)
    torch.cuda.synchronize()
    compare_chain(ref, ot.cpu().numpy(), on.cpu().numpy()).check("noalloc after the reset")


def tree_case(label, ti, mss):
    lg = to_device_logits(ti.logits, ti.dtype)
    tok = to_device(ti.node_tokens.astype(np.int32))
    par = to_device(ti.parents.astype(np.int32))
    T = to_device(ti.temperature.astype(np.float32))
    ua, ud = to_device(ti.uniforms), (to_device(ti.draw_uniforms) if mss else None)
    if mss:
        dl = to_device_logits(ti.draft_logits, ti.dtype)
        need = sv.lib().sv_tree_mss_workspace_bytes(ti.B, ti.N, ti.V, sv.SV_BF16)
        ref = oracle.verify_tree_mss(ti.logits, ti.draft_logits, ti.node_tokens, ti.parents, ti.uniforms,
                                     ti.draw_uniforms, ti.temperature, ti.dtype, ti.max_depth)
        compare = compare_tree_mss
    else:
        need = sv.lib().sv_tree_workspace_bytes(ti.B, ti.N, ti.V, sv.SV_BF16)
        ref = oracle.verify_tree(ti.logits, ti.node_tokens, ti.parents, ti.uniforms, ti.temperature,
                                 ti.dtype, ti.max_depth)
        compare = compare_tree
    ws = torch.zeros(max(int(need), 256), dtype=torch.uint8, device="cuda")

    def call():
        if mss:
            return sv.verify_tree_mss(lg, dl, tok, par, ua, ud, T, ti.max_depth, ws=ws)
        return sv.verify_tree(lg, tok, par, ua, T, ti.max_depth, ws=ws)

    gave_up = 0
    for spin in SPINS:
        print(f"[{label}] spin={spin} B={ti.B} N={ti.N} V={ti.V}", flush=True)
        with sv.library_control(sv.SV_HOOK_SPIN_LIMIT, spin):
            ot, op, on = call()
            torch.cuda.synchronize()
        n = on.cpu().numpy()
        assert ((n >= -2) & (n <= ti.max_depth)).all(), label
        kept = [b for b in range(ti.B) if n[b] != sv.SV_GAVE_UP]
        gave_up += ti.B - len(kept)
        compare(ref, ot.cpu().numpy(), op.cpu().numpy(), n, requests=kept).check(f"{label} spin={spin}")
        sv.recover(on, ws)
        torch.cuda.synchronize()
        assert int(ws.count_nonzero()) == 0, label
    ot, op, on = call()
    torch.cuda.synchronize()
    compare(ref, ot.cpu().numpy(), op.cpu().numpy(), on.cpu().numpy()).check(f"{label}, plain call")
    assert int(ws.count_nonzero()) == 0
    print(f"[{label}] gave up {gave_up}", flush=True)
    assert gave_up > 0


def test_tree_naive_give_up():
    ti = synth.tree_inputs(seed=16201, B=12, N=40, V=30000, max_depth=6, temperature=1.0, draft_sigma=0.3)
    tree_case("tree give-up", ti, mss=False)


def test_tree_mss_give_up():
    ti = synth.tree_inputs(seed=16202, B=12, N=40, V=30000, max_depth=6, temperature=1.0, draft_sigma=0.3,
                           family="gauss", keep_draft=True)
    tree_case("tree mss give-up", ti, mss=True)
