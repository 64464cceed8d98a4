"""spec_verify_chain_hinted: the sampling hint changes only the layout of the
work, so every hint -- right, inverted, random, all or none -- gives exactly
the outputs of spec_verify_chain, which are at parity with the fp64 oracle,
and leaves the workspace zero."""
import numpy as np
import pytest
import torch

import synth
import rejection_sampling_verify_15_amd as sv
from parity import Tally, compare_chain, oracle_chain_many, to_device, to_device_logits

pytestmark = pytest.mark.gpu


def hints_for(ci, rng):
    right = ci.temperature > 0
    return {
        "right": right,
        "inverted": ~right,
        "random": rng.random(ci.B) < 0.5,
        "all": np.ones(ci.B, bool),
        "none": np.zeros(ci.B, bool),
    }


def run_hints(ci, n_sets, label, seed=1):
    tgt = to_device_logits(ci.target, ci.dtype)
    drf = to_device_logits(ci.draft, ci.dtype) if ci.gamma > 0 else None
    tok = to_device(ci.draft_tokens.astype(np.int32))
    T = to_device(ci.temperature.astype(np.float32))
    need = sv.lib().sv_chain_workspace_bytes(ci.B, ci.gamma, ci.V, sv.SV_BF16 if ci.dtype == "bf16" else sv.SV_F32)
    ws = torch.zeros(max(int(need), 256), dtype=torch.uint8, device="cuda")
    u_sets = [ci.uniforms] + [ci.fresh_uniforms(seed * 1000 + s) for s in range(n_sets - 1)]
    refs = oracle_chain_many(ci, u_sets)
    tally = Tally()
    hints = hints_for(ci, np.random.default_rng(seed))
    for u, ref in zip(u_sets, refs):
        ud = to_device(u)
        pt, pn = sv.verify_chain(tgt, drf, tok, ud, T, ws=ws)
        torch.cuda.synchronize()
        plain = (pt.cpu().numpy(), pn.cpu().numpy())
        tally.add(compare_chain(ref, *plain))
        for name, h in hints.items():
            print(f"[{label}] hint={name}", flush=True)
            ht, hn = sv.verify_chain(tgt, drf, tok, ud, T, ws=ws, sampling_hint=h)
            torch.cuda.synchronize()
            assert np.array_equal(ht.cpu().numpy(), plain[0]), (label, name)
            assert np.array_equal(hn.cpu().numpy(), plain[1]), (label, name)
            assert int(ws.count_nonzero()) == 0, (label, name)
    print(f"[{label}] {tally}", flush=True)
    tally.check(label)


def test_hinted_batched_workload():
    """B=64, gamma=4, V=128256, bf16, even requests T=0.7, odd greedy."""
    run_hints(synth.batched_chain(), 4, "hinted batched")


def test_hinted_mixed_small_span_and_f32():
    ci = synth.chain_inputs(16301, B=12, gamma=3, V=20000, dtype="f32", family="gauss",
                            draft_sigma=(0.3, 1.5), temperature=0.9, greedy_odd=True)
    run_hints(ci, 4, "hinted f32 small")


def test_hinted_invalid_and_extreme_requests():
    """Invalid temperatures, a bad draft token and gamma = 0 rows under every hint."""
    ci = synth.chain_inputs(16302, B=20, gamma=4, V=30000, dtype="bf16", family="zipf",
                            draft_sigma=0.8, temperature=1.0, greedy_odd=True)
    ci.temperature[3] = -1.0
    ci.temperature[6] = np.nan
    ci.draft_tokens[9, 2] = ci.V + 5
    run_hints(ci, 3, "hinted invalid")
    g0 = synth.chain_inputs(16303, B=9, gamma=0, V=5000, dtype="bf16", family="peaked",
                            temperature=1.0, greedy_odd=True)
    run_hints(g0, 3, "hinted gamma 0")


def test_hinted_hint_limits():
    """B at the hint's limit (256) and above it (the hint is ignored)."""
    for B in (sv.binding.SV_HINT_MAX_BATCH, sv.binding.SV_HINT_MAX_BATCH + 3):
        ci = synth.chain_inputs(16304 + B, B=B, gamma=2, V=3000, dtype="bf16", family="gauss",
                                draft_sigma=(0.3, 1.5), temperature=1.0, greedy_odd=True)
        run_hints(ci, 2, f"hinted B={B}")


def test_hint_must_be_host_data():
    ci = synth.chain_inputs(16305, B=4, gamma=2, V=1000, dtype="bf16", temperature=1.0)
    tgt = to_device_logits(ci.target, ci.dtype)
    drf = to_device_logits(ci.draft, ci.dtype)
    with pytest.raises(ValueError):
        sv.verify_chain(tgt, drf, to_device(ci.draft_tokens), to_device(ci.uniforms), to_device(ci.temperature),
                        sampling_hint=torch.ones(4, device="cuda"))
    with pytest.raises(ValueError):
        sv.verify_chain(tgt, drf, to_device(ci.draft_tokens), to_device(ci.uniforms), to_device(ci.temperature),
                        sampling_hint=[1, 0, 1])
