"""GPU parity of spec_probs_debug: p(x), q(x) and the residual mass within 1e-5
relative of the fp64 oracle (residual: |d| <= 1e-5 * beta + 1e-7)."""
import numpy as np
import pytest
import torch

import oracle
import synth
import rejection_sampling_verify_15_amd as sv
from parity import assert_shared_workspace_zero, to_device, to_device_logits

pytestmark = pytest.mark.gpu


def check_probs(ci, label):
    tgt = to_device_logits(ci.target, ci.dtype)
    drf = to_device_logits(ci.draft, ci.dtype)
    out = sv.probs_debug(tgt, drf, to_device(ci.draft_tokens.astype(np.int32)),
                         to_device(ci.temperature.astype(np.float32)))
    assert_shared_workspace_zero(label)
    got = {k: v.cpu().numpy().astype(np.float64) for k, v in out.items()}
    ref = oracle.probs_debug(ci.target, ci.draft, ci.draft_tokens, ci.temperature, ci.dtype)
    for k, rv in (("p_at_draft", ref.p_at_draft), ("q_at_draft", ref.q_at_draft)):
        g = got[k]
        assert np.array_equal(np.isnan(g), np.isnan(rv)), (label, k)
        ok = ~np.isnan(rv)
        rel = np.abs(g[ok] - rv[ok]) / np.maximum(np.abs(rv[ok]), 1e-30)
        assert (rel <= 1e-5).all(), (label, k, rel.max())
    g, rv = got["residual_mass"], ref.residual_mass
    ok = ~np.isnan(rv)
    assert np.array_equal(np.isnan(g), np.isnan(rv))
    assert (np.abs(g[ok] - rv[ok]) <= 1e-5 * np.abs(rv[ok]) + 1e-7).all(), label
    for k, rv in (("target_lse", ref.target_lse), ("draft_lse", ref.draft_lse)):
        g = got[k]
        ok = ~np.isnan(rv)
        assert np.array_equal(np.isnan(g), np.isnan(rv))
        assert (np.abs(g[ok] - rv[ok]) <= 1e-5 * np.maximum(1.0, np.abs(rv[ok]))).all(), (label, k)
    print(f"[{label}] max rel p {np.nanmax(np.abs(got['p_at_draft'] - ref.p_at_draft) / ref.p_at_draft):.2e}",
          flush=True)


def test_probs_small_mixed():
    ci = synth.chain_inputs(201, B=10, gamma=4, V=20000, dtype="bf16", family="peaked",
                            draft_sigma=(0.3, 2.0), temperature=0.7, greedy_odd=True)
    ci.draft_tokens[1, 2] = 99999        # out of range -> NaN p/q there
    check_probs(ci, "small mixed")


def test_probs_f32_scalar_path():
    ci = synth.chain_inputs(202, B=6, gamma=3, V=9999, dtype="f32", family="gauss",
                            draft_sigma=1.0, temperature=1.3)
    check_probs(ci, "f32 V=9999")


def test_probs_batched_config():
    check_probs(synth.batched_chain(), "batched")


def test_probs_deep_config_sampled_requests():
    ci = synth.deep_chain(B=48)
    check_probs(ci, "deep B=48")
