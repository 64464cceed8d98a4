"""The seeded input generators: determinism, bf16 rounding, draft sampling law."""
import math

import numpy as np
import torch

import synth


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    x = (rng.standard_normal(200000) * 10).astype(np.float32)
    x[:4] = [1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -(1.0 + 2 ** -8), 0.0]   # ties to even
    ours = synth.bf16_round_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert (ours == ref).all()
    back = synth.bf16_bits_as_float32(ours)
    np.testing.assert_array_equal(back, torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_generators_are_deterministic():
    a = synth.chain_inputs(5, B=3, gamma=2, V=1000, family="peaked", draft_sigma=(0.3, 2.0),
                           temperature=0.7, greedy_odd=True)
    b = synth.chain_inputs(5, B=3, gamma=2, V=1000, family="peaked", draft_sigma=(0.3, 2.0),
                           temperature=0.7, greedy_odd=True)
    for f in ("target", "draft", "draft_tokens", "uniforms", "temperature"):
        assert np.array_equal(getattr(a, f), getattr(b, f))
    assert a.temperature.tolist() == [np.float32(0.7), 0.0, np.float32(0.7)]


def test_uniform_grid():
    u = synth.uniforms(np.random.default_rng(1), (1000, 9))
    assert u.dtype == np.float32 and (u >= 0).all() and (u < 1).all()
    k = u.astype(np.float64) * 2 ** 24
    assert np.array_equal(k, np.round(k))


def test_peaked_rows_have_boosted_entries():
    x = synth.peaked_logits(np.random.default_rng(2), 4, 32000)
    assert x.shape == (4, 32000)
    # 320 boosted entries per row: their mean sits about 8 above the rest
    for r in range(4):
        top = np.sort(x[r])[-320:]
        assert top.mean() > 8.0


def test_gumbel_max_draws_follow_q():
    """Draft tokens are samples of softmax(d / T)."""
    rng = np.random.default_rng(3)
    d = np.array([[[0.3, -1.0, 2.0, 0.0, -0.5]]], dtype=np.float32)
    n = 40000
    drafts = np.broadcast_to(d, (n, 1, 5)).copy()
    T = np.full(n, 0.8, np.float32)
    toks = synth.sample_draft_tokens(rng, drafts, "f32", T)
    z = d[0, 0].astype(np.float64) / 0.8
    q = np.exp(z - z.max()); q /= q.sum()
    for k in range(5):
        obs = (toks[:, 0] == k).sum()
        sd = math.sqrt(n * q[k] * (1 - q[k]))
        assert abs(obs - n * q[k]) < 4.5 * sd


def test_tree_is_depth_first():
    ti = synth.tree_inputs(seed=9, B=4, N=64, V=300, max_depth=8)
    for b in range(ti.B):
        par = ti.parents[b]
        assert par[0] == -1 and all(0 <= par[i] < i for i in range(1, ti.N))
        # preorder: every subtree occupies a contiguous index range
        size = np.ones(ti.N, dtype=int)
        for i in range(ti.N - 1, 0, -1):
            size[par[i]] += size[i]
        for i in range(1, ti.N):
            p = par[i]
            assert p < i < p + size[p]
