"""Pins of two oracle steps every other test leans on: the exact widening of
bf16 logits, and the accept test's boundary u = tau.

The widening is checked over all 65,536 bit patterns against torch's own
bfloat16 -> float64 conversion and against hand-decoded patterns, so a wrong
shift or a dropped sign cannot hide behind tests that widen both sides with
the same function.  The boundary is checked with probabilities whose ratio is
exactly representable: the close-reading notes (section 4, the full
algorithm) accept draft i when r_i <= min(1, p/q), equality included (R1).
Planted mistakes -- a wrong widening, a strict "<" -- must fail these pins.
CPU only.
"""
import numpy as np
import pytest
import torch

import oracle
from oracle import specverify_oracle as so


ALL_BF16 = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)


def torch_bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()


def widening_disagreements(widen) -> int:
    """Number of bit patterns where `widen` differs from torch (NaNs must stay NaN)."""
    got = widen(ALL_BF16, "bf16")
    ref = torch_bf16_to_f64(ALL_BF16)
    nan_ref = np.isnan(ref)
    bad = nan_ref != np.isnan(got)
    ok = ~nan_ref & ~np.isnan(got)
    bad[ok] |= (got[ok] != ref[ok]) | (np.signbit(got[ok]) != np.signbit(ref[ok]))
    return int(bad.sum())


def test_bf16_widening_equals_torch_on_every_pattern():
    assert widening_disagreements(oracle.logits_to_f64) == 0


@pytest.mark.parametrize("bits,value", [
    (0x3F80, 1.0), (0xBF80, -1.0), (0x4000, 2.0), (0x4049, 3.140625), (0xC2F7, -123.5),
    (0x7F7F, 3.3895313892515355e38),          # largest finite: (2 - 2^-7) * 2^127
    (0x0080, 2.0 ** -126),                    # smallest normal
    (0x0001, 2.0 ** -133),                    # smallest subnormal: 2^-7 * 2^-126
    (0x8001, -(2.0 ** -133)),
    (0x7F80, np.inf), (0xFF80, -np.inf),
])
def test_bf16_widening_hand_decoded(bits, value):
    got = oracle.logits_to_f64(np.array([bits], dtype=np.uint16), "bf16")[0]
    assert got == value


def test_bf16_widening_signed_zero_and_nan():
    z = oracle.logits_to_f64(np.array([0x0000, 0x8000], dtype=np.uint16), "bf16")
    assert z[0] == 0.0 and not np.signbit(z[0])
    assert z[1] == 0.0 and np.signbit(z[1])
    n = oracle.logits_to_f64(np.array([0x7FC0, 0xFFC1, 0x7F81], dtype=np.uint16), "bf16")
    assert np.isnan(n).all()


def test_bf16_widening_of_a_random_array_matches_the_generator_bits():
    """A seeded float32 array rounded to bf16 by torch, widened by the oracle,
    equals torch's own widening of the same tensor."""
    rng = np.random.default_rng(11)
    x = (rng.standard_normal((3, 5000)) * 7).astype(np.float32)
    t = torch.from_numpy(x).to(torch.bfloat16)
    bits = t.view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(oracle.logits_to_f64(bits, "bf16"), t.to(torch.float64).numpy())


def test_f32_widening_is_the_identity_on_float32_values():
    rng = np.random.default_rng(12)
    x = (rng.standard_normal(10000) * 50).astype(np.float32)
    x[:3] = [-np.inf, np.float32(1e-45), -0.0]
    got = oracle.logits_to_f64(x, "f32")
    assert got.dtype == np.float64
    np.testing.assert_array_equal(got, x.astype(np.float64))
    assert np.signbit(got[2])


WRONG_WIDENINGS = {
    "shift_by_15": lambda s, d: (s.astype(np.uint32) << np.uint32(15)).view(np.float32).astype(np.float64),
    "low_half": lambda s, d: s.astype(np.uint32).view(np.float32).astype(np.float64),
    "dropped_sign": lambda s, d: ((s.astype(np.uint32) & np.uint32(0x7FFF)) << np.uint32(16))
    .view(np.float32).astype(np.float64),
    "value_not_bits": lambda s, d: s.astype(np.float64),
    "float16_bits": lambda s, d: s.view(np.float16).astype(np.float64),
}


@pytest.mark.parametrize("name", sorted(WRONG_WIDENINGS))
def test_planted_wrong_widening_fails_the_pin(name):
    assert widening_disagreements(WRONG_WIDENINGS[name]) > 0


# ---------------------------------------------------------------------------
# R1: u == tau accepts, the next float above rejects
# ---------------------------------------------------------------------------
def boundary_rows():
    """p(x=0) = 1/4 and q(x=0) = 1/2, so tau = 1/2 exactly; a second position
    keeps the round going after an acceptance."""
    P = [np.array([0.25, 0.75]), np.array([0.5, 0.5]), np.array([0.5, 0.5])]
    Q = [np.array([0.5, 0.5]), np.array([0.5, 0.5])]
    return P, Q


def test_accept_boundary_u_equal_tau_accepts():
    P, Q = boundary_rows()
    assert so.accept_threshold(P[0][0], Q[0][0]) == 0.5
    u = np.array([0.5, 0.0, 0.25], dtype=np.float32)
    emitted, n, dec = oracle.chain_decide_request(P, Q, None, np.array([0, 1]), u, 1.0)
    assert dec[0].kind == "accept" and dec[0].threshold == 0.5 and dec[0].outcome == 1
    assert dec[0].margin == 0.0
    assert n >= 1 and emitted[0] == 0


def test_accept_boundary_next_float_rejects():
    P, Q = boundary_rows()
    above = np.nextafter(np.float32(0.5), np.float32(1.0))
    assert float(above) == 0.5 + 2.0 ** -24
    u = np.array([above, 0.0, 0.25], dtype=np.float32)
    emitted, n, dec = oracle.chain_decide_request(P, Q, None, np.array([0, 1]), u, 1.0)
    assert dec[0].outcome == 0 and n == 0
    # the residual max(0, p - q) = (0, 1/4) leaves token 1 only
    assert emitted == [1]


def test_accept_boundary_through_verify_chain_f32():
    """The same boundary reached from float32 logits: target row [0, 0] gives
    p = (1/2, 1/2) and draft row [0, -inf] gives q = (1, 0), both exact in
    fp64, so tau of token 0 is exactly 1/2."""
    tgt = np.array([[[0.0, 0.0], [0.0, 0.0]]], dtype=np.float32)
    drf = np.array([[[0.0, -np.inf]]], dtype=np.float32)
    T = np.ones(1, np.float32)
    for u0, accepted in ((0.5, True), (float(np.nextafter(np.float32(0.5), np.float32(1))), False),
                         (float(np.nextafter(np.float32(0.5), np.float32(0))), True)):
        u = np.array([[u0, 0.75]], dtype=np.float32)
        r = oracle.verify_chain(tgt, drf, np.zeros((1, 1), np.int32), u, T, "f32")
        assert r.decisions[0][0].threshold == 0.5
        assert bool(r.decisions[0][0].outcome) == accepted
        assert r.num_accepted[0] == (1 if accepted else 0)
        if not accepted:
            assert r.out_tokens[0, 0] == 1   # the residual's only token


def test_mss_accept_boundary_u_equal_tau():
    """The tree MSS test uses the same rule (R1 via R12)."""
    p = np.array([0.25, 0.75])
    q = np.array([0.5, 0.5])
    j, tok, dec = oracle.mss_node(p, [(0, q)], [0.5], 0.9)
    assert dec[0].threshold == 0.5 and j == 0 and tok == 0
    j, tok, dec = oracle.mss_node(p, [(0, q)], [0.5 + 2.0 ** -24], 0.9)
    assert j == -1 and tok == 1


def test_planted_strict_less_fails_the_boundary_pin(monkeypatch):
    monkeypatch.setattr(so, "accepts", lambda u, tau: u < tau)
    P, Q = boundary_rows()
    u = np.array([0.5, 0.0, 0.25], dtype=np.float32)
    _, n, dec = oracle.chain_decide_request(P, Q, None, np.array([0, 1]), u, 1.0)
    assert dec[0].outcome == 0 and n == 0   # the pin above would fail


def test_planted_strict_less_fails_the_verify_chain_pin(monkeypatch):
    monkeypatch.setattr(so, "accepts", lambda u, tau: u < tau)
    tgt = np.array([[[0.0, 0.0], [0.0, 0.0]]], dtype=np.float32)
    drf = np.array([[[0.0, -np.inf]]], dtype=np.float32)
    r = oracle.verify_chain(tgt, drf, np.zeros((1, 1), np.int32), np.array([[0.5, 0.75]], np.float32),
                            np.ones(1, np.float32), "f32")
    assert r.num_accepted[0] == 0
