"""Exact enumeration of verification rounds (test helper, CPU only).

The law of the emitted tokens is computed exactly by enumerating the draft
tuples (weighted by the draft probabilities) and, for every uniform, one
representative point inside each interval on which the verifier's decision
is constant, weighted by the interval's length.  The verifier under test is
called as a black box at those points; if its decisions change anywhere
inside an interval other than where these breakpoints say, or its arithmetic
is wrong, the enumerated law stops matching the target distribution, which
is what the tests compare against (the lossless theorem).
"""
from __future__ import annotations

import itertools
from collections import defaultdict

import numpy as np


def breakpoints_accept(p_x: float, q_x: float) -> float:
    """Acceptance probability of a draft token, used only to place the
    representative uniforms and to weight them."""
    return 1.0 if q_x <= p_x else p_x / q_x


def enumerate_round(P, Q, decide, draft_law=None, accept_fn=None, residual_fn=None):
    """Exact law of one round with fixed rows.

    P : list of gamma+1 probability vectors (target rows)
    Q : list of gamma probability vectors (draft rows)
    decide(tokens, u) -> (emitted list, n) : the verifier under test
    draft_law : optional callable giving the probability of a draft tuple
                (defaults to independent draws from Q[i]).
    accept_fn, residual_fn : where the representative uniforms are placed
                (default: the acceptance probability and max(0, p - q));
                a planted-mistake test passes its planted rule here.
    Returns {emitted tuple: probability}."""
    gamma = len(Q)
    V = len(P[0])
    law = defaultdict(float)
    accept_fn = accept_fn or breakpoints_accept
    residual_fn = residual_fn or (lambda p, q: np.maximum(0.0, np.asarray(p) - np.asarray(q)))
    for tup in itertools.product(range(V), repeat=gamma):
        if draft_law is None:
            w_tup = float(np.prod([Q[i][tup[i]] for i in range(gamma)])) if gamma else 1.0
        else:
            w_tup = draft_law(tup)
        if w_tup == 0.0:
            continue
        taus = [accept_fn(P[i][tup[i]], Q[i][tup[i]]) for i in range(gamma)]
        for j in range(gamma + 1):
            pr = w_tup * float(np.prod(taus[:j])) * ((1.0 - taus[j]) if j < gamma else 1.0)
            if pr <= 0.0:
                continue
            u = np.zeros(gamma + 1)
            for i in range(j):
                u[i] = taus[i] / 2.0
            if j < gamma:
                u[j] = (1.0 + taus[j]) / 2.0
                for i in range(j + 1, gamma):
                    u[i] = 0.5
                w = np.asarray(residual_fn(P[j], Q[j]), dtype=np.float64)
                if not w.sum() > 0:
                    w = np.asarray(P[j])
            else:
                w = np.asarray(P[gamma])
            W = float(w.sum())
            F = np.concatenate([[0.0], np.cumsum(w) / W])
            for k in range(V):
                if w[k] <= 0.0:
                    continue
                u[gamma] = 0.5 * (F[k] + F[k + 1])
                emitted, _n = decide(tup, u.copy())
                law[tuple(int(t) for t in emitted)] += pr * w[k] / W
    return dict(law)


def slot_marginals(law, V, n_slots):
    """P(slot s reached) and P(token at slot s = x | slot s reached)."""
    reach = np.zeros(n_slots)
    joint = np.zeros((n_slots, V))
    for seq, pr in law.items():
        for s, t in enumerate(seq[:n_slots]):
            reach[s] += pr
            joint[s, t] += pr
    cond = np.where(reach[:, None] > 0, joint / np.maximum(reach[:, None], 1e-300), 0.0)
    return reach, cond


def expected_emitted(law):
    return sum(len(seq) * pr for seq, pr in law.items())


def total_variation(a: dict, b: dict) -> float:
    keys = set(a) | set(b)
    return 0.5 * sum(abs(a.get(k, 0.0) - b.get(k, 0.0)) for k in keys)
