"""Plain fp64 oracle of the verification step (chain, token tree, debug probs).

TEST INFRASTRUCTURE ONLY -- see the package docstring.  Float64 throughout;
bf16 inputs are widened exactly, fp32 uniforms and temperatures are promoted
exactly.  No blocking, fusion or reordering: each function follows the
algorithm as the pages state it.

Readings of points the pages leave open (each applied where noted below):

R1  accept test boundary: accept iff u <= tau (the close-reading notes,
    section 4, use "r_i <= min(1, p/q)"; one course page's listing uses a
    strict "<"; the two differ on a set of measure zero).
R2  tau: 1 when q(x) <= p(x), otherwise p(x)/q(x) (lecture 17 notes, section
    2.3, steps 2-3).  This equals min(1, p/q) whenever q > 0 and defines the
    q = 0 case as "accept".
R3  uniforms: u[b, i] for i < gamma is r_{i+1} of the accept test at draft
    position i; u[b, gamma] feeds the single final draw, residual or bonus.
R4  inverse CDF: C = cumsum(w) in vocabulary order, W = C[V-1]; the draw is
    the smallest k with C[k] > u*W, so zero-weight tokens are never drawn.  If
    rounding leaves no such k, the last index with w > 0 is returned.
R5  empty residual (W == 0 after a rejection; only reachable through
    rounding when p and q coincide): draw from p of that position instead.
R6  greedy (T == 0): argmax with the lowest index among equal maxima; at the
    first mismatch emit argmax p_i, if all match emit argmax p_{gamma+1}
    (close-reading notes, section 10).  Draft logits are not read.
R7  one temperature per request for both p and q (close-reading notes,
    section 3: the same decoding strategy on both sides).
R8  accepted count n in [0, gamma]; n + 1 tokens are emitted; the caller
    drops gamma - n cached positions.
R9  token tree: node 0 is the root (the last verified token), parents[0] =
    -1, 0 <= parents[i] < i (depth-first linearisation, ancestors first,
    lecture 17 notes section 4.3); children are visited in index order and
    the lowest-index child carrying the chosen token is taken.
R10 tree uniforms: u[b, n] is used for the draw at node n when n is visited.
R11 bad input makes a whole request invalid (count -1, tokens -1): a draft
    token or tree node token outside [0, V), a temperature that is negative,
    not finite, or positive but below the smallest normal float32, a sampling request with a uniform outside [0, 1), a
    malformed parent array, or a tree deeper than max_depth.
R12 MSS on a tree (T > 0): the children of node n are tested in index order;
    a child whose token repeats an earlier sibling's is skipped (only the
    first child carrying a token can be reached, as in R9).  The children are
    taken to be drawn without replacement from q_n = softmax(draft_n / T), so
    the j-th tested child is tested against q_n with the earlier tested
    children's tokens removed and renormalised (lecture 17 notes section 4.5,
    the fix that keeps MSS unbiased; exercise 7).
R13 MSS degenerate cases (reachable only through rounding or impossible
    draws): a rejection that leaves the residual without mass makes the node
    draw from p_n; once the tested children's tokens hold all of q_n's mass,
    the remaining children are not tested and the node draws from the
    current residual.
R14 MSS uniforms: accept_uniforms[b, j] is the test of node j as a child
    (entry 0 is never used); draw_uniforms[b, n] is the draw when the descent
    stops at node n.  A sampling request needs both in [0, 1) (entry 0 of
    accept_uniforms excepted).
R15 MSS trees allow at most 64 children per node (a contract limit of the
    library, not of the method); a tree with a wider node is invalid (R11).
R16 ragged rounds: request b drafts gammas[b] tokens in arrays padded to
    gamma; it is exactly the round of gammas[b] drafts (R3 with gamma =
    gammas[b]: its final draw takes uniforms[b, gammas[b]]), reads nothing
    past that length, and is invalid if gammas[b] is outside [0, gamma].
R17 consistent top-k (close-reading notes 02, section 5.4: the method stays
    exact when the same decoding rule is applied to p and q): a sampling
    request with top_k[b] = k filters every target and draft row it uses
    alike, keeping the logits >= the row's min(k, V)-th largest value
    (counted with multiplicity, so ties at that value are all kept) and
    setting the rest to -inf before the temperature softmax; verification
    then runs unchanged (R1-R8).  Greedy requests ignore k (the argmax is
    always kept).
R18 top-k contract limits of the library (not of the method): 1 <= k <= 128
    for a sampling request, and at most 256 kept logits per row (k plus the
    ties at the threshold); a request outside them is invalid (R11).
R19 top-p after top-k (the same rule on both sides, as R17): with top_p[b] =
    p in (0, 1], every row the top-k filter left is filtered again on its
    temperature softmax r over the kept logits: the threshold rises to the
    largest kept logit v whose mass M(v) = sum of r over the kept logits >= v
    reaches p, and the logits >= v stay (ties at v included).  p = 1 keeps
    the top-k set; p outside (0, 1] makes the request invalid.
R20 general consistent filter (the rules of R17 and R19 without the limits
    of R18): a sampling request may carry top_k[b] = k >= 1 (k >= V keeps the
    row whole), top_p[b] = p in (0, 1] (p = 1 cuts nothing), or both (top-k
    first, then top-p over what top-k kept); either array may be absent.
    k < 1, or p outside (0, 1], makes the request invalid (R11).  The top-p
    cut is a floating-point decision: its margin is min(M(v*) - p,
    p - M(v+)), v* the cut value and v+ the next larger kept value, which the
    parity tests treat like a decision's distance to its threshold.
"""
from __future__ import annotations

import dataclasses
from typing import List, Optional

import numpy as np


# ---------------------------------------------------------------------------
# inputs
# ---------------------------------------------------------------------------
def logits_to_f64(stored: np.ndarray, dtype: str) -> np.ndarray:
    """Exact widening: bf16 bit patterns (uint16) or float32 -> float64."""
    if dtype == "bf16":
        as_u32 = stored.astype(np.uint32) << np.uint32(16)
        return as_u32.view(np.float32).astype(np.float64)
    if dtype == "f32":
        return np.asarray(stored, dtype=np.float32).astype(np.float64)
    raise ValueError(f"unknown dtype {dtype!r}")


FLT_MIN = 1.1754943508222875e-38   # smallest normal float32


def _temperature_ok(t: float) -> bool:
    """R11: T must be 0 (greedy) or a finite positive normal float32."""
    return bool(np.isfinite(t)) and (t == 0.0 or t >= FLT_MIN)


# ---------------------------------------------------------------------------
# the distributions: p = softmax(l / T), q = softmax(d / T)
# ---------------------------------------------------------------------------
def softmax_t(logits_row: np.ndarray, T: float) -> np.ndarray:
    """Temperature softmax in fp64 (R7: the same T for target and draft)."""
    z = np.asarray(logits_row, dtype=np.float64) / np.float64(T)
    m = np.max(z)
    e = np.exp(z - m)
    return e / np.sum(e)


def log_sum_exp_t(logits_row: np.ndarray, T: float) -> float:
    """log sum_k exp(l_k / T) in fp64."""
    z = np.asarray(logits_row, dtype=np.float64) / np.float64(T)
    m = np.max(z)
    return float(m + np.log(np.sum(np.exp(z - m))))


# ---------------------------------------------------------------------------
# the two elementary steps
# ---------------------------------------------------------------------------
def accept_threshold(p_x: float, q_x: float) -> float:
    """tau = acceptance probability of a draft token x (R2).

    Lecture 17 notes section 2.3: accept outright when q(x) <= p(x), otherwise
    accept with probability p(x)/q(x)."""
    if q_x <= p_x:
        return 1.0
    return p_x / q_x


def accepts(u: float, tau: float) -> bool:
    """The accept test of one draft token (R1): accept iff u <= tau.  The
    close-reading notes (section 4, the full algorithm) accept draft i when
    r_i <= min(1, p(x)/q(x)), equality included."""
    return u <= tau


def residual_weights(p: np.ndarray, q: np.ndarray) -> np.ndarray:
    """Unnormalised residual max(0, p - q) (lecture 17 notes section 2.3 step 4;
    close-reading notes section 5.1)."""
    return np.maximum(0.0, p - q)


def inverse_cdf_draw(w: np.ndarray, u: float):
    """Draw a token from weights w with the uniform u (R4).

    Returns (k, margin) where margin = distance of u from the nearer of the two
    CDF values bracketing k: min(|u - F[k-1]|, |u - F[k]|), F = C / W."""
    C = np.cumsum(np.asarray(w, dtype=np.float64))
    W = C[-1]
    t = np.float64(u) * W
    k = int(np.searchsorted(C, t, side="right"))
    if k >= len(C):
        k = int(np.flatnonzero(np.asarray(w) > 0)[-1])
    lo = 0.0 if k == 0 else C[k - 1] / W
    hi = C[k] / W
    margin = float(min(abs(u - lo), abs(u - hi)))
    return k, margin


# ---------------------------------------------------------------------------
# chain verification (Algorithm 1)
# ---------------------------------------------------------------------------
@dataclasses.dataclass
class Decision:
    """One decision taken by the oracle, kept for parity accounting."""
    kind: str           # "accept" | "draw" | "greedy"
    position: int       # draft position i (accept), row of the draw, or -1
    u: float            # the uniform used (nan for greedy)
    threshold: float    # tau for accept tests, nan otherwise
    outcome: int        # 1/0 for accept tests, token for draws / greedy
    margin: float       # |u - tau| or the draw's CDF margin; inf for greedy


@dataclasses.dataclass
class ChainResult:
    out_tokens: np.ndarray        # [B, gamma+1] int32, -1 padded
    num_accepted: np.ndarray      # [B] int32, -1 => invalid request
    decisions: List[List[Decision]]


def chain_distributions(target_f64: np.ndarray, draft_f64: Optional[np.ndarray], T: float):
    """p_1..p_{gamma+1} and q_1..q_gamma of one sampling request (T > 0)."""
    P = [softmax_t(target_f64[i], T) for i in range(target_f64.shape[0])]
    Q = [softmax_t(draft_f64[i], T) for i in range(draft_f64.shape[0])]
    return P, Q


def _request_invalid(tokens: np.ndarray, u: np.ndarray, T: float, V: int) -> bool:
    if not _temperature_ok(T):
        return True
    if np.any(tokens < 0) or np.any(tokens >= V):
        return True
    if T > 0.0:
        uu = np.asarray(u, dtype=np.float64)
        if not np.all(np.isfinite(uu)) or np.any(uu < 0.0) or np.any(uu >= 1.0):
            return True
    return False


def chain_decide_request(P, Q, target_f64, tokens, u, T):
    """Accept/reject loop of one request (close-reading notes section 4,
    acceptance stage; lecture 17 notes section 2.4 steps 3-4).

    P, Q  : lists of fp64 probability rows (sampling) -- unused when T == 0
    target_f64 : [gamma+1, V] fp64 logits (used for the greedy argmax)
    Returns (emitted tokens, n, decisions)."""
    gamma = len(tokens)
    decisions: List[Decision] = []
    emitted: List[int] = []
    if T == 0.0:
        # R6: greedy verification reduces to argmax equality
        for i in range(gamma):
            a = int(np.argmax(target_f64[i]))
            decisions.append(Decision("greedy", i, float("nan"), float("nan"), a, float("inf")))
            if int(tokens[i]) != a:
                return emitted + [a], i, decisions
            emitted.append(int(tokens[i]))
        a = int(np.argmax(target_f64[gamma]))
        decisions.append(Decision("greedy", gamma, float("nan"), float("nan"), a, float("inf")))
        return emitted + [a], gamma, decisions

    for i in range(gamma):
        x = int(tokens[i])
        tau = accept_threshold(P[i][x], Q[i][x])
        ui = float(u[i])
        ok = accepts(ui, tau)                              # R1
        decisions.append(Decision("accept", i, ui, tau, int(ok), abs(ui - tau)))
        if ok:
            emitted.append(x)
            continue
        w = residual_weights(P[i], Q[i])
        if not np.sum(w) > 0.0:                            # R5
            w = P[i]
        k, margin = inverse_cdf_draw(w, float(u[gamma]))   # R3
        decisions.append(Decision("draw", i, float(u[gamma]), float("nan"), k, margin))
        return emitted + [k], i, decisions
    # every draft accepted: bonus token from p_{gamma+1}
    k, margin = inverse_cdf_draw(P[gamma], float(u[gamma]))
    decisions.append(Decision("draw", gamma, float(u[gamma]), float("nan"), k, margin))
    return emitted + [k], gamma, decisions


def verify_chain(target: np.ndarray, draft: Optional[np.ndarray], draft_tokens: np.ndarray,
                 uniforms: np.ndarray, temperature: np.ndarray, dtype: str,
                 requests=None) -> ChainResult:
    """Chain verification of a batch.

    target [B, gamma+1, V], draft [B, gamma, V] (bf16 bits or float32),
    draft_tokens [B, gamma] int, uniforms [B, gamma+1] float32,
    temperature [B] float32.  `requests` optionally restricts the work to a
    subset of request indices (the others are left at -1)."""
    B, G1, V = target.shape
    gamma = G1 - 1
    out = np.full((B, gamma + 1), -1, dtype=np.int32)
    nacc = np.full(B, -1, dtype=np.int32)
    decisions: List[List[Decision]] = [[] for _ in range(B)]
    todo = range(B) if requests is None else requests
    for b in todo:
        T = float(np.float32(temperature[b]))
        toks = np.asarray(draft_tokens[b], dtype=np.int64)
        u = np.asarray(uniforms[b], dtype=np.float32)
        if _request_invalid(toks, u, T, V):
            continue
        tgt = logits_to_f64(target[b], dtype)
        if T > 0.0:
            drf = logits_to_f64(draft[b], dtype)
            P, Q = chain_distributions(tgt, drf, T)
        else:
            P, Q = None, None
        emitted, n, dec = chain_decide_request(P, Q, tgt, toks, u, T)
        out[b, :len(emitted)] = emitted
        nacc[b] = n
        decisions[b] = dec
    return ChainResult(out, nacc, decisions)


@dataclasses.dataclass
class RaggedChainResult:
    out_tokens: np.ndarray        # [B, gamma+1] int32, -1 padded
    num_accepted: np.ndarray      # [B] int32, -1 => invalid request
    accept_prob: np.ndarray       # [B, gamma] float64: tau of each test taken, -1 elsewhere
    decisions: List[List[Decision]]


def verify_chain_ragged(target: np.ndarray, draft: Optional[np.ndarray], draft_tokens: np.ndarray,
                        uniforms: np.ndarray, temperature: np.ndarray, gammas: np.ndarray,
                        dtype: str, requests=None) -> RaggedChainResult:
    """Chain verification with a draft length per request (R16).

    The arrays are padded to gamma = target.shape[1] - 1.  Request b with
    g = gammas[b] is the round of g drafts: its tests use draft_tokens[b, :g]
    and uniforms[b, :g] against target rows 0..g-1 and draft rows 0..g-1, and
    its final draw (residual or bonus from target row g) uses uniforms[b, g].
    Nothing past g is read.  accept_prob[b, i] is tau of the test at position
    i when that test is taken (greedy: 1 if the draft equals the argmax, else
    0), and -1 for positions not tested; over draft tokens x ~ q its mean is
    sum_x min(p, q), the position's acceptance rate (lecture 17 notes section
    2.3; close-reading notes section 5.1), so the taus of a round give an
    unbiased acceptance estimate for choosing the next round's length."""
    B, G1, V = target.shape
    gamma = G1 - 1
    out = np.full((B, gamma + 1), -1, dtype=np.int32)
    nacc = np.full(B, -1, dtype=np.int32)
    acc = np.full((B, gamma), -1.0, dtype=np.float64)
    decisions: List[List[Decision]] = [[] for _ in range(B)]
    todo = range(B) if requests is None else requests
    for b in todo:
        g = int(gammas[b])
        if not 0 <= g <= gamma:
            continue
        T = float(np.float32(temperature[b]))
        toks = np.asarray(draft_tokens[b, :g], dtype=np.int64)
        u = np.asarray(uniforms[b, :g + 1], dtype=np.float32)
        if _request_invalid(toks, u, T, V):
            continue
        tgt = logits_to_f64(target[b, :g + 1], dtype)
        if T > 0.0:
            drf = logits_to_f64(draft[b, :g], dtype)
            P, Q = chain_distributions(tgt, drf, T)
        else:
            P, Q = None, None
        emitted, n, dec = chain_decide_request(P, Q, tgt, toks, u, T)
        out[b, :len(emitted)] = emitted
        nacc[b] = n
        for d in dec:
            if d.kind == "accept":
                acc[b, d.position] = d.threshold
            elif d.kind == "greedy" and d.position < g:
                acc[b, d.position] = 1.0 if int(toks[d.position]) == d.outcome else 0.0
        decisions[b] = dec
    return RaggedChainResult(out, nacc, acc, decisions)


# ---------------------------------------------------------------------------
# consistent top-k (R17, R18)
# ---------------------------------------------------------------------------
TOPK_MAX = 128
TOPK_MAX_KEPT = 256


def topk_filter(row_f64: np.ndarray, k: int):
    """R17: keep the logits >= the min(k, V)-th largest value of the row (ties
    included), -inf elsewhere.  Returns (filtered row, kept count)."""
    row = np.asarray(row_f64, dtype=np.float64)
    V = row.shape[0]
    kk = min(int(k), V)
    thr = np.sort(row)[V - kk]            # ascending order: the kk-th largest
    keep = row >= thr
    return np.where(keep, row, -np.inf), int(np.count_nonzero(keep))


def topp_filter(filtered_row: np.ndarray, p: float, T: float):
    """R19: on a row the top-k filter left (-inf elsewhere), keep the logits
    >= the largest kept value v with M(v) >= p, where M(v) is the
    temperature-softmax mass of the kept logits >= v.  Returns (filtered
    row, kept count)."""
    row = np.asarray(filtered_row, dtype=np.float64)
    kept = np.isfinite(row)
    if p < 1.0:
        r = softmax_t(row, T)
        best = -np.inf
        for v in row[kept]:
            if r[row >= v].sum() >= p and v > best:
                best = v
        if np.isfinite(best):
            kept = kept & (row >= best)
    return np.where(kept, row, -np.inf), int(np.count_nonzero(kept))


def topp_cut(filtered_row: np.ndarray, p: float, T: float):
    """R19/R20 by sorting (a library sort as a step): the kept (finite)
    values in descending order, their temperature-softmax masses summed value
    by value (equal values together), and the first value whose cumulative
    mass reaches p.  Returns (cut value, margin); (-inf, inf) when p >= 1 or
    nothing is kept, i.e. nothing is cut."""
    row = np.asarray(filtered_row, dtype=np.float64)
    fin = np.isfinite(row)
    if p >= 1.0 or not fin.any():
        return -np.inf, np.inf
    r = softmax_t(row, T)
    vals, mass = row[fin], r[fin]
    order = np.argsort(-vals, kind="stable")
    vals, mass = vals[order], mass[order]
    starts = np.concatenate(([0], 1 + np.nonzero(vals[1:] != vals[:-1])[0]))
    cum = np.cumsum(np.add.reduceat(mass, starts))
    j = min(int(np.searchsorted(cum, p, side="left")), len(cum) - 1)
    below = cum[j - 1] if j > 0 else 0.0
    return float(vals[starts[j]]), float(min(cum[j] - p, p - below))


@dataclasses.dataclass
class FilteredChainResult(ChainResult):
    cut_margin: np.ndarray = None   # [B] smallest top-p cut margin of the request's rows (inf: none)


def filtered_distributions(tgt_f64: np.ndarray, drf_f64: Optional[np.ndarray], T: float,
                           k: Optional[int], p: Optional[float]):
    """R20 on one request: every target and draft row filtered alike (top-k,
    then top-p), then the temperature softmax.  Returns (P, Q, smallest cut
    margin)."""
    margin = np.inf

    def filt(row):
        nonlocal margin
        f = row
        if k is not None:
            f, _ = topk_filter(f, k)
        if p is not None:
            v, m = topp_cut(f, p, T)
            margin = min(margin, m)
            f = np.where(f >= v, f, -np.inf)
        return f

    ft = np.array([filt(r) for r in tgt_f64])
    fd = np.array([filt(r) for r in drf_f64]) if drf_f64 is not None and len(drf_f64) else \
        np.zeros((0, tgt_f64.shape[1]))
    P, Q = chain_distributions(ft, fd, T)
    return P, Q, margin


def filter_params(b: int, top_k, top_p):
    """R20: (valid, k, p) of request b; k or p is None when its array is
    absent or it cuts nothing."""
    k = p = None
    if top_k is not None:
        k = int(top_k[b])
        if k < 1:
            return False, None, None
    if top_p is not None:
        p = float(np.float32(top_p[b]))
        if not 0.0 < p <= 1.0:
            return False, None, None
        if p >= 1.0:
            p = None
    return True, k, p


def verify_chain_filtered(target: np.ndarray, draft: Optional[np.ndarray], draft_tokens: np.ndarray,
                          uniforms: np.ndarray, temperature: np.ndarray, dtype: str,
                          top_k: Optional[np.ndarray] = None, top_p: Optional[np.ndarray] = None,
                          requests=None) -> FilteredChainResult:
    """Chain verification with p and q filtered alike by top-k and/or top-p
    over the whole vocabulary (R20); otherwise as verify_chain."""
    B, G1, V = target.shape
    gamma = G1 - 1
    out = np.full((B, gamma + 1), -1, dtype=np.int32)
    nacc = np.full(B, -1, dtype=np.int32)
    margins = np.full(B, np.inf)
    decisions: List[List[Decision]] = [[] for _ in range(B)]
    todo = range(B) if requests is None else requests
    for b in todo:
        T = float(np.float32(temperature[b]))
        toks = np.asarray(draft_tokens[b], dtype=np.int64)
        u = np.asarray(uniforms[b], dtype=np.float32)
        if _request_invalid(toks, u, T, V):
            continue
        tgt = logits_to_f64(target[b], dtype)
        if T > 0.0:
            ok, k, p = filter_params(b, top_k, top_p)
            if not ok:
                continue
            drf = logits_to_f64(draft[b], dtype) if gamma > 0 else None
            P, Q, margins[b] = filtered_distributions(tgt, drf, T, k, p)
        else:
            P, Q = None, None
        emitted, n, dec = chain_decide_request(P, Q, tgt, toks, u, T)
        out[b, :len(emitted)] = emitted
        nacc[b] = n
        decisions[b] = dec
    return FilteredChainResult(out, nacc, decisions, margins)


def verify_chain_topk(target: np.ndarray, draft: Optional[np.ndarray], draft_tokens: np.ndarray,
                      uniforms: np.ndarray, temperature: np.ndarray, top_k: np.ndarray,
                      dtype: str, requests=None, top_p: Optional[np.ndarray] = None) -> ChainResult:
    """Chain verification with p and q both filtered to their top-k logits
    (R17, R18), then, with top_p, to their top-p mass (R19); otherwise as
    verify_chain."""
    B, G1, V = target.shape
    gamma = G1 - 1
    out = np.full((B, gamma + 1), -1, dtype=np.int32)
    nacc = np.full(B, -1, dtype=np.int32)
    decisions: List[List[Decision]] = [[] for _ in range(B)]
    todo = range(B) if requests is None else requests
    for b in todo:
        T = float(np.float32(temperature[b]))
        toks = np.asarray(draft_tokens[b], dtype=np.int64)
        u = np.asarray(uniforms[b], dtype=np.float32)
        if _request_invalid(toks, u, T, V):
            continue
        tgt = logits_to_f64(target[b], dtype)
        if T > 0.0:
            k = int(top_k[b])
            if not 1 <= k <= TOPK_MAX:
                continue
            ft = [topk_filter(r, k) for r in tgt]
            fd = [topk_filter(r, k) for r in logits_to_f64(draft[b], dtype)] if gamma > 0 else []
            if max(c for _, c in ft + fd) > TOPK_MAX_KEPT:
                continue
            if top_p is not None:
                pp = float(np.float32(top_p[b]))
                if not 0.0 < pp <= 1.0:
                    continue
                ft = [topp_filter(r, pp, T) for r, _ in ft]
                fd = [topp_filter(r, pp, T) for r, _ in fd]
            P, Q = chain_distributions(np.array([r for r, _ in ft]),
                                       np.array([r for r, _ in fd]).reshape(gamma, V), T)
        else:
            P, Q = None, None
        emitted, n, dec = chain_decide_request(P, Q, tgt, toks, u, T)
        out[b, :len(emitted)] = emitted
        nacc[b] = n
        decisions[b] = dec
    return ChainResult(out, nacc, decisions)


# ---------------------------------------------------------------------------
# token tree verification
# ---------------------------------------------------------------------------
@dataclasses.dataclass
class TreeResult:
    out_tokens: np.ndarray      # [B, max_depth+1] int32, -1 padded
    out_path: np.ndarray        # [B, max_depth+1] int32 accepted node ids, -1 padded
    num_accepted: np.ndarray    # [B] int32, -1 => invalid request
    decisions: List[List[Decision]]


def tree_node_depths(parents: np.ndarray) -> Optional[np.ndarray]:
    """Depth of every node, or None when the parent array is malformed (R9)."""
    N = len(parents)
    if N < 1 or int(parents[0]) != -1:
        return None
    depth = np.zeros(N, dtype=np.int64)
    for i in range(1, N):
        p = int(parents[i])
        if p < 0 or p >= i:
            return None
        depth[i] = depth[p] + 1
    return depth


def _node_softmax(cache, key, logits_row, dtype, T):
    """softmax_t of a node's row, memoised in `cache` (a dict, or None) under
    `key`: the same logits give the same distribution, so a caller verifying
    one batch of trees under many uniform sets computes each row once."""
    if cache is not None and key in cache:
        return cache[key]
    p = softmax_t(logits_to_f64(logits_row, dtype), T)
    if cache is not None:
        cache[key] = p
    return p


def verify_tree(logits: np.ndarray, node_tokens: np.ndarray, parents: np.ndarray,
                uniforms: np.ndarray, temperature: np.ndarray, dtype: str,
                max_depth: int, requests=None, dist_cache=None) -> TreeResult:
    """Tree verification of a batch (lecture 17 notes section 4.4 VerifyGreedy
    for T == 0, section 4.5 naive sampling for T > 0).

    Starting at the root: choose c = argmax p_n (greedy) or draw c from p_n
    with u[b, n] (naive sampling); if a child of n carries c, accept that
    child and continue from it, otherwise emit c and stop.  At a leaf the
    chosen token is the extra token.  `dist_cache` (optional dict) keeps the
    node distributions across calls on the same logits and temperatures."""
    B, N, V = logits.shape
    L1 = max_depth + 1
    out = np.full((B, L1), -1, dtype=np.int32)
    path_out = np.full((B, L1), -1, dtype=np.int32)
    nacc = np.full(B, -1, dtype=np.int32)
    decisions: List[List[Decision]] = [[] for _ in range(B)]
    todo = range(B) if requests is None else requests
    for b in todo:
        T = float(np.float32(temperature[b]))
        par = np.asarray(parents[b], dtype=np.int64)
        tok = np.asarray(node_tokens[b], dtype=np.int64)
        u = np.asarray(uniforms[b], dtype=np.float32)
        depth = tree_node_depths(par)
        if depth is None or not _temperature_ok(T):
            continue
        if np.any(depth > max_depth):
            continue
        if N > 1 and (np.any(tok[1:] < 0) or np.any(tok[1:] >= V)):
            continue
        if T > 0.0:
            uu = u.astype(np.float64)
            if not np.all(np.isfinite(uu)) or np.any(uu < 0.0) or np.any(uu >= 1.0):
                continue
        node = 0
        path: List[int] = []
        dec: List[Decision] = []
        while True:
            if T == 0.0:
                c = int(np.argmax(logits_to_f64(logits[b, node], dtype)))
                dec.append(Decision("greedy", node, float("nan"), float("nan"), c, float("inf")))
            else:
                p = _node_softmax(dist_cache, (b, node, "p", T), logits[b, node], dtype, T)
                c, margin = inverse_cdf_draw(p, float(u[node]))
                dec.append(Decision("draw", node, float(u[node]), float("nan"), c, margin))
            nxt = -1
            for j in range(node + 1, N):           # children in index order (R9)
                if int(par[j]) == node and int(tok[j]) == c:
                    nxt = j
                    break
            if nxt < 0:
                break
            path.append(nxt)
            node = nxt
        emitted = [int(tok[j]) for j in path] + [c]
        out[b, :len(emitted)] = emitted
        path_out[b, :len(path)] = path
        nacc[b] = len(path)
        decisions[b] = dec
    return TreeResult(out, path_out, nacc, decisions)


# ---------------------------------------------------------------------------
# multi-step speculative sampling on a token tree (MSS)
# ---------------------------------------------------------------------------
def mss_thresholds(p: np.ndarray, proposals):
    """Multi-step speculative sampling at one node along the path on which
    every proposal is rejected (lecture 17 notes section 4.5,
    VerifyStochastic; exercise 6).

    p is the target distribution at the node; proposals is the list of
    (token x_j, q_j) in test order, q_j being the distribution x_j was drawn
    from.  The residual starts as r_1 = p.  Proposal j is accepted with
    probability tau_j = min(1, r_j(x_j) / q_j(x_j)) (R2); on rejection the
    residual becomes r_{j+1} = norm(max(0, r_j - q_j)).

    Returns (taus, residuals): tau_j for each proposal reached, and r_{j+1}
    after each rejection.  The lists stop early where a rejection has
    probability zero (tau_j == 1), and residuals[j] is None where a rejection
    leaves no residual mass (R13)."""
    r = np.asarray(p, dtype=np.float64)
    taus, residuals = [], []
    for x, q in proposals:
        tau = accept_threshold(float(r[x]), float(q[x]))
        taus.append(tau)
        if tau >= 1.0:
            break
        w = residual_weights(r, q)
        W = float(w.sum())
        if W <= 0.0:
            residuals.append(None)
            break
        r = w / W
        residuals.append(r)
    return taus, residuals


def mss_node(p: np.ndarray, proposals, u_accept, u_draw: float):
    """One node's MSS decision with the caller's uniforms: the first proposal
    j with u_accept[j] <= tau_j is accepted; if none is, the token is drawn
    from the last residual with u_draw (R4), or from p where the residual is
    empty (R13).  Returns (accepted index or -1, token, decisions)."""
    taus, residuals = mss_thresholds(p, proposals)
    dec: List[Decision] = []
    for j, tau in enumerate(taus):
        u = float(u_accept[j])
        ok = accepts(u, tau)
        dec.append(Decision("accept", j, u, tau, int(ok), abs(u - tau)))
        if ok:
            return j, int(proposals[j][0]), dec
    w = p if not residuals else residuals[-1]
    if w is None:
        w = p
    c, margin = inverse_cdf_draw(w, u_draw)
    dec.append(Decision("draw", -1, float(u_draw), float("nan"), c, margin))
    return -1, c, dec


def mss_proposals(q: np.ndarray, tokens):
    """Children drawn without replacement from q, tested in order (R12): the
    j-th child's distribution q_j is q with the tokens of the earlier children
    removed and renormalised (lecture 17 notes section 4.5: the fix that
    keeps MSS unbiased for sampled children; exercise 7).  Stops where the
    earlier children hold all of q's mass (R13)."""
    proposals = []
    qj = np.asarray(q, dtype=np.float64)
    for x in tokens:
        proposals.append((int(x), qj))
        rest = qj.copy()
        rest[x] = 0.0
        s = float(rest.sum())
        if s <= 0.0:
            break
        qj = rest / s
    return proposals


def tree_children(par: np.ndarray, tok: np.ndarray, node: int):
    """Children of `node` in index order, skipping a child whose token repeats
    an earlier sibling's (R12).  Returns (node ids, tokens)."""
    ids, seen = [], set()
    for j in range(node + 1, len(par)):
        if int(par[j]) == node and int(tok[j]) not in seen:
            ids.append(j)
            seen.add(int(tok[j]))
    return ids, [int(tok[j]) for j in ids]


MSS_MAX_CHILDREN = 64


def verify_tree_mss(logits: np.ndarray, draft_logits: np.ndarray, node_tokens: np.ndarray,
                    parents: np.ndarray, accept_uniforms: np.ndarray, draw_uniforms: np.ndarray,
                    temperature: np.ndarray, dtype: str, max_depth: int,
                    requests=None, dist_cache=None) -> TreeResult:
    """Tree verification by multi-step speculative sampling (lecture 17 notes
    section 4.5, VerifyStochastic with the children sampled without
    replacement; section 4.4 VerifyGreedy for T == 0).

    At node n with target p_n and draft q_n = softmax(draft_logits[n] / T)
    (the distribution n's children were drawn from), the children are tested
    in index order as in mss_node, child j with accept_uniforms[b, j].  An
    accepted child becomes the next node; if every child is rejected, or n
    has none, the token drawn with draw_uniforms[b, n] is emitted and the
    descent stops.  Greedy requests descend by argmax as in verify_tree.
    `dist_cache` (optional dict) keeps the node distributions across calls on
    the same logits and temperatures."""
    B, N, V = logits.shape
    L1 = max_depth + 1
    out = np.full((B, L1), -1, dtype=np.int32)
    path_out = np.full((B, L1), -1, dtype=np.int32)
    nacc = np.full(B, -1, dtype=np.int32)
    decisions: List[List[Decision]] = [[] for _ in range(B)]
    todo = range(B) if requests is None else requests
    for b in todo:
        T = float(np.float32(temperature[b]))
        par = np.asarray(parents[b], dtype=np.int64)
        tok = np.asarray(node_tokens[b], dtype=np.int64)
        depth = tree_node_depths(par)
        if depth is None or not _temperature_ok(T) or np.any(depth > max_depth):
            continue
        if N > 1 and (np.any(tok[1:] < 0) or np.any(tok[1:] >= V)):
            continue
        if N > 1 and np.bincount(par[1:], minlength=N).max() > MSS_MAX_CHILDREN:    # R15
            continue
        ua = np.asarray(accept_uniforms[b], dtype=np.float32).astype(np.float64)
        ud = np.asarray(draw_uniforms[b], dtype=np.float32).astype(np.float64)
        if T > 0.0:
            used = np.concatenate([ua[1:], ud])
            if not np.all(np.isfinite(used)) or np.any(used < 0.0) or np.any(used >= 1.0):
                continue
        node = 0
        path: List[int] = []
        dec: List[Decision] = []
        while True:
            if T == 0.0:
                c = int(np.argmax(logits_to_f64(logits[b, node], dtype)))
                dec.append(Decision("greedy", node, float("nan"), float("nan"), c, float("inf")))
                nxt = -1
                for j in range(node + 1, N):
                    if int(par[j]) == node and int(tok[j]) == c:
                        nxt = j
                        break
            else:
                p = _node_softmax(dist_cache, (b, node, "p", T), logits[b, node], dtype, T)
                ids, toks = tree_children(par, tok, node)
                props = []
                if ids:
                    q = _node_softmax(dist_cache, (b, node, "q", T), draft_logits[b, node], dtype, T)
                    props = mss_proposals(q, toks)
                ids = ids[:len(props)]
                j, c, d = mss_node(p, props, [ua[i] for i in ids], float(ud[node]))
                dec.extend(d)
                nxt = ids[j] if j >= 0 else -1
            if nxt < 0:
                break
            path.append(nxt)
            node = nxt
        emitted = [int(tok[j]) for j in path] + [c]
        out[b, :len(emitted)] = emitted
        path_out[b, :len(path)] = path
        nacc[b] = len(path)
        decisions[b] = dec
    return TreeResult(out, path_out, nacc, decisions)


# ---------------------------------------------------------------------------
# tree attention mask and depth positions
# ---------------------------------------------------------------------------
@dataclasses.dataclass
class TreeMaskResult:
    mask: np.ndarray        # [B, N, N] bool: node i may attend to node j
    depth: np.ndarray       # [B, N] int32 edges from the root, -1 => invalid request
    tree_depth: np.ndarray  # [B] int32 depth of the deepest node, -1 => invalid request


def tree_attention_mask(parents: np.ndarray, max_depth: int) -> TreeMaskResult:
    """Topology-aware causal mask and depth positions of a depth-first
    linearised token tree (lecture 17 notes section 4.3, tree-parallel
    decoding: steps 2 and 3, and the remark that positions follow depth;
    exercise 5).

    Row i allows node i itself and every node on its path to the root, the
    root included, and nothing else of the tree: a node placed earlier in the
    linear order on another branch stays hidden.  The verified prefix before
    the root is visible to every row and is not part of the mask.  Nodes at
    equal depth share a position offset, depth(i) being the number of edges
    from the root.  A malformed parent array (R9) or a node deeper than
    max_depth makes the request invalid (R11): all-false rows, depth -1."""
    parents = np.asarray(parents, dtype=np.int64)
    B, N = parents.shape
    mask = np.zeros((B, N, N), dtype=bool)
    depth = np.full((B, N), -1, dtype=np.int32)
    tree_depth = np.full(B, -1, dtype=np.int32)
    for b in range(B):
        d = tree_node_depths(parents[b])
        if d is None or np.any(d > max_depth):
            continue
        for i in range(N):
            j = i
            while j >= 0:          # node i, then each ancestor up to the root
                mask[b, i, j] = True
                j = int(parents[b, j])
        depth[b] = d
        tree_depth[b] = int(d.max())
    return TreeMaskResult(mask, depth, tree_depth)


# ---------------------------------------------------------------------------
# debug probabilities
# ---------------------------------------------------------------------------
@dataclasses.dataclass
class ProbsResult:
    p_at_draft: np.ndarray      # [B, gamma]
    q_at_draft: np.ndarray      # [B, gamma]
    residual_mass: np.ndarray   # [B, gamma] = sum_k max(0, p_i(k) - q_i(k))
    target_lse: np.ndarray      # [B, gamma+1] log sum_k exp(l_k / T)
    draft_lse: np.ndarray       # [B, gamma]


def probs_debug(target: np.ndarray, draft: np.ndarray, draft_tokens: np.ndarray,
                temperature: np.ndarray, dtype: str, requests=None) -> ProbsResult:
    """For every draft position i < gamma regardless of where verification
    stops: p_i(x~_i), q_i(x~_i), the residual mass sum_k max(0, p_i - q_i)
    (= 1 - sum_k min(p_i, q_i), close-reading notes section 5.1) and the
    log-normalisers.  Requests with T == 0 (or invalid T) are NaN; a token
    outside [0, V) gives NaN p/q at that position."""
    B, G1, V = target.shape
    gamma = G1 - 1
    nan = np.float64("nan")
    pa = np.full((B, gamma), nan)
    qa = np.full((B, gamma), nan)
    rm = np.full((B, gamma), nan)
    lt = np.full((B, gamma + 1), nan)
    ld = np.full((B, gamma), nan)
    todo = range(B) if requests is None else requests
    for b in todo:
        T = float(np.float32(temperature[b]))
        if not (_temperature_ok(T) and T > 0.0):
            continue
        tgt = logits_to_f64(target[b], dtype)
        drf = logits_to_f64(draft[b], dtype)
        for i in range(gamma + 1):
            lt[b, i] = log_sum_exp_t(tgt[i], T)
        for i in range(gamma):
            P = softmax_t(tgt[i], T)
            Q = softmax_t(drf[i], T)
            ld[b, i] = log_sum_exp_t(drf[i], T)
            rm[b, i] = float(np.sum(residual_weights(P, Q)))
            x = int(draft_tokens[b, i])
            if 0 <= x < V:
                pa[b, i] = P[x]
                qa[b, i] = Q[x]
    return ProbsResult(pa, qa, rm, lt, ld)
