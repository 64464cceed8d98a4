"""Seeded synthetic inputs for the speculative-decoding verification step.

This module only *produces* inputs: logits, draft tokens, per-position
uniforms, temperatures and token trees.  It holds none of the verification
arithmetic (no softmax, no accept test, no inverse-CDF draw), so that the fp64
oracle and the HIP library can both consume its output without sharing any
of the method's code.

Draft tokens must be genuine samples from the draft distribution q
(Leviathan et al., as restated in the CMU 15-779 lecture 17 notes, section
2.3: the lossless argument needs the draft token to be drawn from q).  They
are produced with the Gumbel-max construction -- argmax_k(d_k/T + G_k) with
G_k = -log(E_k), E_k ~ Exp(1) -- and tree children are drawn without
replacement with its top-k extension (lecture 17 notes, section 4.5: children
must be sampled, without replacement).  Neither construction appears in the
verifier.

bf16 values are produced by round-to-nearest-even of a float32 value and are
stored as raw uint16 bit patterns; the consumers convert them exactly.
Uniforms are k * 2**-24 for integer k in [0, 2**24): exact in fp32 and fp64,
and always in [0, 1).
"""
from __future__ import annotations

import dataclasses
import os
from concurrent.futures import ThreadPoolExecutor
from typing import Optional

import numpy as np

SEED_BASE = 15000
UNIFORM_BITS = 24

# Named workloads (sizes from the workload list of the verification step).
TOY = dict(B=4096, gamma=4, V=5)
SINGLE = dict(B=1, gamma=4, V=32000)
BATCHED = dict(B=64, gamma=4, V=128256)
DEEP = dict(B=256, gamma=8, V=151936)
TREE = dict(B=32, N=64, V=128256, max_depth=8)


# --------------------------------------------------------------------------
# primitive helpers (no verification arithmetic)
# --------------------------------------------------------------------------
def bf16_round_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit pattern (uint16), round to nearest, ties to even."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.shape, dtype=np.uint16)
    src = x.reshape(-1).view(np.uint32)
    dst = out.reshape(-1)
    step = 1 << 20
    n = src.size

    def work(i):
        u = src[i * step:(i + 1) * step]
        t = u >> np.uint32(16)
        t &= np.uint32(1)
        t += np.uint32(0x7FFF)
        t += u
        t >>= np.uint32(16)
        dst[i * step:(i + 1) * step] = t
    _run_blocks(work, (n + step - 1) // step)
    return out


def bf16_bits_as_float32(bits: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns to float32 (exact).  Used only to sample drafts."""
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)


def uniforms(rng: np.random.Generator, shape) -> np.ndarray:
    """U[0,1) values on the 2**-24 grid (exact in fp32)."""
    k = rng.integers(0, 1 << UNIFORM_BITS, size=shape, dtype=np.int64)
    return (k.astype(np.float64) * 2.0 ** -UNIFORM_BITS).astype(np.float32)


def gumbel(rng: np.random.Generator, shape) -> np.ndarray:
    e = rng.standard_exponential(size=shape, dtype=np.float32)
    np.maximum(e, np.float32(1e-38), out=e)
    return -np.log(e)


def _streams(seed: int, n: int):
    return [np.random.default_rng(s) for s in np.random.SeedSequence(seed).spawn(n)]


# Bulk generation runs on fixed blocks of rows, each with its own generator
# spawned from the stream's seed, so results do not depend on the number of
# worker threads.
ROWS_PER_BLOCK = 16
_THREADS = max(1, min(16, os.cpu_count() or 1))


def _block_rngs(rng: np.random.Generator, rows: int):
    nblk = (rows + ROWS_PER_BLOCK - 1) // ROWS_PER_BLOCK
    seeds = rng.integers(0, 2 ** 63 - 1, size=nblk, dtype=np.int64)
    return [np.random.default_rng(int(x)) for x in seeds]


def _run_blocks(fn, nblk: int):
    if nblk <= 1 or _THREADS == 1:
        for i in range(nblk):
            fn(i)
        return
    with ThreadPoolExecutor(_THREADS) as ex:
        list(ex.map(fn, range(nblk)))


def normal_rows(rng: np.random.Generator, rows: int, V: int, std: float = 1.0) -> np.ndarray:
    """float32 [rows, V] of N(0, std^2), generated block-parallel."""
    out = np.empty((rows, V), dtype=np.float32)
    gens = _block_rngs(rng, rows)

    def work(i):
        sl = out[i * ROWS_PER_BLOCK:(i + 1) * ROWS_PER_BLOCK]
        gens[i].standard_normal(out=sl, dtype=np.float32)
        if std != 1.0:
            sl *= np.float32(std)
    _run_blocks(work, len(gens))
    return out


def shuffle_rows(rng: np.random.Generator, x: np.ndarray) -> np.ndarray:
    """Independent uniform random permutation of every row of x (in place)."""
    gens = _block_rngs(rng, x.shape[0])

    def work(i):
        sl = x[i * ROWS_PER_BLOCK:(i + 1) * ROWS_PER_BLOCK]
        for r in range(sl.shape[0]):
            gens[i].shuffle(sl[r])
    _run_blocks(work, len(gens))
    return x


# --------------------------------------------------------------------------
# logit families
# --------------------------------------------------------------------------
def gaussian_logits(rng, rows: int, V: int, std: float = 1.0) -> np.ndarray:
    """i.i.d. N(0, std^2) logits, float32 [rows, V]."""
    return normal_rows(rng, rows, V, std)


def peaked_logits(rng, rows: int, V: int, std: float = 2.0, boost: float = 8.0,
                  frac: float = 0.01) -> np.ndarray:
    """N(0, std^2) logits with round(frac*V) distinct entries per row raised by
    `boost` (a confident head over a long tail)."""
    x = normal_rows(rng, rows, V, std)
    k = int(round(frac * V))
    if k > 0:
        for r in range(rows):
            idx = rng.choice(V, size=k, replace=False)
            x[r, idx] += np.float32(boost)
    return x


def zipf_logits(rng, rows: int, V: int, slope: float = 1.1,
                noise: float = 0.5) -> np.ndarray:
    """-slope*ln(rank) + N(0, noise^2), ranks permuted independently per row."""
    base = (-slope * np.log(np.arange(1, V + 1, dtype=np.float64))).astype(np.float32)
    x = normal_rows(rng, rows, V, noise)
    x += base[None, :]
    return shuffle_rows(rng, x)


FAMILIES = {"gauss": gaussian_logits, "peaked": peaked_logits, "zipf": zipf_logits}


# --------------------------------------------------------------------------
# chain inputs
# --------------------------------------------------------------------------
@dataclasses.dataclass
class ChainInputs:
    """One batch for the chain verification step.

    target : [B, gamma+1, V]  uint16 (bf16 bits) or float32
    draft  : [B, gamma,   V]  same dtype
    draft_tokens : [B, gamma] int32
    uniforms     : [B, gamma+1] float32, entries 0..gamma-1 feed the accept
                   tests, entry gamma feeds the final draw
    temperature  : [B] float32, 0 => greedy
    """
    target: np.ndarray
    draft: np.ndarray
    draft_tokens: np.ndarray
    uniforms: np.ndarray
    temperature: np.ndarray
    dtype: str
    B: int
    gamma: int
    V: int
    name: str = ""
    recipe: str = ""

    def fresh_uniforms(self, seed: int) -> np.ndarray:
        return uniforms(np.random.default_rng(seed), (self.B, self.gamma + 1))


def _as_dtype(x: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return bf16_round_bits(x)
    if dtype == "f32":
        return np.ascontiguousarray(x, dtype=np.float32)
    raise ValueError(dtype)


def _widen(stored: np.ndarray, dtype: str) -> np.ndarray:
    return bf16_bits_as_float32(stored) if dtype == "bf16" else stored


def sample_draft_tokens(rng, draft_stored: np.ndarray, dtype: str,
                        temperature: np.ndarray) -> np.ndarray:
    """x~_i ~ q_i = softmax(d_i / T) via Gumbel-max on the stored (rounded)
    draft logits; argmax of the draft logits for greedy (T == 0) requests."""
    B, G, V = draft_stored.shape
    out = np.empty((B, G), dtype=np.int32)
    seeds = rng.integers(0, 2 ** 63 - 1, size=B, dtype=np.int64)

    def work(b):
        d = _widen(draft_stored[b], dtype).astype(np.float32)
        t = float(temperature[b])
        if t > 0.0:
            keys = d / np.float32(t) + gumbel(np.random.default_rng(int(seeds[b])), d.shape)
            out[b] = np.argmax(keys, axis=1)
        else:
            out[b] = np.argmax(d, axis=1)
    _run_blocks(work, B)
    return out


def chain_inputs(seed: int, B: int, gamma: int, V: int, dtype: str = "bf16",
                 family: str = "peaked", draft_sigma=1.0, temperature=1.0,
                 greedy_odd: bool = False, name: str = "",
                 family_kwargs: Optional[dict] = None) -> ChainInputs:
    """Generic chain workload.

    draft_sigma : float, or (lo, hi) for a per-request U[lo, hi] noise scale.
    temperature : sampling temperature for sampling requests.
    greedy_odd  : odd-indexed requests run greedy (T = 0).
    """
    r_tgt, r_noise, r_tok, r_u, r_mode = _streams(seed, 5)
    fam = FAMILIES[family]
    kw = dict(family_kwargs or {})
    tgt = fam(r_tgt, B * (gamma + 1), V, **kw).reshape(B, gamma + 1, V)
    if isinstance(draft_sigma, tuple):
        sig = r_mode.uniform(draft_sigma[0], draft_sigma[1], size=B).astype(np.float32)
    else:
        sig = np.full(B, draft_sigma, dtype=np.float32)
    drf = normal_rows(r_noise, B * gamma, V).reshape(B, gamma, V)
    drf *= sig[:, None, None]
    drf += tgt[:, :gamma, :]
    T = np.full(B, temperature, dtype=np.float32)
    if greedy_odd:
        T[1::2] = 0.0
    target = _as_dtype(tgt.reshape(B, gamma + 1, V), dtype)
    del tgt
    draft = _as_dtype(drf, dtype)
    del drf
    toks = sample_draft_tokens(r_tok, draft, dtype, T) if gamma > 0 else \
        np.zeros((B, 0), dtype=np.int32)
    u = uniforms(r_u, (B, gamma + 1))
    recipe = (f"seed={seed} family={family} draft_sigma={draft_sigma} T={temperature} "
              f"greedy_odd={greedy_odd} dtype={dtype}")
    return ChainInputs(target, draft, toks, u, T, dtype, B, gamma, V, name, recipe)


def topk_draft_tokens(ci: ChainInputs, top_k, seed: int) -> np.ndarray:
    """Draft tokens of a draft model that decodes with top-k: Gumbel-max over
    the k largest stored draft logits of each row (k per request, clamped to
    [1, V]); argmax rows for greedy requests."""
    rng = np.random.default_rng(seed)
    out = np.empty((ci.B, ci.gamma), dtype=np.int32)
    for b in range(ci.B):
        d = _widen(ci.draft[b], ci.dtype).astype(np.float32)
        t = float(ci.temperature[b])
        for i in range(ci.gamma):
            if t > 0.0:
                k = min(max(int(top_k[b]), 1), ci.V)
                top = np.argpartition(-d[i], k - 1)[:k]
                keys = d[i, top] / np.float32(t) + gumbel(rng, (k,))
                out[b, i] = int(top[np.argmax(keys)])
            else:
                out[b, i] = int(np.argmax(d[i]))
    return out


def topp_draft_tokens(ci: ChainInputs, top_p, seed: int) -> np.ndarray:
    """Draft tokens of a draft model that decodes with top-p (nucleus)
    sampling over the whole vocabulary: the draft row's softmax at the
    request's temperature, its values sorted in descending order, the
    smallest prefix whose mass reaches p (every value equal to the last one
    kept), then a Gumbel-max draw among the kept logits; argmax rows for
    greedy requests."""
    rng = np.random.default_rng(seed)
    out = np.empty((ci.B, ci.gamma), dtype=np.int32)
    for b in range(ci.B):
        d = _widen(ci.draft[b], ci.dtype).astype(np.float64)
        t = float(ci.temperature[b])
        for i in range(ci.gamma):
            if t > 0.0:
                z = d[i] / t
                w = np.exp(z - z.max())
                w /= w.sum()
                order = np.argsort(-d[i], kind="stable")
                cum = np.cumsum(w[order])
                last = min(int(np.searchsorted(cum, float(np.float32(top_p[b])), side="left")), ci.V - 1)
                keep = d[i] >= d[i][order[last]]
                out[b, i] = int(np.argmax(np.where(keep, z + gumbel(rng, (ci.V,)), -np.inf)))
            else:
                out[b, i] = int(np.argmax(d[i]))
    return out


def toy_chain(seed: int = SEED_BASE + 1, B: int = 4096, gamma: int = 4, V: int = 5):
    """V=5 fp32 toy: target N(0,1), draft = target + N(0, 0.5^2), T = 1."""
    return chain_inputs(seed, B, gamma, V, dtype="f32", family="gauss",
                        draft_sigma=0.5, temperature=1.0, name="toy")


def single_chain(seed: int = SEED_BASE + 2, B: int = 1, gamma: int = 4, V: int = 32000):
    """B=1 bf16 peaked target, draft noise sigma 1.0, T = 1."""
    return chain_inputs(seed, B, gamma, V, dtype="bf16", family="peaked",
                        draft_sigma=1.0, temperature=1.0, name="single")


def batched_chain(seed: int = SEED_BASE + 3, B: int = 64, gamma: int = 4, V: int = 128256):
    """B=64 bf16 peaked target, per-request draft sigma ~ U[0.3, 2.0],
    even requests sample at T = 0.7, odd requests are greedy."""
    return chain_inputs(seed, B, gamma, V, dtype="bf16", family="peaked",
                        draft_sigma=(0.3, 2.0), temperature=0.7, greedy_odd=True,
                        name="batched")


def deep_chain(seed: int = SEED_BASE + 4, B: int = 256, gamma: int = 8, V: int = 151936):
    """B=256 gamma=8 bf16 Zipf-like target, draft noise sigma 0.8, T = 1."""
    return chain_inputs(seed, B, gamma, V, dtype="bf16", family="zipf",
                        draft_sigma=0.8, temperature=1.0, name="deep")


def replicated_pair_chain(seed: int, p_logits: np.ndarray, q_logits: np.ndarray,
                          B: int, gamma: int, temperature: float = 1.0) -> ChainInputs:
    """One (target, draft) logit pair repeated at every position of every request
    (float32), so that the per-position acceptance rate is one constant alpha.
    Draft tokens are sampled from q independently per position."""
    V = p_logits.shape[-1]
    r_tok, r_u = _streams(seed, 2)
    tgt = np.broadcast_to(np.asarray(p_logits, np.float32), (B, gamma + 1, V)).copy()
    drf = np.broadcast_to(np.asarray(q_logits, np.float32), (B, gamma, V)).copy()
    T = np.full(B, temperature, dtype=np.float32)
    toks = sample_draft_tokens(r_tok, drf, "f32", T)
    u = uniforms(r_u, (B, gamma + 1))
    return ChainInputs(tgt, drf, toks, u, T, "f32", B, gamma, V, "replicated",
                       f"seed={seed} replicated pair")


# --------------------------------------------------------------------------
# token trees
# --------------------------------------------------------------------------
@dataclasses.dataclass
class TreeInputs:
    """One batch for the token-tree verification step.

    logits      : [B, N, V] target logits, one row per node, depth-first order
    node_tokens : [B, N] int32 (entry 0, the root, is the last verified token)
    parents     : [B, N] int32, parents[:,0] = -1, 0 <= parents[:,i] < i
    uniforms    : [B, N] float32, one per node (used when the node is visited)
    temperature : [B] float32, 0 => greedy descent, > 0 => naive sampling
    draft_logits  : [B, N, V] draft logits of every node (the row its children
                    were drawn from), or None when not kept
    draw_uniforms : [B, N] float32, a second uniform per node, or None
    """
    logits: np.ndarray
    node_tokens: np.ndarray
    parents: np.ndarray
    uniforms: np.ndarray
    temperature: np.ndarray
    dtype: str
    B: int
    N: int
    V: int
    max_depth: int
    name: str = ""
    recipe: str = ""
    draft_logits: Optional[np.ndarray] = None
    draw_uniforms: Optional[np.ndarray] = None


def random_tree_shape(rng, N: int, max_depth: int, max_branch: int = 4):
    """Grow a tree of exactly N nodes (root included): repeatedly pick a random
    open node (depth < max_depth, fewer than max_branch children) and give it
    U{1..max_branch} more children, capped by its remaining branch capacity and
    by the node budget.  Returns creation-order parents and children lists."""
    parent = [-1]
    depth = [0]
    children = [[]]
    open_nodes = [0] if max_depth > 0 else []
    while len(parent) < N:
        if not open_nodes:
            raise RuntimeError("tree budget cannot be met under the depth cap")
        j = int(rng.integers(0, len(open_nodes)))
        n = open_nodes[j]
        room = max_branch - len(children[n])
        k = min(int(rng.integers(1, max_branch + 1)), room, N - len(parent))
        for _ in range(k):
            c = len(parent)
            parent.append(n)
            depth.append(depth[n] + 1)
            children.append([])
            children[n].append(c)
            if depth[c] < max_depth:
                open_nodes.append(c)
        if len(children[n]) >= max_branch:
            open_nodes.remove(n)
    return parent, children


def dfs_relabel(children):
    """Preorder (ancestors first) relabelling; children keep creation order."""
    order = []
    stack = [0]
    while stack:
        n = stack.pop()
        order.append(n)
        stack.extend(reversed(children[n]))
    new_id = {old: i for i, old in enumerate(order)}
    return order, new_id


def tree_parent_arrays(seed: int, B: int, N: int, max_depth: int, max_branch: int = 4,
                       dfs: bool = True) -> np.ndarray:
    """[B, N] int32 parent arrays of random trees grown by random_tree_shape:
    depth-first relabelled when dfs, else left in creation order (every
    parent still precedes its children, but sibling subtrees interleave)."""
    (r_shape,) = _streams(seed, 1)
    parents = np.empty((B, N), dtype=np.int32)
    for b in range(B):
        par_c, ch_c = random_tree_shape(r_shape, N, max_depth, max_branch)
        if not dfs:
            parents[b] = par_c
            continue
        _, new_id = dfs_relabel(ch_c)
        for old in range(N):
            parents[b, new_id[old]] = -1 if par_c[old] < 0 else new_id[par_c[old]]
    return parents


def tree_inputs(seed: int = SEED_BASE + 5, B: int = 32, N: int = 64, V: int = 128256,
                max_depth: int = 8, temperature: float = 0.0, dtype: str = "bf16",
                family: str = "peaked", draft_sigma: float = 1.0,
                max_branch: int = 4, name: str = "tree", keep_draft: bool = False) -> TreeInputs:
    """Token trees: random shape (<= max_depth, branching 1..max_branch),
    depth-first relabelled; per-node target logits from `family`; the children
    of each node are drawn without replacement from the draft softmax at that
    node (draft logits = node target logits + N(0, draft_sigma^2), T = 1).

    With keep_draft, every node's draft row is kept (rounded to dtype, and the
    children are drawn from exactly that rounded row), and a second uniform
    array is drawn; the target rows, shapes and first uniforms are the same
    as without it."""
    r_shape, r_tgt, r_noise, r_tok, r_u = _streams(seed, 5)
    fam = FAMILIES[family]
    parents = np.empty((B, N), dtype=np.int32)
    tokens = np.zeros((B, N), dtype=np.int32)
    logits32 = fam(r_tgt, B * N, V).reshape(B, N, V)
    stored = _as_dtype(logits32, dtype)
    del logits32
    draft = np.empty_like(stored) if keep_draft else None
    for b in range(B):
        par_c, ch_c = random_tree_shape(r_shape, N, max_depth, max_branch)
        order, new_id = dfs_relabel(ch_c)
        for old in range(N):
            parents[b, new_id[old]] = -1 if par_c[old] < 0 else new_id[par_c[old]]
        for old in order:
            kids = ch_c[old]
            n = new_id[old]
            if not kids and not keep_draft:
                continue
            row = _widen(stored[b, n], dtype).astype(np.float32)
            d = row + r_noise.standard_normal(V, dtype=np.float32) * np.float32(draft_sigma)
            if keep_draft:
                draft[b, n] = _as_dtype(d, dtype)
                d = _widen(draft[b, n], dtype).astype(np.float32)
            if not kids:
                continue
            keys = d + gumbel(r_tok, V)
            top = np.argpartition(-keys, len(kids) - 1)[:len(kids)]
            top = top[np.argsort(-keys[top], kind="stable")]
            for c_old, tok in zip(kids, top):
                tokens[b, new_id[c_old]] = int(tok)
    u = uniforms(r_u, (B, N))
    u2 = uniforms(r_u, (B, N)) if keep_draft else None
    T = np.full(B, temperature, dtype=np.float32)
    recipe = (f"seed={seed} family={family} draft_sigma={draft_sigma} T={temperature} "
              f"max_depth={max_depth} branch=1..{max_branch} dtype={dtype}"
              + (" draft rows kept" if keep_draft else ""))
    return TreeInputs(stored, tokens, parents, u, T, dtype, B, N, V, max_depth, name, recipe,
                      draft, u2)

