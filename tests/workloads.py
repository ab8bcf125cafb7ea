"""Seeded synthetic inputs for draft-tree verification.

This module only *generates* inputs: draft distributions, the draft tree built
from them, target logits, attention Q/K/V and the caller's uniforms.  It holds
none of the verification arithmetic (no exit law, no sampling, no attention)
and imports neither the HIP binding nor the CPU oracle, so both sides can be
fed from it.

Workload shapes follow the pages' settings:

* Qwen3-shaped vocabulary V = 151936, head layouts 32/8 and 40/8 and 64/8
  with head_dim 128, budgets of 16/64/128/256 nodes and 15-16 draft positions
  ("Where Draft Trees Lose Target Mass", App. D.3 setup; "CAST", Sec. 2 and
  App. C "Candidate construction"; "Multi-Future Drafting", Sec. 5.1).
* Trees are the top-B prefixes of a product of per-position draft
  distributions, enumerated best first ("CAST" App. C; tie-break toward
  shorter prefixes, then lexicographic rank order, "CAST" proof of Thm. 1),
  or for the mixture workload the top-B distinct prefixes under the best-mode
  score built with the merged heap ("Multi-Future Drafting" Eq. 2 and App. B).
* Stand-in statement: the pages measure on chat/code/math benchmarks with
  trained drafters and real targets.  None of those prompts, datasets or
  weights is used; these seeded arrays take only their shapes and value
  structure (peaked drafts, a few tokens of coverage per round, two-future
  targets).

Node 0 is the root (parents[0] = -1) and the other nodes follow the builder's
pop order, which is topological.  B counts the root: logits have B rows.
bf16 values are stored as uint16 bit patterns, rounded to nearest even.
"""
from __future__ import annotations

import hashlib
import heapq
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np

V_QWEN = 151936

# RNG streams: np.random.default_rng([config_id, request, stream, ...])
S_DRAFT, S_TARGET, S_MODES, S_Q, S_K, S_V, S_UNIF, S_ROOT = 1, 2, 3, 4, 5, 6, 7, 8


# --------------------------------------------------------------------------
# small numeric helpers (input generation only)
# --------------------------------------------------------------------------
def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (nearest even); returns uint16 bit patterns."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    rounded = u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return (rounded >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _softmax64(x: np.ndarray) -> np.ndarray:
    """Draft-side softmax used only to score candidate prefixes."""
    x = np.asarray(x, dtype=np.float64)
    m = x.max(axis=-1, keepdims=True)
    e = np.exp(x - m)
    return e / e.sum(axis=-1, keepdims=True)


def _rng(*key: int) -> np.random.Generator:
    return np.random.default_rng(list(key))


def digest(a: np.ndarray) -> str:
    return hashlib.sha256(np.ascontiguousarray(a).tobytes()).hexdigest()


# --------------------------------------------------------------------------
# tree builders (draft side)
# --------------------------------------------------------------------------
def _top_tokens(q: np.ndarray, K: int) -> tuple[np.ndarray, np.ndarray]:
    """Per position: the K most likely tokens (ties to smaller token id) and their log-probs."""
    L, V = q.shape
    K = min(K, V)
    order = np.argsort(-q, axis=1, kind="stable")[:, :K]
    logq = np.log(np.take_along_axis(q, order, axis=1))
    return order.astype(np.int64), logq


def best_first_tree(q: np.ndarray, n_nodes: int) -> tuple[np.ndarray, np.ndarray]:
    """Root plus the top-(n_nodes-1) prefixes of a product of per-position
    distributions q[j] (j = 0..L-1 is draft position j+1), best first.

    Successor scheme ("Multi-Future Drafting" App. B, with one mode): popping a
    prefix whose last token has rank k pushes its next sibling (rank k+1) and
    its first child (rank 0 at the next position).  Keys are (-log score,
    depth, rank sequence), so ties go to shorter prefixes, then lexicographic
    rank order.  Only each position's n_nodes most likely tokens can appear in
    the top-n_nodes set, so the universe is restricted to them.
    Returns parents, tokens (int32 [n_nodes]); tokens[0] is filled by the caller.
    """
    L, V = q.shape
    toks, logq = _top_tokens(q, n_nodes)
    K = toks.shape[1]
    parents = [-1]
    tokens = [0]
    node_of: dict[tuple, int] = {(): 0}
    heap = [(-logq[0, 0], 1, (0,), 0.0)] if L > 0 else []
    while heap and len(parents) < n_nodes:
        negs, d, ranks, _ = heapq.heappop(heap)
        idx = len(parents)
        node_of[ranks] = idx
        parents.append(node_of[ranks[:-1]])
        tokens.append(int(toks[d - 1, ranks[-1]]))
        base = -negs - logq[d - 1, ranks[-1]]
        if ranks[-1] + 1 < K:                               # next sibling
            sib = ranks[:-1] + (ranks[-1] + 1,)
            heapq.heappush(heap, (-(base + logq[d - 1, ranks[-1] + 1]), d, sib, 0.0))
        if d < L:                                           # first child
            heapq.heappush(heap, (-(-negs + logq[d, 0]), d + 1, ranks + (0,), 0.0))
    return np.asarray(parents, np.int32), np.asarray(tokens, np.int32)


def merged_heap_tree(qs: np.ndarray, n_nodes: int, log_prior: np.ndarray | None = None
                     ) -> tuple[np.ndarray, np.ndarray]:
    """Root plus the top-(n_nodes-1) distinct prefixes under the best-mode score
    s(v) = max_k [log pi_k + sum_j log q_{k,j}(v_j)] ("Multi-Future Drafting",
    Eq. 2), by the merged heap of its App. B: entries (k, v) keyed by
    s_k(v); popping (k, v) adds node v unless present and pushes v's
    successors under mode k either way.

    qs: [K][L][V] per-mode per-position draft distributions.
    """
    Km, L, V = qs.shape
    if log_prior is None:
        log_prior = np.full(Km, -np.log(Km))
    per_mode = [_top_tokens(qs[k], n_nodes) for k in range(Km)]
    Kt = per_mode[0][0].shape[1]
    parents = [-1]
    tokens = [0]
    node_of: dict[tuple, int] = {(): 0}
    heap = []
    for k in range(Km):
        toks, logq = per_mode[k]
        heapq.heappush(heap, (-(log_prior[k] + logq[0, 0]), 1, (0,), k))
    while heap and len(parents) < n_nodes:
        negs, d, ranks, k = heapq.heappop(heap)
        toks, logq = per_mode[k]
        seq = tuple(int(toks[j, ranks[j]]) for j in range(d))
        if seq not in node_of:
            node_of[seq] = len(parents)
            parents.append(node_of[seq[:-1]])
            tokens.append(seq[-1])
        s = -negs
        if ranks[-1] + 1 < Kt:
            heapq.heappush(heap, (-(s - logq[d - 1, ranks[-1]] + logq[d - 1, ranks[-1] + 1]), d,
                                  ranks[:-1] + (ranks[-1] + 1,), k))
        if d < L:
            heapq.heappush(heap, (-(s + logq[d, 0]), d + 1, ranks + (0,), k))
    return np.asarray(parents, np.int32), np.asarray(tokens, np.int32)


def depths_of(parents: np.ndarray) -> np.ndarray:
    d = np.zeros(len(parents), np.int64)
    for i in range(1, len(parents)):
        d[i] = d[parents[i]] + 1
    return d


def chain_tree(n_nodes: int, V: int, rng: np.random.Generator) -> tuple[np.ndarray, np.ndarray]:
    parents = np.arange(-1, n_nodes - 1, dtype=np.int32)
    tokens = rng.integers(0, V, size=n_nodes).astype(np.int32)
    return parents, tokens


def star_tree(n_nodes: int, V: int, rng: np.random.Generator) -> tuple[np.ndarray, np.ndarray]:
    parents = np.zeros(n_nodes, np.int32)
    parents[0] = -1
    tokens = np.concatenate([[0], rng.choice(V, size=n_nodes - 1, replace=False)]).astype(np.int32)
    return parents, tokens


def random_tree(n_nodes: int, V: int, rng: np.random.Generator, max_children: int | None = None
                ) -> tuple[np.ndarray, np.ndarray]:
    """Random recursive tree (parents[i] uniform on 0..i-1), distinct sibling tokens."""
    parents = np.empty(n_nodes, np.int32)
    parents[0] = -1
    tokens = np.empty(n_nodes, np.int32)
    tokens[0] = rng.integers(0, V)
    used: dict[int, set] = {}
    for i in range(1, n_nodes):
        while True:
            p = int(rng.integers(0, i))
            if max_children is None or len(used.get(p, ())) < max_children:
                break
        s = used.setdefault(p, set())
        if len(s) >= V:
            raise ValueError("vocabulary too small for this tree")
        while True:
            t = int(rng.integers(0, V))
            if t not in s:
                break
        s.add(t)
        parents[i] = p
        tokens[i] = t
    return parents, tokens


# --------------------------------------------------------------------------
# workload container
# --------------------------------------------------------------------------
@dataclass
class Workload:
    name: str
    config_id: int
    R: int
    B: int
    V: int
    dtype: str                 # "f32" or "bf16": logits and attention inputs
    logits: np.ndarray         # [R][B][V] float32, or uint16 bf16 bits
    parents: np.ndarray        # [R][B] int32
    tokens: np.ndarray         # [R][B] int32
    uniforms: np.ndarray       # [R][n][2] float32, values k * 2^-24
    Hq: int
    Hkv: int
    D: int
    P: int
    inv_temperature: float = 1.0
    q: np.ndarray | None = None   # [R][B][Hq][D]
    k: np.ndarray | None = None   # [R][Hkv][P+B][D]
    v: np.ndarray | None = None
    meta: dict = field(default_factory=dict)

    @property
    def scale(self) -> float:
        return 1.0 / float(np.sqrt(self.D))

    @property
    def n_draws(self) -> int:
        return int(self.uniforms.shape[1])

    def digests(self) -> dict:
        out = {}
        for name in ("logits", "parents", "tokens", "uniforms", "q", "k", "v"):
            a = getattr(self, name)
            if a is not None:
                out[name] = digest(a)[:16]
        return out


def uniforms_for(cfg: int, req: int, n: int) -> np.ndarray:
    """n pairs (u1, u2) with u = k * 2^-24, k uniform on {0..2^24-1}: exact in f32 and f64."""
    k = _rng(cfg, req, S_UNIF).integers(0, 1 << 24, size=(n, 2))
    return (k.astype(np.float64) * 2.0 ** -24).astype(np.float32)


def _normal_store(rng: np.random.Generator, shape, dtype: str, scale: float = 1.0) -> np.ndarray:
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if scale != 1.0:
        x *= np.float32(scale)
    return x if dtype == "f32" else f32_to_bf16_bits(x)


def _pool_map(fn, items):
    """Map over independent seeded items on a few threads (numpy's generators
    and array arithmetic release the GIL); each item has its own seed, so the
    result does not depend on the number of threads."""
    items = list(items)
    workers = min(len(items), max(1, min(16, len(os.sched_getaffinity(0)))))
    if workers <= 1:
        return [fn(x) for x in items]
    with ThreadPoolExecutor(max_workers=workers) as ex:
        return list(ex.map(fn, items))


def make_attention(cfg: int, R: int, B: int, Hq: int, Hkv: int, D: int, P: int, dtype: str):
    """Q, K, V ~ N(0, 1) per request and kv head; cache rows P..P+B-1 are the tree nodes."""
    st = np.float32 if dtype == "f32" else np.uint16
    q = np.empty((R, B, Hq, D), st)
    k = np.empty((R, Hkv, P + B, D), st)
    v = np.empty((R, Hkv, P + B, D), st)

    def fill(item):
        r, g = item
        if g < 0:
            q[r] = _normal_store(_rng(cfg, r, S_Q), (B, Hq, D), dtype)
        else:
            k[r, g] = _normal_store(_rng(cfg, r, S_K, g), (P + B, D), dtype)
            v[r, g] = _normal_store(_rng(cfg, r, S_V, g), (P + B, D), dtype)

    _pool_map(fill, [(r, g) for r in range(R) for g in range(-1, Hkv)])
    return q, k, v


# --------------------------------------------------------------------------
# the five named workloads
# --------------------------------------------------------------------------
def _peaked_draft(rng, L, V, sigma=4.0, peak=8.0, n_peak=8):
    ell = rng.standard_normal(size=(L, V)) * sigma
    top = np.argpartition(-ell, n_peak, axis=1)[:, :n_peak]
    np.put_along_axis(ell, top, np.take_along_axis(ell, top, axis=1) + peak, axis=1)
    return ell


def _request_tiny(cfg, r):
    V, L, B = 1000, 4, 16
    ell = _rng(cfg, r, S_DRAFT).standard_normal(size=(L, V)) * 3.0
    parents, tokens = best_first_tree(_softmax64(ell), B)
    tokens[0] = _rng(cfg, r, S_ROOT).integers(0, V)
    logits = _rng(cfg, r, S_TARGET).standard_normal(size=(B, V)) * 3.0
    for u in range(1, B):                       # drafted child tokens boosted by +4
        logits[parents[u], tokens[u]] += 4.0
    return parents, tokens, logits.astype(np.float32)


def _qwen_ell(cfg, r, L=16, V=V_QWEN):
    return _peaked_draft(_rng(cfg, r, S_DRAFT), L + 1, V)


def _request_qwen_peaked(cfg, r, B, L=16, V=V_QWEN):
    ell = _qwen_ell(cfg, r, L, V)
    parents, tokens = best_first_tree(_softmax64(ell[:L]), B)
    tokens[0] = _rng(cfg, r, S_ROOT).integers(0, V)
    d = depths_of(parents)
    noise = _rng(cfg, r, S_TARGET).standard_normal(size=(B, V), dtype=np.float32)
    logits = ell[d].astype(np.float32) + noise   # row of a depth-d node follows position d+1
    return parents, tokens, f32_to_bf16_bits(logits)


def _wide_ell(cfg, r, L=16, V=V_QWEN):
    rng = _rng(cfg, r, S_DRAFT)
    ell = rng.standard_normal(size=(L + 1, V)) * 4.0
    top = np.argpartition(-ell, 8, axis=1)[:, :8]
    np.put_along_axis(ell, top, 20.0 + rng.standard_normal(size=top.shape) * 0.5, axis=1)
    return ell


def _request_wide_zipf(cfg, r, B=128, L=16, V=V_QWEN):
    ell = _wide_ell(cfg, r, L, V)
    q = _softmax64(ell)
    parents, tokens = best_first_tree(q[:L], B)
    tokens[0] = _rng(cfg, r, S_ROOT).integers(0, V)
    d = depths_of(parents)
    order = np.argsort(-q, axis=1, kind="stable")[:, :8]       # draft top-8 per position
    trng = _rng(cfg, r, S_TARGET)
    zipf = (-1.1 * np.log(np.arange(1, V + 1, dtype=np.float64))).astype(np.float32)
    logits = np.empty((B, V), np.float32)
    for i in range(B):
        top8 = order[d[i]]
        rest = np.setdiff1d(np.arange(V), top8, assume_unique=False)
        rest = trng.permutation(rest)
        ranked = np.concatenate([top8, rest])                   # rank 1..V
        logits[i, ranked] = zipf
    return parents, tokens, f32_to_bf16_bits(logits)


def _mixture_ells(cfg, r, L=16, V=V_QWEN, K=8):
    """The K modes' position-wise draft logits of a mixture request and its
    two futures A, B."""
    mrng = _rng(cfg, r, S_MODES)
    A = mrng.choice(V, size=L + 1, replace=False)
    Bf = np.empty(L + 1, np.int64)
    for j in range(L + 1):                                      # B_j != A_j
        while True:
            t = int(mrng.integers(0, V))
            if t != A[j]:
                Bf[j] = t
                break
    futures = [A, A, A, Bf, Bf, Bf,
               mrng.integers(0, V, size=L + 1), mrng.integers(0, V, size=L + 1)]
    drng = _rng(cfg, r, S_DRAFT)
    ells = np.empty((K, L, V))
    for k in range(K):
        ell = _peaked_draft(drng, L, V)
        for j in range(L):
            ell[j, futures[k][j]] = ell[j].max() + 2.0
        ells[k] = ell
    return ells, A, Bf


def _request_mixture(cfg, r, B=256, L=16, V=V_QWEN, K=8):
    ells, A, Bf = _mixture_ells(cfg, r, L, V, K)
    qs = np.stack([_softmax64(ells[k]) for k in range(K)])
    parents, tokens = merged_heap_tree(qs, B)
    tokens[0] = _rng(cfg, r, S_ROOT).integers(0, V)
    # target: bimodal masses -> log -> bf16
    trng = _rng(cfg, r, S_TARGET)
    d = depths_of(parents)
    seqs = [()] * B
    for i in range(1, B):
        seqs[i] = seqs[parents[i]] + (int(tokens[i]),)
    logits = np.empty((B, V), np.float32)
    for i in range(B):
        bg = _softmax64(trng.standard_normal(size=V) * 3.0)
        s = seqs[i]
        on_a = all(s[j] == A[j] for j in range(len(s)))
        on_b = all(s[j] == Bf[j] for j in range(len(s)))
        if i == 0:
            p = 0.03 * bg
            p[A[0]] += 0.582
            p[Bf[0]] += 0.388
        elif on_a:
            p = 0.03 * bg
            p[A[d[i]]] += 0.97
        elif on_b:
            p = 0.03 * bg
            p[Bf[d[i]]] += 0.97
        else:
            p = bg
        with np.errstate(divide="ignore"):
            logits[i] = np.log(p).astype(np.float32)
    return parents, tokens, f32_to_bf16_bits(logits)


CONFIGS = {
    # name: (config id, R, B, V, dtype, Hq, Hkv, D, P)
    "tiny": (1, 1, 16, 1000, "f32", 4, 4, 64, 128),
    "qwen3_4b": (2, 1, 64, V_QWEN, "bf16", 32, 8, 128, 4096),
    "qwen3_8b_wide": (3, 1, 128, V_QWEN, "bf16", 32, 8, 128, 8192),
    "mixture": (4, 1, 256, V_QWEN, "bf16", 40, 8, 128, 16384),
    "batched": (5, 32, 64, V_QWEN, "bf16", 64, 8, 128, 32768),
}
CONFIG_ORDER = ["tiny", "qwen3_4b", "qwen3_8b_wide", "mixture", "batched"]

DESCRIPTIONS = {
    "tiny": "1 request, B=16 (depth<=4) best-first over 4 draft positions, V=1000 f32, "
            "4/4 heads D=64, P=128",
    "qwen3_4b": "1 request, B=64 best-first over 16 peaked draft positions, V=151936 bf16, "
                "32/8 heads D=128, P=4096",
    "qwen3_8b_wide": "1 request, B=128 wide best-first tree, Zipf(1.1) target ranks, "
                     "V=151936 bf16, 32/8 heads D=128, P=8192",
    "mixture": "1 request, B=256 merged-heap tree of 8 draft modes, bimodal target, "
               "V=151936 bf16, 40/8 heads D=128, P=16384",
    "batched": "32 requests x B=64 best-first trees, V=151936 bf16, 64/8 heads D=128, "
               "P=32768 per request",
}


def make_config(name: str, n_uniform: int = 4096, with_attention: bool = True,
                requests: int | None = None) -> Workload:
    """Build one of the five named workloads.  ``requests`` limits the batched
    workload to its first requests (each request is generated independently)."""
    cfg, R, B, V, dtype, Hq, Hkv, D, P = CONFIGS[name]
    if requests is not None:
        R = min(R, int(requests))
    par = np.empty((R, B), np.int32)
    tok = np.empty((R, B), np.int32)
    st = np.float32 if dtype == "f32" else np.uint16
    logits = np.empty((R, B, V), st)
    if name not in ("tiny", "qwen3_4b", "batched", "qwen3_8b_wide", "mixture"):
        raise KeyError(name)

    def request(r):
        if name == "tiny":
            p, t, lg = _request_tiny(cfg, r)
        elif name in ("qwen3_4b", "batched"):
            p, t, lg = _request_qwen_peaked(cfg, r, B)
        elif name == "qwen3_8b_wide":
            p, t, lg = _request_wide_zipf(cfg, r, B)
        else:
            p, t, lg = _request_mixture(cfg, r, B)
        if len(p) != B:
            raise RuntimeError(f"{name}: builder returned {len(p)} nodes, expected {B}")
        par[r], tok[r], logits[r] = p, t, lg

    _pool_map(request, range(R))
    uni = np.stack([uniforms_for(cfg, r, n_uniform) for r in range(R)])
    w = Workload(name, cfg, R, B, V, dtype, logits, par, tok, uni, Hq, Hkv, D, P)
    if with_attention:
        w.q, w.k, w.v = make_attention(cfg, R, B, Hq, Hkv, D, P, dtype)
    w.meta["description"] = DESCRIPTIONS[name]
    return w


def make_qwen_budget(B: int, n_uniform: int = 1) -> Workload:
    """The Qwen3-4B-shaped round at another node budget B (root included):
    the same seeds, draft rows and target recipe as "qwen3_4b" (which is B =
    64), the best-first tree cut at B nodes; logits only (no attention).  The
    node budgets 32 / 64 / 128 are those of the pages' verifier-stage
    comparison."""
    cfg, _, _, V, dtype, Hq, Hkv, D, P = CONFIGS["qwen3_4b"]
    p, t, lg = _request_qwen_peaked(cfg, 0, B)
    w = Workload(f"qwen3_4b_B{B}", cfg, 1, B, V, dtype, lg[None], p[None].astype(np.int32),
                 t[None].astype(np.int32), uniforms_for(cfg, 0, n_uniform)[None], Hq, Hkv, D, P)
    w.meta["description"] = f"1 request, B={B} best-first over 16 peaked draft positions, V={V} bf16"
    return w


def draft_rows(name: str, requests: int | None = None) -> np.ndarray:
    """The position-wise draft logits a named workload's trees were built from:
    [R][L][V], row j scoring the nodes of depth j + 1 (the drafter's rows for
    the exit-guided loss).  f32 for "tiny", bf16 bits otherwise.  The mixture
    workload has K draft modes rather than one row per position: KeyError."""
    cfg, R, B, V, dtype, *_ = CONFIGS[name]
    if requests is not None:
        R = min(R, int(requests))
    rows = []
    for r in range(R):
        if name == "tiny":
            rows.append(_rng(cfg, r, S_DRAFT).standard_normal(size=(4, V)) * 3.0)
        elif name in ("qwen3_4b", "batched"):
            rows.append(_qwen_ell(cfg, r)[:16])
        elif name == "qwen3_8b_wide":
            rows.append(_wide_ell(cfg, r)[:16])
        else:
            raise KeyError(f"{name} has no single position-wise drafter (see draft_rows_modes)")
    z = np.stack(rows).astype(np.float32)
    return z if dtype == "f32" else f32_to_bf16_bits(z)


def draft_rows_modes(name: str = "mixture") -> np.ndarray:
    """The K draft modes' position-wise logits of the mixture workload:
    [R][K][L][V] bf16 bits (mode k, row j scores depth j + 1)."""
    if name != "mixture":
        raise KeyError(name)
    cfg, R, *_ = CONFIGS[name]
    z = np.stack([_mixture_ells(cfg, r)[0] for r in range(R)]).astype(np.float32)
    return f32_to_bf16_bits(z)


def make_custom(name: str, *, R: int = 1, B: int = 16, V: int = 1000, dtype: str = "f32",
                tree: str = "random", Hq: int = 4, Hkv: int = 2, D: int = 64, P: int = 100,
                seed: int = 100, n_uniform: int = 256, logit_sigma: float = 3.0,
                child_boost: float = 4.0, with_attention: bool = True,
                inv_temperature: float = 1.0) -> Workload:
    """Small parity cases: random / chain / star / best-first trees over
    N(0, sigma^2) target logits with drafted children boosted."""
    par = np.empty((R, B), np.int32)
    tok = np.empty((R, B), np.int32)
    lgs = np.empty((R, B, V), np.float32)
    for r in range(R):
        rng = _rng(seed, r, S_DRAFT)
        if tree == "random":
            p, t = random_tree(B, V, rng)
        elif tree == "chain":
            p, t = chain_tree(B, V, rng)
        elif tree == "star":
            p, t = star_tree(B, V, rng)
        elif tree == "best_first":
            L = max(1, min(16, B - 1))
            p, t = best_first_tree(_softmax64(rng.standard_normal(size=(L, V)) * logit_sigma), B)
            t[0] = rng.integers(0, V)
        else:
            raise KeyError(tree)
        lg = _rng(seed, r, S_TARGET).standard_normal(size=(B, V)) * logit_sigma
        for u in range(1, B):
            lg[p[u], t[u]] += child_boost
        par[r], tok[r], lgs[r] = p, t, lg.astype(np.float32)
    logits = lgs if dtype == "f32" else f32_to_bf16_bits(lgs)
    uni = np.stack([uniforms_for(seed, r, n_uniform) for r in range(R)])
    w = Workload(name, 0, R, B, V, dtype, logits, par, tok, uni, Hq, Hkv, D, P,
                 inv_temperature=inv_temperature)
    if with_attention:
        w.q, w.k, w.v = make_attention(seed, R, B, Hq, Hkv, D, P, dtype)
    w.meta["description"] = f"custom {tree} tree R={R} B={B} V={V} {dtype}"
    return w
