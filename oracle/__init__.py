"""Plain fp64 CPU oracle for draft-tree verification -- TEST INFRASTRUCTURE.

Only the test suite, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product path (the HIP library and
its binding) never imports, links or executes anything here, and this package
imports nothing from the product.

The arithmetic lives in ``tev_oracle.c`` (plain loops, double precision,
optional OpenMP over independent rows); this module only marshals numpy
arrays.  Sources:

* "Where Draft Trees Lose Target Mass: Exit-Guided Speculative Decoding"
  (arXiv 2610.11750): Sec. 3 Eq. 1-2 (p_v, reach P), Sec. 3.1 Eq. 4 (A(v),
  rho, w), Lemma 1 Eq. 5, Sec. 3.2 Eq. 6 (coverage), Eq. 7 (residual law),
  App. B Algorithm 1 (TEV's two draws), Sec. 5 Eq. 14 (the exit-guided
  draft-tree loss, ``exit_loss``).
* "CAST" App. C "Candidate construction" and "Multi-Future Drafting" App. B
  (the best-first tree builder, ``build_tree``; the merged heap over several
  draft modes, ``build_tree_modes``).
* "CAST: Cost-Aware Speculative Trees from One-Pass Block Drafters"
  (arXiv 2610.00321): App. B Lemma 1 and App. C "Packed verification"
  (ancestor-only attention mask).

Parity pins live in ``tests/test_oracle_*.py``.  Every function here is pinned
(see those tests); none is "parity unpinned" except the exact index a given
uniform maps to, which no page prints and which follows from the inverse-CDF
reading together with the enumerated law.
"""
from __future__ import annotations

import ctypes
import heapq
import os
import subprocess
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "tev_oracle.c")
_LIB_PATH = os.path.join(_HERE, "_build", "liboracle.so")

F32, BF16, F64 = 0, 1, 2
_DTYPE_CODES = {"f32": F32, "bf16": BF16, "f64": F64}


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (-O2, IEEE semantics, OpenMP)."""
    os.makedirs(os.path.dirname(_LIB_PATH), exist_ok=True)
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        subprocess.check_call(
            ["gcc", "-std=c11", "-O2", "-fopenmp", "-fPIC", "-shared", "-Wall", "-Wextra",
             "-Werror", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build(force=True)
        lib = ctypes.CDLL(_LIB_PATH)
        vp, ip, dp = ctypes.c_void_p, ctypes.c_int, ctypes.c_double
        lib.oracle_exit_law.argtypes = [vp, ip, vp, vp, ip, ip, ip, dp, vp, vp, vp, vp, vp, ip]
        lib.oracle_sample.argtypes = [vp, ip, vp, vp, ip, ip, ip, dp, vp, vp, ip, vp, vp, vp, ip]
        lib.oracle_residual_cdf.argtypes = [vp, ip, vp, vp, ip, ip, ip, dp, vp]
        lib.oracle_predraw.argtypes = [vp, ip, vp, vp, ip, ip, ip, dp, vp, ip, vp, vp, vp, vp, vp, ip]
        lib.oracle_tree_attn.argtypes = [vp, vp, vp, ip, vp, ip, ip, ip, ip, ip, ip, dp, vp, vp,
                                         ctypes.c_int64, ip]
        lib.oracle_check_tree.argtypes = [vp, vp, ip, ip]
        lib.oracle_max_threads.argtypes = [ip]
        for f in ("oracle_exit_law", "oracle_sample", "oracle_residual_cdf", "oracle_predraw", "oracle_tree_attn",
                  "oracle_check_tree", "oracle_max_threads"):
            getattr(lib, f).restype = ctypes.c_int
        _lib = lib
    return _lib


def _ptr(a: np.ndarray | None):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _as_input(x: np.ndarray, dtype: str) -> np.ndarray:
    """Contiguous view with the element type the C widening expects."""
    want = {"f32": np.float32, "bf16": np.uint16, "f64": np.float64}[dtype]
    x = np.ascontiguousarray(x)
    if x.dtype != want:
        raise TypeError(f"expected {want} storage for dtype {dtype}, got {x.dtype}")
    return x


class OracleError(RuntimeError):
    pass


def max_threads(nthreads: int = 0) -> int:
    return int(_load().oracle_max_threads(int(nthreads)))


def check_tree(parents: np.ndarray, tokens: np.ndarray, V: int) -> bool:
    p = np.ascontiguousarray(parents, dtype=np.int32)
    t = np.ascontiguousarray(tokens, dtype=np.int32)
    return _load().oracle_check_tree(_ptr(p), _ptr(t), int(p.shape[-1]), int(V)) == 0


@dataclass
class ExitLaw:
    rho: np.ndarray        # [R][B]
    reach: np.ndarray      # [R][B]
    exit_mass: np.ndarray  # [R][B]
    coverage: np.ndarray   # [R]
    logZ: np.ndarray       # [R][B]


def exit_law(logits: np.ndarray, dtype: str, parents: np.ndarray, tokens: np.ndarray,
             inv_temperature: float = 1.0, nthreads: int = 0) -> ExitLaw:
    """rho, P, w, C of 2610.11750 Sec. 3 (Eq. 2, 4, 6) per request.

    ``logits`` has shape [R][B][V] (or [B][V] for one request) and storage
    float32 (dtype "f32"), uint16 bf16 bits ("bf16") or float64 ("f64").
    """
    lg = _as_input(logits, dtype)
    if lg.ndim == 2:
        lg = lg[None]
    R, B, V = lg.shape
    par = np.ascontiguousarray(parents, dtype=np.int32).reshape(R, B)
    tok = np.ascontiguousarray(tokens, dtype=np.int32).reshape(R, B)
    rho = np.empty((R, B)); reach = np.empty((R, B)); w = np.empty((R, B))
    cov = np.empty(R); logZ = np.empty((R, B))
    st = _load().oracle_exit_law(_ptr(lg), _DTYPE_CODES[dtype], _ptr(par), _ptr(tok), R, B, V,
                                 float(inv_temperature), _ptr(rho), _ptr(reach), _ptr(w),
                                 _ptr(cov), _ptr(logZ), int(nthreads))
    if st != 0:
        raise OracleError(f"oracle_exit_law failed with status {st}")
    return ExitLaw(rho, reach, w, cov, logZ)


@dataclass
class Draws:
    exit_node: np.ndarray    # [R][n] int32
    bonus_token: np.ndarray  # [R][n] int32
    band_exit: np.ndarray    # [R][n] bool: u1 within 1e-6 of a boundary of its bin
    band_bonus: np.ndarray   # [R][n] bool


def sample(logits: np.ndarray, dtype: str, parents: np.ndarray, tokens: np.ndarray,
           exit_mass: np.ndarray, uniforms: np.ndarray, inv_temperature: float = 1.0,
           nthreads: int = 0) -> Draws:
    """TEV's exit-node and bonus-token draws (2610.11750 App. B, Algorithm 1)."""
    lg = _as_input(logits, dtype)
    if lg.ndim == 2:
        lg = lg[None]
    R, B, V = lg.shape
    par = np.ascontiguousarray(parents, dtype=np.int32).reshape(R, B)
    tok = np.ascontiguousarray(tokens, dtype=np.int32).reshape(R, B)
    w = np.ascontiguousarray(exit_mass, dtype=np.float64).reshape(R, B)
    u = np.ascontiguousarray(uniforms, dtype=np.float32).reshape(R, -1, 2)
    n = u.shape[1]
    en = np.empty((R, n), np.int32); bt = np.empty((R, n), np.int32)
    band = np.empty((R, n, 2), np.uint8)
    st = _load().oracle_sample(_ptr(lg), _DTYPE_CODES[dtype], _ptr(par), _ptr(tok), R, B, V,
                               float(inv_temperature), _ptr(w), _ptr(u), n, _ptr(en), _ptr(bt),
                               _ptr(band), int(nthreads))
    if st != 0:
        raise OracleError(f"oracle_sample failed with status {st}")
    return Draws(en, bt, band[..., 0].astype(bool), band[..., 1].astype(bool))


@dataclass
class PredrawDraws:
    node_draw: np.ndarray    # [R][n][B] int32: R_v of every node
    exit_node: np.ndarray    # [R][n] int32
    bonus_token: np.ndarray  # [R][n] int32
    band: np.ndarray         # [R][n] bool: a draw on the walked path within 1e-6 of a boundary
    node_band: np.ndarray    # [R][n][B] bool: node v's own draw within 1e-6 of a boundary of its bin


def predraw(logits: np.ndarray, dtype: str, parents: np.ndarray, tokens: np.ndarray,
            uniforms: np.ndarray, inv_temperature: float = 1.0, nthreads: int = 0) -> PredrawDraws:
    """Predraw-and-follow verification (2610.11750 App. A.4.1): one draw per
    node from its full target row, then the walk from the root.
    uniforms [R][n][B] (one per node per draw)."""
    lg = _as_input(logits, dtype)
    if lg.ndim == 2:
        lg = lg[None]
    R, B, V = lg.shape
    par = np.ascontiguousarray(parents, dtype=np.int32).reshape(R, B)
    tok = np.ascontiguousarray(tokens, dtype=np.int32).reshape(R, B)
    u = np.ascontiguousarray(uniforms, dtype=np.float32).reshape(R, -1, B)
    n = u.shape[1]
    nd = np.empty((R, n, B), np.int32)
    en = np.empty((R, n), np.int32); bt = np.empty((R, n), np.int32)
    band = np.empty((R, n), np.uint8)
    nband = np.empty((R, n, B), np.uint8)
    st = _load().oracle_predraw(_ptr(lg), _DTYPE_CODES[dtype], _ptr(par), _ptr(tok), R, B, V,
                                float(inv_temperature), _ptr(u), n, _ptr(nd), _ptr(en), _ptr(bt),
                                _ptr(band), _ptr(nband), int(nthreads))
    if st != 0:
        raise OracleError(f"oracle_predraw failed with status {st}")
    return PredrawDraws(nd, en, bt, band.astype(bool), nband.astype(bool))


def commit_kv(k: np.ndarray, v: np.ndarray, parents: np.ndarray, exit_node: np.ndarray, P: int):
    """Cache commit after verification (2610.00321 App. C "Packed
    verification": the accepted root path keeps its packed entries, compacted
    after the prefix).  k, v [L][R][Hkv][P+B][D] (not modified);
    exit_node [R].  For the root path 0 = a_0, ..., a_A = V of each request,
    row P + d of the result is row P + a_d of the input (d = 0..A); every other
    row is copied unchanged.  Returns (k', v', new_len [R] = P + A + 1)."""
    k2, v2 = np.array(k, copy=True), np.array(v, copy=True)
    R = k.shape[1]
    B = k.shape[3] - P
    par = np.asarray(parents).reshape(R, B)
    new_len = np.empty(R, np.int32)
    for r in range(R):
        path = [int(exit_node[r])]
        while path[-1] != 0:
            path.append(int(par[r, path[-1]]))
        path.reverse()
        for d, a in enumerate(path):
            k2[:, r, :, P + d] = k[:, r, :, P + a]
            v2[:, r, :, P + d] = v[:, r, :, P + a]
        new_len[r] = P + len(path)
    return k2, v2, new_len


@dataclass
class ExitLoss:
    loss: float              # L_exit
    numerator: float         # sum of w(v) * (-log q) over every non-root node
    row_lse: np.ndarray      # [R][H] logsumexp of every draft-logit row
    row_weight: np.ndarray   # [R][H] summed weight of the nodes scored by the row
    grad: np.ndarray         # [R][H][V] d L_exit / d draft_logits


def _logsumexp64(z: np.ndarray) -> float:
    """log sum_a exp(z_a) in fp64, shifted by the maximum; -inf for an all -inf row."""
    m = float(np.max(z))
    if m == -np.inf:
        return -np.inf
    return m + float(np.log(np.sum(np.exp(z - m))))


def exit_loss(draft_logits: np.ndarray, dtype: str, parents: np.ndarray, tokens: np.ndarray,
              weights: np.ndarray) -> ExitLoss:
    """Exit-guided draft-tree loss ("Where Draft Trees Lose Target Mass",
    Sec. 5 Eq. 14) and its gradient in the draft logits.

    draft_logits [R][H][V]: row (r, d - 1) holds the drafter's position-wise
    logits for future draft position d = 1..H of example r, shared by every
    node of depth d (Sec. 5; App. C.2 row(v)).  weights [R][B] are the
    detached exit weights w(v); tokens [R][B] the incoming draft tokens x_v.

    Written node by node as Eq. 14 states it: each non-root node v of depth d
    contributes w(v) * (-log q_d(x_v)), with log q_d = z - logsumexp(z) of its
    own row (one logsumexp per node: none of App. C.2's sharing), and the sum
    over the minibatch is divided by the number of non-root nodes,
    sum_i (|V_i| - 1) = R (B - 1).  Readings: a node whose weight is exactly 0
    contributes nothing (so a zero-probability token under a zero weight is
    not 0 * inf); with no non-root node the loss and gradient are 0; a node
    deeper than H has no draft row and is an error.

    The gradient of -log q_d(x_v) in row d's logits is softmax(z) - e_{x_v};
    grad sums w(v) times it over the row's nodes, divided by the same count.
    row_weight[r][d-1] is the sum of w(v) over the row's nonzero-weight nodes
    (Eq. 67's per-row factor), reported alongside."""
    z = _as_input(draft_logits, dtype)
    if dtype == "bf16":                                   # bf16 = upper half of a binary32
        z = (z.astype(np.uint32) << np.uint32(16)).view(np.float32)
    z = z.astype(np.float64)
    R, H, V = z.shape
    par = np.asarray(parents, dtype=np.int64).reshape(R, -1)
    tok = np.asarray(tokens, dtype=np.int64).reshape(R, -1)
    w = np.asarray(weights, dtype=np.float64).reshape(R, -1)
    B = par.shape[1]
    n_nodes = R * (B - 1)
    row_lse = np.array([[_logsumexp64(z[r, d]) for d in range(H)] for r in range(R)])
    row_weight = np.zeros((R, H))
    grad = np.zeros((R, H, V))
    num = 0.0
    for r in range(R):
        if not check_tree(par[r].astype(np.int32), tok[r].astype(np.int32), V):
            raise OracleError(f"request {r}: invalid tree")
        depth = np.zeros(B, np.int64)
        for v in range(1, B):
            depth[v] = depth[par[r, v]] + 1
            if depth[v] > H:
                raise OracleError(f"request {r}: node {v} has depth {depth[v]} > H = {H}")
        for v in range(1, B):
            if w[r, v] == 0.0:
                continue
            row = z[r, depth[v] - 1]
            lse = _logsumexp64(row)                       # this node's own normaliser
            num += w[r, v] * (lse - row[tok[r, v]])       # w(v) * (-log q_d(x_v))
            row_weight[r, depth[v] - 1] += w[r, v]
            g = np.exp(row - lse)
            g[tok[r, v]] -= 1.0
            grad[r, depth[v] - 1] += w[r, v] * g
    if n_nodes == 0:
        return ExitLoss(0.0, 0.0, row_lse, row_weight, grad)
    return ExitLoss(num / n_nodes, num, row_lse, row_weight, grad / n_nodes)


@dataclass
class BuiltTree:
    parents: np.ndarray    # [R][B] int32, node order = pop order
    tokens: np.ndarray     # [R][B] int32, tokens[r][0] = the root token
    scores: np.ndarray     # [R][B] float64, log of the plug-in prefix score (root 0)
    near_tie: np.ndarray   # [R] bool: two keys the heap compared differ by <= tie_eps


def build_tree(draft_logits: np.ndarray, dtype: str, topk: int, n_nodes: int,
               root_tokens: np.ndarray, tie_eps: float = 1e-9) -> BuiltTree:
    """Best-first draft tree over the retained universe ("CAST", App. C
    "Candidate construction"; "Multi-Future Drafting", App. B, the merged heap
    with one mode, i.e. DDTree's builder).

    draft_logits [R][L][V]: row j is draft position j + 1.  q_j = softmax of
    row j over the whole vocabulary (scores use the original q_j, not a
    renormalised top-K).  Each position keeps its topk most likely tokens
    (larger logit first, then smaller token id); rank r is the position in
    that list.  The plug-in score of a prefix y_1..y_d is
    prod_j q_j(y_j); its key is
        s = (sum_j z_{j, y_j}) - (sum_j lse_j)        (= log of the score)
    with the logit sum accumulated along the path in f64 (exact for bf16
    logits) and the logsumexp sum per depth.

    The heap holds candidate prefixes keyed by s; popping a prefix emits it
    as the next node and pushes its next sibling (its last token replaced by
    the one of the next rank) and its first child (the rank-0 token of the
    next position, while its depth is below L).  It starts from the rank-0
    token of position 1 and stops after n_nodes - 1 pops.  Equal keys go to
    the shorter prefix, then to the lexicographically smaller rank sequence.

    near_tie[r] reports whether two keys of request r that the build orders
    (every emitted node and every entry left in the heap) differ by at most
    tie_eps without being computed from identical logit sums."""
    z = _as_input(draft_logits, dtype)
    if dtype == "bf16":
        z = (z.astype(np.uint32) << np.uint32(16)).view(np.float32)
    z = z.astype(np.float64)
    R, L, V = z.shape
    if not (1 <= topk <= V) or n_nodes < 1:
        raise OracleError("bad topk / n_nodes")
    universe = sum(topk ** d for d in range(1, L + 1))
    if n_nodes - 1 > universe:
        raise OracleError("the retained universe holds fewer prefixes than n_nodes - 1")
    par = np.full((R, n_nodes), -1, np.int32)
    tok = np.zeros((R, n_nodes), np.int32)
    sc = np.zeros((R, n_nodes))
    near = np.zeros(R, bool)
    for r in range(R):
        lse = np.array([_logsumexp64(z[r, j]) for j in range(L)])
        C = np.concatenate([[0.0], np.cumsum(lse)])          # C[d] = sum of lse over depths 1..d
        order = [np.lexsort((np.arange(V), -z[r, j]))[:topk] for j in range(L)]
        ztop = [z[r, j, order[j]] for j in range(L)]
        tok[r, 0] = int(root_tokens[r])
        node_sz = [0.0]                                       # exact logit sums of the nodes
        keys_seen = []                                        # (s, Sz, depth) of ordered keys

        def entry(sz, depth, ranks, parent):
            return (-(sz - C[depth]), depth, ranks, parent, sz)

        heap = [entry(ztop[0][0], 1, (0,), 0)] if n_nodes > 1 else []
        for n in range(1, n_nodes):
            negs, depth, ranks, parent, sz = heapq.heappop(heap)
            par[r, n] = parent
            tok[r, n] = int(order[depth - 1][ranks[-1]])
            sc[r, n] = -negs
            node_sz.append(sz)
            keys_seen.append((-negs, sz, depth))
            rk = ranks[-1]
            if rk + 1 < topk:                                 # next sibling
                heapq.heappush(heap, entry(node_sz[parent] + ztop[depth - 1][rk + 1], depth,
                                           ranks[:-1] + (rk + 1,), parent))
            if depth < L:                                     # first child
                heapq.heappush(heap, entry(sz + ztop[depth][0], depth + 1, ranks + (0,), n))
        keys_seen += [(-e[0], e[4], e[1]) for e in heap]
        keys_seen.sort()
        for (s1, z1, d1), (s2, z2, d2) in zip(keys_seen, keys_seen[1:]):
            if s2 - s1 <= tie_eps and not (z1 == z2 and d1 == d2):
                near[r] = True
                break
    return BuiltTree(par, tok, sc, near)


def build_tree_modes(draft_logits: np.ndarray, dtype: str, topk: int, n_nodes: int,
                     root_tokens: np.ndarray, log_prior: np.ndarray | None = None,
                     tie_eps: float = 1e-9) -> BuiltTree:
    """The merged heap over several draft modes ("Multi-Future Drafting",
    App. B, Prop. 6): the tree of the n_nodes - 1 distinct prefixes with the
    largest best-mode score s(v) = max_k s_k(v), in the order of their first
    pops.

    draft_logits [R][M][L][V]: mode k's position-wise logits.  log_prior
    [R][M] (log pi_k; uniform -log M when None).  Mode k's key of a prefix of
    its retained universe (its own top-K tokens per position) is
        s_k(v) = ((sum_j z_{k,j,y_j}) - (sum_j lse_{k,j})) + log pi_k
    (the single-mode key of ``build_tree`` plus the log prior).  The heap holds
    entries (k, v) keyed by s_k(v) and starts from every mode's rank-0 token
    of position 1; popping (k, v) adds a node for v unless the tree holds it
    already, and pushes v's next sibling and first child under mode k either
    way.  Equal keys go to the shorter prefix, then the smaller rank sequence,
    then the smaller mode.  With one mode and no prior this is ``build_tree``.
    If the modes' universes hold fewer than n_nodes - 1 distinct prefixes, the
    missing nodes get parent and token -1 and score NaN.

    near_tie[r] as in ``build_tree``, over every popped entry and every entry
    left in the heap (keys computed from identical logit sums, logsumexp sums
    and priors are exact ties on both sides and are not reported)."""
    z = _as_input(draft_logits, dtype)
    if dtype == "bf16":
        z = (z.astype(np.uint32) << np.uint32(16)).view(np.float32)
    z = z.astype(np.float64)
    R, M, L, V = z.shape
    if not (1 <= topk <= V) or n_nodes < 1:
        raise OracleError("bad topk / n_nodes")
    if n_nodes - 1 > M * sum(topk ** d for d in range(1, L + 1)):
        raise OracleError("the retained universes hold fewer prefixes than n_nodes - 1")
    lp = (np.full((R, M), -np.log(M)) if log_prior is None
          else np.asarray(log_prior, dtype=np.float32).astype(np.float64).reshape(R, M))
    if M == 1 and log_prior is None:
        lp[:] = 0.0
    par = np.full((R, n_nodes), -1, np.int32)
    tok = np.zeros((R, n_nodes), np.int32)
    sc = np.zeros((R, n_nodes))
    near = np.zeros(R, bool)
    for r in range(R):
        C, order, ztop = [], [], []
        for k in range(M):
            lse = np.array([_logsumexp64(z[r, k, j]) for j in range(L)])
            C.append(np.concatenate([[0.0], np.cumsum(lse)]))
            order.append([np.lexsort((np.arange(V), -z[r, k, j]))[:topk] for j in range(L)])
            ztop.append([z[r, k, j, order[k][j]] for j in range(L)])
        tok[r, 0] = int(root_tokens[r])
        node_of = {(): 0}                          # token sequence -> node
        seq_sz = {}                                # (mode, rank sequence) -> logit sum of the path
        keys_seen = []

        def entry(k, sz, ranks):
            d = len(ranks)
            return (-((sz - C[k][d]) + lp[r, k]), d, ranks, k, sz)

        heap = []
        if n_nodes > 1:
            for k in range(M):
                heapq.heappush(heap, entry(k, ztop[k][0][0], (0,)))
        n = 1
        while heap and n < n_nodes:
            negs, d, ranks, k, sz = heapq.heappop(heap)
            keys_seen.append((-negs, sz, C[k][d], lp[r, k]))
            seq_sz[(k, ranks)] = sz
            seq = tuple(int(order[k][j][ranks[j]]) for j in range(d))
            if seq not in node_of:
                node_of[seq] = n
                par[r, n] = node_of[seq[:-1]]
                tok[r, n] = seq[-1]
                sc[r, n] = -negs
                n += 1
            rk = ranks[-1]
            if rk + 1 < topk:                      # next sibling under mode k
                psz = seq_sz[(k, ranks[:-1])] if d > 1 else 0.0
                heapq.heappush(heap, entry(k, psz + ztop[k][d - 1][rk + 1], ranks[:-1] + (rk + 1,)))
            if d < L:                              # first child under mode k
                heapq.heappush(heap, entry(k, sz + ztop[k][d][0], ranks + (0,)))
        if n < n_nodes:                            # fewer distinct prefixes than nodes
            tok[r, n:] = -1
            sc[r, n:] = np.nan
        keys_seen += [(-e[0], e[4], C[e[3]][e[1]], lp[r, e[3]]) for e in heap]
        keys_seen.sort()
        for (s1, z1, c1, p1), (s2, z2, c2, p2) in zip(keys_seen, keys_seen[1:]):
            if s2 - s1 <= tie_eps and not (z1 == z2 and c1 == c2 and p1 == p2):
                near[r] = True
                break
    return BuiltTree(par, tok, sc, near)


def residual_cdf(logits_req: np.ndarray, dtype: str, parents: np.ndarray, tokens: np.ndarray,
                 node: int, inv_temperature: float = 1.0) -> np.ndarray:
    """Normalised residual CDF of one node's row in token order (Eq. 7)."""
    lg = _as_input(logits_req, dtype)
    B, V = lg.shape
    par = np.ascontiguousarray(parents, dtype=np.int32).reshape(B)
    tok = np.ascontiguousarray(tokens, dtype=np.int32).reshape(B)
    out = np.empty(V)
    st = _load().oracle_residual_cdf(_ptr(lg), _DTYPE_CODES[dtype], _ptr(par), _ptr(tok), B, V,
                                     int(node), float(inv_temperature), _ptr(out))
    if st != 0:
        raise OracleError(f"oracle_residual_cdf failed with status {st}")
    return out


def tree_attn(q: np.ndarray, k: np.ndarray, v: np.ndarray, dtype: str, parents: np.ndarray,
              P: int, scale: float, rows: np.ndarray | None = None,
              nthreads: int = 0) -> np.ndarray:
    """Ancestor-masked tree attention (2610.00321 App. B Lemma 1, App. C).

    q [R][B][Hq][D]; k, v [R][Hkv][P+B][D].  Returns [R][B][Hq][D] float64, or
    [len(rows)][D] for the flat query indices in ``rows``.
    """
    qq = _as_input(q, dtype); kk = _as_input(k, dtype); vv = _as_input(v, dtype)
    R, B, Hq, D = qq.shape
    Hkv = kk.shape[1]
    if kk.shape != (R, Hkv, P + B, D) or vv.shape != kk.shape:
        raise ValueError("k/v shape must be [R][Hkv][P+B][D]")
    par = np.ascontiguousarray(parents, dtype=np.int32).reshape(R, B)
    if rows is None:
        out = np.empty((R, B, Hq, D))
        rr, nr = None, 0
    else:
        rr = np.ascontiguousarray(rows, dtype=np.int64)
        nr = int(rr.shape[0])
        out = np.empty((nr, D))
    st = _load().oracle_tree_attn(_ptr(qq), _ptr(kk), _ptr(vv), _DTYPE_CODES[dtype], _ptr(par),
                                  R, B, Hq, Hkv, D, int(P), float(scale), _ptr(out), _ptr(rr),
                                  nr, int(nthreads))
    if st != 0:
        raise OracleError(f"oracle_tree_attn failed with status {st}")
    return out
