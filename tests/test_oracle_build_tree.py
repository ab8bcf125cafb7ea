"""Pins of the oracle's best-first tree builder ("CAST: Cost-Aware Speculative
Trees from One-Pass Block Drafters", App. C "Candidate construction" and
Thm. 1; "Multi-Future Drafting", App. B, the merged heap with one mode).
CPU only.

What fixes the oracle here, other than its own heap:
  * Thm. 1: the tree is the top (B - 1) prefixes of the retained universe by
    plug-in score, ties toward prefixes -- brute force over every prefix of
    small universes gives the same nodes in the same order;
  * CAST's own heap (each pop pushes all top-K children of the popped node)
    returns the same tree as the sibling / first-child heap;
  * node scores are logs of products of library softmax probabilities;
  * equal logits everywhere: every prefix of one depth ties, so the order is
    by depth, then lexicographic rank (closed form);
  * top-1: the chain of per-position argmaxes;
  * the merged heap over several modes ("Multi-Future Drafting" Prop. 6)
    returns the B - 1 distinct prefixes with the largest best-mode score, by
    brute force over the union of the modes' universes; one mode is the
    single-mode builder; identical modes collapse to it.
"""
import heapq
import itertools

import numpy as np
import pytest
import scipy.special

import oracle


def _rows(seed, R, L, V, scale=2.0, dtype="f32"):
    z = (np.random.default_rng(seed).standard_normal((R, L, V)) * scale).astype(np.float32)
    return z


def _retained(z_row, K):
    return np.lexsort((np.arange(z_row.shape[0]), -z_row))[:K]


def _brute_force(z, K, B):
    """Every prefix of the retained universe, scored with scipy's log-softmax,
    sorted by (score desc, depth, rank sequence) -- the first B - 1."""
    L, V = z.shape
    logq = scipy.special.log_softmax(z.astype(np.float64), axis=-1)
    keep = [_retained(z[j], K) for j in range(L)]
    cands = []
    for d in range(1, L + 1):
        for ranks in itertools.product(range(K), repeat=d):
            s = sum(logq[j, keep[j][ranks[j]]] for j in range(d))
            cands.append((-s, d, ranks))
    cands.sort()
    chosen = cands[:B - 1]
    node_of = {(): 0}
    parents, tokens, scores = [-1], [0], [0.0]
    for negs, d, ranks in chosen:
        node_of[ranks] = len(parents)
        parents.append(node_of[ranks[:-1]])
        tokens.append(int(keep[d - 1][ranks[-1]]))
        scores.append(-negs)
    gaps = np.diff(sorted(-c[0] for c in cands))
    return np.array(parents), np.array(tokens), np.array(scores), gaps


@pytest.mark.parametrize("seed,L,V,K,B", [(0, 3, 12, 4, 30), (1, 4, 9, 3, 40), (2, 2, 50, 8, 25),
                                         (3, 5, 6, 2, 31), (4, 3, 7, 7, 60)])
def test_top_prefixes_by_brute_force(seed, L, V, K, B):
    z = _rows(seed, 1, L, V)
    got = oracle.build_tree(z, "f32", K, B, np.array([5]))
    par, tok, sc, gaps = _brute_force(z[0], K, B)
    assert not got.near_tie[0]
    np.testing.assert_array_equal(got.parents[0], par)
    np.testing.assert_array_equal(got.tokens[0, 1:], tok[1:])
    assert got.tokens[0, 0] == 5
    np.testing.assert_allclose(got.scores[0], sc, rtol=0, atol=1e-12)


def _cast_heap(z, K, B):
    """CAST App. C: seed with the root's top-K children; each pop emits a node
    and pushes all of its top-K children at the next depth while depth < L."""
    L, V = z.shape
    logq = scipy.special.log_softmax(z.astype(np.float64), axis=-1)
    keep = [_retained(z[j], K) for j in range(L)]
    heap = [(-logq[0, keep[0][r]], 1, (r,), 0) for r in range(K)]
    heapq.heapify(heap)
    parents, tokens = [-1], [0]
    pushes = K
    while len(parents) < B:
        negs, d, ranks, p = heapq.heappop(heap)
        n = len(parents)
        parents.append(p)
        tokens.append(int(keep[d - 1][ranks[-1]]))
        if d < L:
            for r in range(K):
                heapq.heappush(heap, (negs - logq[d, keep[d][r]], d + 1, ranks + (r,), n))
                pushes += 1
    assert pushes <= K + (B - 1) * K            # "at most K + NK pushes and N pops"
    return np.array(parents), np.array(tokens)


@pytest.mark.parametrize("seed", [5, 6, 7])
def test_matches_cast_all_children_heap(seed):
    R, L, V, K, B = 3, 6, 300, 8, 64
    z = _rows(seed, R, L, V, scale=3.0)
    got = oracle.build_tree(z, "f32", K, B, np.zeros(R, np.int32))
    for r in range(R):
        assert not got.near_tie[r]
        par, tok = _cast_heap(z[r], K, B)
        np.testing.assert_array_equal(got.parents[r], par)
        np.testing.assert_array_equal(got.tokens[r, 1:], tok[1:])


def test_scores_are_library_log_products():
    R, L, V, K, B = 2, 8, 1000, 16, 100
    z = _rows(11, R, L, V, scale=4.0)
    got = oracle.build_tree(z, "f32", K, B, np.zeros(R, np.int32))
    logq = scipy.special.log_softmax(z.astype(np.float64), axis=-1)
    for r in range(R):
        for n in range(1, B):
            path, v = [], n
            while v != 0:
                path.append(v)
                v = got.parents[r, v]
            path.reverse()
            s = sum(logq[r, d, got.tokens[r, u]] for d, u in enumerate(path))
            assert got.scores[r, n] == pytest.approx(s, abs=1e-11)
        # pop order is best first: scores never increase
        assert np.all(np.diff(got.scores[r, 1:]) <= 1e-12)


def test_equal_logits_order_by_depth_then_rank():
    """Every retained token has the same probability: all prefixes of one
    depth tie, shorter prefixes come first, then lexicographic rank order,
    and rank order among equal logits is token order."""
    L, V, K, B = 3, 10, 3, 1 + 3 + 9 + 5
    z = np.zeros((1, L, V), np.float32)
    got = oracle.build_tree(z, "f32", K, B, np.array([0]))
    want_par = [-1, 0, 0, 0, 1, 1, 1, 2, 2, 2, 3, 3, 3, 4, 4, 4, 5, 5]
    want_tok = [0, 0, 1, 2, 0, 1, 2, 0, 1, 2, 0, 1, 2, 0, 1, 2, 0, 1]
    np.testing.assert_array_equal(got.parents[0], want_par)
    np.testing.assert_array_equal(got.tokens[0], want_tok)
    np.testing.assert_allclose(got.scores[0, 1:4], -np.log(V))
    assert not got.near_tie[0]                      # exact ties, computed identically


def test_top1_is_the_argmax_chain():
    L, V = 6, 77
    z = _rows(13, 1, L, V)
    got = oracle.build_tree(z, "f32", 1, L + 1, np.array([3]))
    np.testing.assert_array_equal(got.parents[0], np.arange(-1, L))
    np.testing.assert_array_equal(got.tokens[0, 1:], np.argmax(z[0], axis=-1))


def test_bf16_input_and_universe_limit():
    z = _rows(17, 1, 2, 40)
    bits = ((z.view(np.uint32) + 0x7FFF + ((z.view(np.uint32) >> 16) & 1)) >> 16).astype(np.uint16)
    wid = (bits.astype(np.uint32) << 16).view(np.float32)
    a = oracle.build_tree(bits, "bf16", 4, 15, np.array([0]))
    b = oracle.build_tree(wid, "f32", 4, 15, np.array([0]))
    np.testing.assert_array_equal(a.parents, b.parents)
    np.testing.assert_array_equal(a.tokens, b.tokens)
    with pytest.raises(oracle.OracleError):
        oracle.build_tree(z, "f32", 2, 8, np.array([0]))   # 2 + 4 = 6 < 7 prefixes


# ----------------------------------------------------------------------------
# The merged heap over several modes ("Multi-Future Drafting", App. B, Prop. 6)
def _brute_force_modes(z, K, B, lp):
    """Every prefix that some mode's retained universe holds, scored by the
    best such mode's log pi_k + log q_k(v) (scipy log-softmax), the B - 1
    largest, best first (ties: shorter first)."""
    M, L, V = z.shape
    logq = scipy.special.log_softmax(z.astype(np.float64), axis=-1)
    keep = [[_retained(z[k, j], K) for j in range(L)] for k in range(M)]
    best = {}
    for k in range(M):
        for d in range(1, L + 1):
            for ranks in itertools.product(range(K), repeat=d):
                seq = tuple(int(keep[k][j][ranks[j]]) for j in range(d))
                s = lp[k] + sum(logq[k, j, seq[j]] for j in range(d))
                if seq not in best or s > best[seq]:
                    best[seq] = s
    chosen = sorted(best.items(), key=lambda kv: (-kv[1], len(kv[0])))[:B - 1]
    return chosen


@pytest.mark.parametrize("seed,M,L,V,K,B,prior", [(0, 3, 3, 9, 3, 25, False), (1, 4, 2, 12, 4, 20, True),
                                                  (2, 2, 4, 6, 2, 30, True), (3, 8, 2, 40, 6, 33, False)])
def test_merged_heap_is_top_distinct_prefixes(seed, M, L, V, K, B, prior):
    """Prop. 6: the B - 1 distinct prefixes with the largest best-mode score,
    in nonincreasing order; node scores are those best-mode scores."""
    rng = np.random.default_rng(seed)
    z = (rng.standard_normal((1, M, L, V)) * 2.0).astype(np.float32)
    # modes share some structure: mode 1 copies mode 0's first position
    if M > 1:
        z[0, 1, 0] = z[0, 0, 0]
    lp = np.log(rng.dirichlet(np.ones(M))).astype(np.float32) if prior else None
    got = oracle.build_tree_modes(z, "f32", K, B, np.array([0]), log_prior=None if lp is None else lp[None])
    assert not got.near_tie[0]
    want = _brute_force_modes(z[0], K, B, np.full(M, -np.log(M)) if lp is None else lp.astype(np.float64))
    seqs = [()]
    for n in range(1, B):
        seqs.append(seqs[got.parents[0, n]] + (int(got.tokens[0, n]),))
    assert [s for s, _ in want] == seqs[1:]
    np.testing.assert_allclose(got.scores[0, 1:], [v for _, v in want], rtol=0, atol=1e-11)
    # distinct siblings, parents before children
    for n in range(1, B):
        assert 0 <= got.parents[0, n] < n
    assert len(set(seqs)) == B


def test_one_mode_is_the_single_mode_builder():
    z = (np.random.default_rng(21).standard_normal((3, 1, 6, 500)) * 3).astype(np.float32)
    a = oracle.build_tree(z[:, 0], "f32", 16, 80, np.arange(3))
    b = oracle.build_tree_modes(z, "f32", 16, 80, np.arange(3))
    np.testing.assert_array_equal(a.parents, b.parents)
    np.testing.assert_array_equal(a.tokens, b.tokens)
    np.testing.assert_array_equal(a.scores, b.scores)


def test_identical_modes_collapse():
    """Copies of one mode under a uniform prior give the one-mode tree (every
    prefix ties across the copies; the lowest mode creates the node), with
    scores shifted by log(1 / M)."""
    z1 = (np.random.default_rng(22).standard_normal((1, 1, 4, 200)) * 3).astype(np.float32)
    z = np.repeat(z1, 4, axis=1)
    a = oracle.build_tree(z1[:, 0], "f32", 8, 50, np.array([0]))
    b = oracle.build_tree_modes(z, "f32", 8, 50, np.array([0]))
    np.testing.assert_array_equal(a.parents, b.parents)
    np.testing.assert_array_equal(a.tokens, b.tokens)
    np.testing.assert_allclose(b.scores[0, 1:], a.scores[0, 1:] - np.log(4), rtol=0, atol=1e-12)


def test_merged_heap_short_universe():
    """Two identical modes of 2 + 4 prefixes each hold 6 distinct prefixes: a
    tree of 13 nodes keeps its last 6 unfilled."""
    z = (np.random.default_rng(23).standard_normal((1, 1, 2, 30)) * 2).astype(np.float32)
    got = oracle.build_tree_modes(np.repeat(z, 2, axis=1), "f32", 2, 13, np.array([0]))
    assert np.all(got.parents[0, 1:7] >= 0)
    assert np.all(got.parents[0, 7:] == -1) and np.all(got.tokens[0, 7:] == -1)
    assert np.all(np.isnan(got.scores[0, 7:]))
