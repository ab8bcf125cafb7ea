"""Pins of the oracle's predraw-and-follow verifier ("Where Draft Trees Lose
Target Mass: Exit-Guided Speculative Decoding", App. A.4.1): per-node draws
against the library's inverse CDF, the walk on trees whose draws are
certain, the root-only special case, and the joint (exit node, bonus token)
law against the target-flow enumeration (Cor. 1).  CPU only."""
import numpy as np
import pytest
from scipy.special import softmax

import oracle
from tests import workloads as W
from tests import lawtools as LT


def _small_case(seed, B=7, V=5):
    rng = np.random.default_rng(seed)
    parents, tokens = W.random_tree(B, V, rng)
    lg = rng.standard_normal((B, V)) * 1.2
    for u in range(1, B):
        lg[parents[u], tokens[u]] += 1.0
    return parents, tokens, lg


def _uniforms(seed, R, n, B):
    rng = np.random.default_rng(seed)
    k = rng.integers(0, 1 << 24, size=(R, n, B))
    return (k.astype(np.float64) * 2.0 ** -24).astype(np.float32)


def test_node_draws_are_the_library_inverse_cdf():
    """R_v = smallest a with u * total < cumsum(p_v)[a] (numpy searchsorted on
    scipy's softmax), for every node, outside the 1e-6 band of its bin."""
    rng = np.random.default_rng(11)
    B, V = 20, 3000
    parents, tokens = W.random_tree(B, V, rng)
    lg = (rng.standard_normal((B, V)) * 3.0).astype(np.float32)
    u = _uniforms(12, 1, 64, B)
    dr = oracle.predraw(lg, "f32", parents, tokens, u)
    p = softmax(lg.astype(np.float64), axis=1)
    checked = 0
    for v in range(B):
        c = np.cumsum(p[v])
        cn = c / c[-1]
        for n in range(u.shape[1]):
            uu = float(u[0, n, v])
            j = int(np.searchsorted(c, uu * c[-1], side="right"))
            lo = 0.0 if j == 0 else cn[j - 1]
            in_band = abs(uu - lo) < 1e-6 or abs(uu - cn[j]) < 1e-6
            if in_band:
                continue
            assert not dr.node_band[0, n, v], (v, n)
            assert dr.node_draw[0, n, v] == j, (v, n)
            checked += 1
    assert checked > 0.99 * B * u.shape[1]


def test_walk_band_is_the_band_of_the_walked_draws():
    """The walk's band flag is set exactly when some node on the walked path
    (root to exit node) has its own draw in the band; draws off the path do
    not count.  Uniforms are placed on bin boundaries on purpose."""
    rng = np.random.default_rng(21)
    B, V = 12, 40
    parents, tokens = W.random_tree(B, V, rng)
    lg = (rng.standard_normal((B, V)) * 1.5).astype(np.float32)
    for u_ in range(1, B):
        lg[parents[u_], tokens[u_]] += 2.0
    u = _uniforms(22, 1, 300, B)
    p = softmax(lg.astype(np.float64), axis=1)
    cn = np.cumsum(p, axis=1)
    cn /= cn[:, -1:]
    # every fifth draw: put some node's uniform on a boundary of its row CDF
    for n in range(0, u.shape[1], 5):
        v = int(rng.integers(0, B))
        u[0, n, v] = np.float32(cn[v, int(rng.integers(0, V - 1))])
    dr = oracle.predraw(lg, "f32", parents, tokens, u)
    assert dr.node_band.any()
    for n in range(u.shape[1]):
        path, v = [], int(dr.exit_node[0, n])
        while v >= 0:
            path.append(v)
            v = int(parents[v]) if v > 0 else -1
        assert dr.band[0, n] == bool(dr.node_band[0, n, path].any()), n


def test_root_only_tree_is_plain_sampling():
    """With T = {r} the verifier stops at the root and emits its draw."""
    rng = np.random.default_rng(5)
    V = 777
    lg = rng.standard_normal((1, V)).astype(np.float32)
    u = _uniforms(6, 1, 200, 1)
    dr = oracle.predraw(lg, "f32", np.array([-1], np.int32), np.array([0], np.int32), u)
    c = np.cumsum(softmax(lg[0].astype(np.float64)))
    ref = np.searchsorted(c, u[0, :, 0].astype(np.float64) * c[-1], side="right")
    ok = ~dr.band[0]
    assert np.all(dr.exit_node[0] == 0)
    np.testing.assert_array_equal(dr.bonus_token[0][ok], ref[ok])


def test_walk_follows_certain_draws():
    """Rows that put all mass on one token: the walk follows the drafted
    chain while each node's certain token is its child's, and stops at the
    first node whose certain token has no matching child."""
    V, D = 50, 9
    parents = np.array([-1] + list(range(D - 1)), np.int32)            # chain 0-1-..-8
    tokens = np.array([0] + [10 + i for i in range(1, D)], np.int32)
    lg = np.full((D, V), -30000.0, np.float32)
    for v in range(D - 1):
        lg[v, tokens[v + 1]] = 0.0          # node v certainly draws its child's token
    lg[D - 1, 3] = 0.0                      # the leaf draws token 3
    u = _uniforms(7, 1, 32, D)
    dr = oracle.predraw(lg, "f32", parents, tokens, u)
    assert np.all(dr.exit_node == D - 1) and np.all(dr.bonus_token == 3)
    lg[4, tokens[5]] = -30000.0
    lg[4, 7] = 0.0                          # node 4 now draws a token no child carries
    dr = oracle.predraw(lg, "f32", parents, tokens, u)
    assert np.all(dr.exit_node == 4) and np.all(dr.bonus_token == 7)


@pytest.mark.parametrize("seed", [21, 22])
def test_predraw_law_is_the_target_flow_law(seed):
    """Cor. 1: the oracle's predraw-and-follow, driven by 2^-24-grid
    uniforms, realises the enumerated joint law of (exit node, bonus)."""
    parents, tokens, lg = _small_case(seed)
    p = softmax(lg, axis=1)
    J = LT.exact_law(parents, tokens, p)
    n = 100_000
    u = _uniforms(seed + 100, 1, n, len(parents))
    dr = oracle.predraw(lg, "f64", parents, tokens, u)
    H = np.zeros_like(J)
    np.add.at(H, (dr.exit_node[0], dr.bonus_token[0]), 1.0)
    assert LT.chi2_pvalue(H, J) > 1e-4
    assert LT.tv_distance(H, J) < LT.mc_tv_floor(J, n, np.random.default_rng(seed))


def test_walk_matches_an_independent_follower():
    """Given the oracle's own node draws, a plain follower over the child
    lists reaches the same exit node and bonus token."""
    rng = np.random.default_rng(31)
    B, V = 40, 60
    parents, tokens = W.random_tree(B, V, rng)
    lg = rng.standard_normal((B, V)).astype(np.float32) * 2.0
    for u in range(1, B):
        lg[parents[u], tokens[u]] += 3.0
    uu = _uniforms(32, 1, 300, B)
    dr = oracle.predraw(lg, "f32", parents, tokens, uu)
    ch = LT.children_of(parents)
    for n in range(uu.shape[1]):
        v = 0
        while True:
            d = dr.node_draw[0, n, v]
            nxt = [c for c in ch[v] if tokens[c] == d]
            if not nxt:
                break
            v = nxt[0]
        assert dr.exit_node[0, n] == v and dr.bonus_token[0, n] == dr.node_draw[0, n, v]
