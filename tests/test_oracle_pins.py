"""Pins for the CPU oracle: values, closed forms, invariants, special cases and
brute force fixed by the pages and by mathematics -- never the oracle's own
formulas retyped.  All CPU-only."""
import itertools
import json
import os

import numpy as np
import pytest
from scipy.special import logsumexp, softmax

import oracle
from tests import workloads as W
from tests import lawtools as LT

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
NEG = -30000.0   # exp(-30000) underflows to exactly 0 in fp64


def _law_from_oracle(logits, parents, tokens, s=1.0):
    """J[v, a] = w(v) p_v^res(a) assembled from the oracle's outputs."""
    B, V = logits.shape
    el = oracle.exit_law(logits.astype(np.float64), "f64", parents, tokens, s)
    J = np.zeros((B, V))
    for v in range(B):
        w = el.exit_mass[0, v]
        if w <= 0:
            continue
        cdf = oracle.residual_cdf(logits.astype(np.float64), "f64", parents, tokens, v, s)
        J[v] = w * np.diff(np.concatenate([[0.0], cdf]))
    return el, J


# ---------------------------------------------------------------- worked examples
def _two_future_case(fx, case):
    V = fx["V"]
    f1, f2 = fx["f1"], fx["f2"]
    parents, tokens, kind = [-1], [0], ["root"]
    prev = 0
    for d in range(case["depth_f1"]):
        parents.append(prev); tokens.append(f1[d]); kind.append(("f1", d + 1)); prev = len(parents) - 1
    prev = 0
    for d in range(case["depth_f2"]):
        parents.append(prev); tokens.append(f2[d]); kind.append(("f2", d + 1)); prev = len(parents) - 1
    B = len(parents)
    lg = np.full((B, V), NEG, np.float32)
    for i, k in enumerate(kind):
        if k == "root":
            lg[i, f1[0]] = 0.0
            lg[i, f2[0]] = np.float32(np.log(fx["masses"][1] / fx["masses"][0]))
        else:
            fut = f1 if k[0] == "f1" else f2
            lg[i, fut[k[1]]] = 0.0
    return np.array(parents, np.int32), np.array(tokens, np.int32), lg, kind


@pytest.mark.parametrize("case_idx", [0, 1])
def test_two_futures_printed_values(case_idx):
    """Multi-Future Drafting, 'Unequal futures' (App. A): 13.5 and 7.9."""
    with open(os.path.join(GOLDEN, "two_futures.json")) as f:
        fx = json.load(f)
    case = fx["cases"][case_idx]
    parents, tokens, lg, kind = _two_future_case(fx, case)
    assert len(parents) == 16
    el = oracle.exit_law(lg, "f32", parents, tokens)
    # f32 log(1/9) carries ~3e-8 relative error into the 0.9/0.1 split
    assert el.coverage[0] == pytest.approx(case["coverage"], abs=1e-6)
    w = el.exit_mass[0]
    leaf1 = max(i for i, k in enumerate(kind) if k != "root" and k[0] == "f1")
    assert w[0] == pytest.approx(case["exit_mass"]["root"], abs=1e-7)
    assert w[leaf1] == pytest.approx(case["exit_mass"]["f1_leaf"], abs=1e-7)
    if "f2_leaf" in case["exit_mass"]:
        leaf2 = max(i for i, k in enumerate(kind) if k != "root" and k[0] == "f2")
        assert w[leaf2] == pytest.approx(case["exit_mass"]["f2_leaf"], abs=1e-7)
    # every other node passes all its mass on
    others = [i for i in range(16) if i not in (0, leaf1) and not (
        "f2_leaf" in case["exit_mass"] and i == max(j for j, k in enumerate(kind) if k != "root" and k[0] == "f2"))]
    assert np.all(np.abs(w[others]) < 1e-12)


@pytest.mark.parametrize("M,D", [(2, 4), (3, 5), (4, 3)])
def test_separation_model_closed_form(M, D):
    """Multi-Future Drafting Prop. 2(i): M equal futures differing everywhere,
    a tree holding all of them to depth D accepts D in expectation."""
    V = M * D + 3
    fut = [[1 + m * D + d for d in range(D)] for m in range(M)]
    parents, tokens, kind = [-1], [0], ["root"]
    for m in range(M):
        prev = 0
        for d in range(D):
            parents.append(prev); tokens.append(fut[m][d]); kind.append((m, d)); prev = len(parents) - 1
    B = len(parents)
    lg = np.full((B, V), NEG)
    for i, k in enumerate(kind):
        if k == "root":
            for m in range(M):
                lg[i, fut[m][0]] = 0.0
        else:
            m, d = k
            lg[i, fut[m][d + 1] if d + 1 < D else 0] = 0.0   # after the block: any token
    el = oracle.exit_law(lg, "f64", np.array(parents), np.array(tokens))
    assert el.coverage[0] == pytest.approx(D, abs=1e-12)


# ---------------------------------------------------------------- invariants
def _random_case(seed, B, V, sigma=2.0, boost=2.0):
    rng = np.random.default_rng(seed)
    parents, tokens = W.random_tree(B, V, rng)
    lg = rng.standard_normal((B, V)) * sigma
    for u in range(1, B):
        lg[parents[u], tokens[u]] += boost
    return parents, tokens, lg


@pytest.mark.parametrize("seed", range(6))
def test_exit_law_invariants(seed):
    """Lemma 1 (sum w = 1), Eq. 24-26 (local and subtree conservation),
    Eq. 6 (two forms of C) and rho = 1 at leaves."""
    B, V = 30, 50
    parents, tokens, lg = _random_case(seed, B, V)
    el = oracle.exit_law(lg, "f64", parents, tokens, 1.0)
    P, w, rho = el.reach[0], el.exit_mass[0], el.rho[0]
    ch = LT.children_of(parents)
    assert w.sum() == pytest.approx(1.0, abs=1e-12)
    for v in range(B):
        assert w[v] + sum(P[u] for u in ch[v]) == pytest.approx(P[v], abs=1e-12)
        if not ch[v]:
            assert rho[v] == 1.0
    # subtree sums: sum_{v below u} w(v) = P(u)
    depth = W.depths_of(parents)
    for u in range(B):
        sub = [v for v in range(B) if _is_ancestor(parents, u, v)]
        assert sum(w[v] for v in sub) == pytest.approx(P[u], abs=1e-12)
    assert el.coverage[0] == pytest.approx((w * depth).sum(), abs=1e-12)
    assert el.coverage[0] == pytest.approx(P[1:].sum(), abs=1e-12)


def _is_ancestor(parents, u, v):
    while v >= 0:
        if v == u:
            return True
        v = parents[v]
    return False


def test_log_normaliser_matches_library():
    parents, tokens, lg = _random_case(11, 12, 3000, sigma=5.0)
    el = oracle.exit_law(lg, "f64", parents, tokens, 0.7)
    np.testing.assert_allclose(el.logZ[0], logsumexp(lg * 0.7, axis=1), rtol=0, atol=1e-11)


def test_child_probabilities_and_rho_match_library_softmax():
    """rho(v) against 1 - sum of children under scipy's softmax; P along a path
    against a product of scipy softmax entries."""
    parents, tokens, lg = _random_case(12, 20, 400, sigma=3.0, boost=5.0)
    p = softmax(lg, axis=1)
    el = oracle.exit_law(lg, "f64", parents, tokens)
    ch = LT.children_of(parents)
    for v in range(20):
        want = 1.0 - sum(p[v, tokens[u]] for u in ch[v])
        assert el.rho[0, v] == pytest.approx(want, abs=1e-12)
    for u in range(1, 20):
        prod, a = 1.0, u
        while a > 0:
            prod *= p[parents[a], tokens[a]]
            a = parents[a]
        assert el.reach[0, u] == pytest.approx(prod, rel=1e-12)


# ---------------------------------------------------------------- brute force
def _all_trees(n_nodes):
    """Every parent array with parents[i] < i (root first)."""
    for pars in itertools.product(*[range(i) for i in range(1, n_nodes)]):
        yield np.array((-1,) + pars, np.int32)


def test_exact_law_matches_target_flow_enumeration():
    """The oracle's w(v) p_v^res(a) equals the target-flow law, enumerated
    through the tree without using P, rho or w (Sec. 3.1 definition of the exit
    node; Thm. 1 Eq. 10), on every tree shape with up to 5 nodes."""
    rng = np.random.default_rng(7)
    V = 5
    checked = 0
    for n in range(1, 6):
        for parents in _all_trees(n):
            ch = LT.children_of(parents)
            if max(len(c) for c in ch) > V:
                continue
            tokens = np.zeros(n, np.int32)
            for v in range(n):
                toks = rng.choice(V, size=len(ch[v]), replace=False)
                for u, t in zip(ch[v], toks):
                    tokens[u] = t
            lg = rng.standard_normal((n, V)) * 1.5
            p = softmax(lg, axis=1)
            J_flow = LT.exact_law(parents, tokens, p)
            el, J = _law_from_oracle(lg, parents, tokens)
            np.testing.assert_allclose(J, J_flow, rtol=0, atol=1e-12)
            assert J_flow.sum() == pytest.approx(1.0, abs=1e-12)
            checked += 1
    assert checked == 1 + 1 + 2 + 6 + 24


def test_inverse_temperature_enters_as_logit_scale():
    parents, tokens, lg = _random_case(3, 8, 6, sigma=1.0)
    s = 0.37
    el, J = _law_from_oracle(lg, parents, tokens, s)
    J_flow = LT.exact_law(parents, tokens, softmax(lg * s, axis=1))
    np.testing.assert_allclose(J, J_flow, rtol=0, atol=1e-12)


# ---------------------------------------------------------------- special cases
def test_root_only_tree_is_inverse_cdf_sampling():
    """B = 1: w(r) = 1, C = 0 and the bonus draw is plain inverse-CDF sampling
    of p_r (numpy searchsorted on the library softmax)."""
    rng = np.random.default_rng(5)
    V = 700
    lg = (rng.standard_normal((1, V)) * 3).astype(np.float32)
    parents = np.array([-1], np.int32); tokens = np.array([3], np.int32)
    el = oracle.exit_law(lg, "f32", parents, tokens)
    assert el.exit_mass[0, 0] == 1.0 and el.coverage[0] == 0.0 and el.rho[0, 0] == 1.0
    u = W.uniforms_for(99, 0, 2000)[None]
    dr = oracle.sample(lg, "f32", parents, tokens, el.exit_mass, u)
    p = softmax(lg[0].astype(np.float64))
    c = np.cumsum(p)
    want = np.searchsorted(c, u[0, :, 1].astype(np.float64) * c[-1], side="right")
    ok = ~dr.band_bonus[0]
    assert np.all(dr.exit_node == 0)
    np.testing.assert_array_equal(dr.bonus_token[0][ok], want[ok])


def test_chain_is_textbook_speculative_sampling():
    """A chain whose draft is a point mass on each drafted token: the law is
    textbook speculative sampling (accept x with prob min(1, p(x)/q(x)) = p(x),
    else resample from max(0, p - q) renormalised)."""
    rng = np.random.default_rng(21)
    V, k = 7, 4
    parents = np.arange(-1, k, dtype=np.int32)
    tokens = np.concatenate([[0], rng.integers(0, V, k)]).astype(np.int32)
    lg = rng.standard_normal((k + 1, V))
    p = softmax(lg, axis=1)
    J_text = np.zeros((k + 1, V))
    alive = 1.0
    for j in range(k + 1):
        if j == k:                                  # no draft left: plain sample
            J_text[j] += alive * p[j]
            break
        q = np.zeros(V); q[tokens[j + 1]] = 1.0
        x = tokens[j + 1]
        acc = min(1.0, p[j, x] / q[x])
        resid = np.maximum(0.0, p[j] - q)
        if resid.sum() > 0:
            J_text[j] += alive * (1 - acc) * resid / resid.sum()
        alive *= acc
    el, J = _law_from_oracle(lg, parents, tokens)
    np.testing.assert_allclose(J, J_text, rtol=0, atol=1e-12)


def test_sibling_order_invariance():
    """Another valid node order (siblings permuted, subtrees interleaved)
    leaves rho, P and w of every node identity unchanged (Sec. 4
    'Efficiency': TEV is sibling-order invariant)."""
    parents, tokens, lg = _random_case(31, 25, 60)
    el = oracle.exit_law(lg, "f64", parents, tokens)
    rng = np.random.default_rng(0)
    for _ in range(5):
        # random topological order: repeatedly pick a random available node
        B = len(parents)
        ch = LT.children_of(parents)
        order, avail = [0], list(ch[0])
        while avail:
            j = avail.pop(rng.integers(0, len(avail)))
            order.append(j)
            avail.extend(ch[j])
        pos = {old: new for new, old in enumerate(order)}
        p2 = np.array([-1] + [pos[parents[o]] for o in order[1:]], np.int32)
        t2 = tokens[order]
        el2 = oracle.exit_law(lg[order], "f64", p2, t2)
        np.testing.assert_allclose(el2.exit_mass[0], el.exit_mass[0][order], rtol=0, atol=1e-14)
        np.testing.assert_allclose(el2.reach[0], el.reach[0][order], rtol=0, atol=1e-14)
        assert el2.coverage[0] == pytest.approx(el.coverage[0], abs=1e-13)


# ---------------------------------------------------------------- conventions
def test_inverse_cdf_convention_and_band():
    """Strict '<' against u * total, index order, zero-mass nodes never drawn."""
    V = 4
    parents = np.array([-1, 0, 0], np.int32)
    tokens = np.array([0, 1, 2], np.int32)
    # root: p = (1/4, 1/4, 1/4, 1/4); children take tokens 1, 2 -> rho(root) = 1/2
    lg = np.zeros((3, V))
    el = oracle.exit_law(lg, "f64", parents, tokens)
    np.testing.assert_allclose(el.exit_mass[0], [0.5, 0.25, 0.25], atol=1e-15)
    u = np.array([[[0.5, 0.5], [0.49, 0.25], [0.75, 0.99], [0.1, 0.3]]], np.float32)
    dr = oracle.sample(lg, "f64", parents, tokens, el.exit_mass, u)
    # u1 = 0.5 hits W_0/S = 0.5 exactly: not '<', so node 1; band flagged
    assert dr.exit_node[0, 0] == 1 and dr.band_exit[0, 0]
    assert dr.exit_node[0, 1] == 0 and not dr.band_exit[0, 1]
    assert dr.exit_node[0, 2] == 2 and dr.exit_node[0, 3] == 0
    # root residual keeps tokens {0, 3}: CDF (0.5, 0.5, 0.5, 1.0)
    assert dr.bonus_token[0, 1] == 0       # u2 = 0.25 < 0.5
    assert dr.bonus_token[0, 3] == 0
    assert dr.bonus_token[0, 0] in (0, 1, 2, 3)
    # leaves keep their full row: u2 = 0.99 -> token 3
    assert dr.bonus_token[0, 2] == 3


def test_zero_mass_nodes_never_drawn():
    V = 3
    parents = np.array([-1, 0, 0, 0], np.int32)
    tokens = np.array([0, 0, 1, 2], np.int32)     # children cover the whole vocabulary
    lg = np.random.default_rng(2).standard_normal((4, V))
    el = oracle.exit_law(lg, "f64", parents, tokens)
    assert el.exit_mass[0, 0] == pytest.approx(0.0, abs=1e-15)
    u = W.uniforms_for(5, 0, 3000)[None]
    dr = oracle.sample(lg, "f64", parents, tokens, el.exit_mass, u)
    assert np.all(dr.exit_node[0] != 0)


def test_invalid_inputs_are_rejected():
    lg = np.zeros((3, 4))
    with pytest.raises(oracle.OracleError):
        oracle.exit_law(lg, "f64", np.array([-1, 0, 3]), np.array([0, 1, 2]))   # parent after child
    with pytest.raises(oracle.OracleError):
        oracle.exit_law(lg, "f64", np.array([-1, 0, 0]), np.array([0, 1, 1]))   # duplicate siblings
    with pytest.raises(oracle.OracleError):
        oracle.exit_law(lg, "f64", np.array([-1, 0, 0]), np.array([0, 1, 9]))   # token out of range
    bad = lg.copy(); bad[1, 2] = np.nan
    with pytest.raises(oracle.OracleError):
        oracle.exit_law(bad, "f64", np.array([-1, 0, 0]), np.array([0, 1, 2]))
    neg = np.full((3, 4), -np.inf)
    with pytest.raises(oracle.OracleError):
        oracle.exit_law(neg, "f64", np.array([-1, 0, 0]), np.array([0, 1, 2]))


def test_neg_inf_logits_mean_zero_probability():
    lg = np.array([[0.0, -np.inf, 0.0, -np.inf], [0.0, 0.0, 0.0, 0.0]])
    parents = np.array([-1, 0], np.int32); tokens = np.array([0, 2], np.int32)
    el = oracle.exit_law(lg, "f64", parents, tokens)
    assert el.rho[0, 0] == pytest.approx(0.5, abs=1e-15)
    cdf = oracle.residual_cdf(lg, "f64", parents, tokens, 0)
    np.testing.assert_allclose(cdf, [1.0, 1.0, 1.0, 1.0])
