"""Statistical and library pins for the oracle: TEV's draws, predraw-and-follow
and sequential residual Monte Carlo against the enumerated law, tree attention
against the library's scaled-dot-product attention, and the workload builders
against brute force.  CPU only."""
import itertools

import numpy as np
import pytest
import torch
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


# ---------------------------------------------------------------- Monte Carlo
@pytest.mark.parametrize("seed", [0, 1])
def test_tev_draws_follow_enumerated_law(seed):
    """Alg. 1's two draws, driven by 2^-24-grid uniforms, reproduce the joint
    target-flow law (Cor. 2, Eq. 56)."""
    parents, tokens, lg = _small_case(seed)
    p = softmax(lg, axis=1)
    J = LT.exact_law(parents, tokens, p)
    el = oracle.exit_law(lg, "f64", parents, tokens)
    n = 200_000
    u = W.uniforms_for(1000 + seed, 0, n)[None]
    dr = oracle.sample(lg, "f64", parents, tokens, el.exit_mass, u)
    H = np.zeros_like(J)
    np.add.at(H, (dr.exit_node[0], dr.bonus_token[0]), 1.0)
    assert LT.chi2_pvalue(H, J) > 1e-4
    assert LT.tv_distance(H, J) < LT.mc_tv_floor(J, n, np.random.default_rng(seed))


@pytest.mark.parametrize("seed", [2, 3])
def test_predraw_and_follow_has_the_same_law(seed):
    """Cor. 1 and App. A.4.1: predraw-and-follow realises the same law."""
    parents, tokens, lg = _small_case(seed)
    p = softmax(lg, axis=1)
    J = LT.exact_law(parents, tokens, p)
    el, n = oracle.exit_law(lg, "f64", parents, tokens), 400_000
    H = LT.mc_predraw(parents, tokens, p, n, np.random.default_rng(seed))
    assert LT.chi2_pvalue(H, J) > 1e-4
    assert LT.tv_distance(H, J) < LT.mc_tv_floor(J, n, np.random.default_rng(seed + 50))
    # the oracle's exit law is this law's marginal over exit nodes
    np.testing.assert_allclose(J.sum(axis=1), el.exit_mass[0], atol=1e-12)


@pytest.mark.parametrize("seed", [4])
def test_sequential_residual_has_the_same_law(seed):
    """Cor. 1 and App. A.4.2: exact sequential residual verification with a
    random child order at every visit realises the same law."""
    parents, tokens, lg = _small_case(seed, B=6, V=4)
    p = softmax(lg, axis=1)
    J = LT.exact_law(parents, tokens, p)
    n = 60_000
    H = LT.mc_seqres(parents, tokens, p, n, np.random.default_rng(seed))
    assert LT.chi2_pvalue(H, J) > 1e-4
    el = oracle.exit_law(lg, "f64", parents, tokens)
    np.testing.assert_allclose(J.sum(axis=1), el.exit_mass[0], atol=1e-12)


def test_tiny_config_draw_statistics():
    """Tiny workload, its 4096 uniform pairs: exit histogram against w
    (chi-square), mean block length against 1 + C (Cor. 2 Eq. 11, within 4
    standard errors) and subtree hit rates against P(u) (Eq. 58)."""
    wl = W.make_config("tiny", with_attention=False)
    el = oracle.exit_law(wl.logits, "f32", wl.parents, wl.tokens)
    dr = oracle.sample(wl.logits, "f32", wl.parents, wl.tokens, el.exit_mass, wl.uniforms)
    V = dr.exit_node[0]
    n = len(V)
    hist = np.bincount(V, minlength=wl.B)
    assert LT.chi2_pvalue(hist, el.exit_mass[0]) > 1e-4
    depth = W.depths_of(wl.parents[0])
    L = depth[V] + 1
    sd = np.sqrt((el.exit_mass[0] * (depth + 1 - (1 + el.coverage[0])) ** 2).sum() / n)
    assert abs(L.mean() - (1 + el.coverage[0])) < 4 * sd
    for u in range(1, wl.B):
        in_sub = np.array([_below(wl.parents[0], u, x) for x in range(wl.B)])
        rate = in_sub[V].mean()
        P = el.reach[0, u]
        assert abs(rate - P) < 4 * np.sqrt(P * (1 - P) / n) + 1e-9
    # the bonus token is never a drafted child of the exit node
    for x, y in zip(V, dr.bonus_token[0]):
        kids = wl.tokens[0][wl.parents[0] == x]
        assert y not in kids


def _below(parents, u, v):
    while v >= 0:
        if v == u:
            return True
        v = parents[v]
    return False


# ---------------------------------------------------------------- attention
def _sdpa_reference(q, k, v, mask, scale):
    """torch's scaled_dot_product_attention in fp64 on the CPU (library)."""
    return torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v),
        attn_mask=torch.from_numpy(mask), scale=scale).numpy()


def test_chain_tree_attention_is_causal_attention():
    """A chain tree reduces to causal attention over [prefix, chain]
    (CAST App. B Lemma 1): compared with the library's causal SDPA."""
    rng = np.random.default_rng(3)
    B, Hq, Hkv, D, P = 9, 4, 2, 16, 23
    parents = np.arange(-1, B - 1, dtype=np.int32)
    q = rng.standard_normal((1, B, Hq, D))
    k = rng.standard_normal((1, Hkv, P + B, D))
    v = rng.standard_normal((1, Hkv, P + B, D))
    out = oracle.tree_attn(q, k, v, "f64", parents, P, 0.25)
    G = Hq // Hkv
    qt = torch.from_numpy(q[0].transpose(1, 0, 2))                 # [Hq][B][D]
    kt = torch.from_numpy(np.repeat(k[0], G, axis=0))               # [Hq][P+B][D]
    vt = torch.from_numpy(np.repeat(v[0], G, axis=0))
    # causal over the full sequence, queries are its last B positions
    full_q = torch.zeros((Hq, P + B, D), dtype=torch.float64)
    full_q[:, P:] = qt
    ref = torch.nn.functional.scaled_dot_product_attention(full_q, kt, vt, is_causal=True, scale=0.25)
    np.testing.assert_allclose(out[0].transpose(1, 0, 2), ref[:, P:].numpy(), rtol=0, atol=1e-12)


@pytest.mark.parametrize("seed", [0, 1])
def test_tree_attention_rows_are_standalone_path_attention(seed):
    """Every row equals attention over [prefix, root path] alone, with the
    library's SDPA and an explicit dense mask (CAST App. C 'Packed
    verification'); kv head g serves q heads g*G .. g*G+G-1."""
    rng = np.random.default_rng(seed)
    B, Hq, Hkv, D, P = 14, 6, 2, 8, 11
    parents, _ = W.random_tree(B, 50, rng)
    q = rng.standard_normal((1, B, Hq, D))
    k = rng.standard_normal((1, Hkv, P + B, D))
    v = rng.standard_normal((1, Hkv, P + B, D))
    out = oracle.tree_attn(q, k, v, "f64", parents, P, 0.3)
    G = Hq // Hkv
    for i in range(B):
        path = []
        a = i
        while a >= 0:
            path.append(a)
            a = parents[a]
        keys = list(range(P)) + [P + j for j in sorted(path)]
        for h in range(Hq):
            g = h // G
            ref = _sdpa_reference(q[0, i, h][None, None], k[0, g, keys][None], v[0, g, keys][None],
                                  np.ones((1, 1, len(keys)), bool), 0.3)[0, 0]
            np.testing.assert_allclose(out[0, i, h], ref, rtol=0, atol=1e-12)
    # sampled-row interface returns the same rows
    rows = np.array([5, 17, 80], np.int64)
    sub = oracle.tree_attn(q, k, v, "f64", parents, P, 0.3, rows=rows)
    np.testing.assert_allclose(sub, out.reshape(-1, D)[rows], rtol=0, atol=0)


def test_tree_attention_bf16_widening_is_exact():
    rng = np.random.default_rng(9)
    B, Hq, Hkv, D, P = 5, 2, 1, 8, 4
    parents = np.array([-1, 0, 0, 1, 1], np.int32)
    qf = rng.standard_normal((1, B, Hq, D)).astype(np.float32)
    kf = rng.standard_normal((1, Hkv, P + B, D)).astype(np.float32)
    vf = rng.standard_normal((1, Hkv, P + B, D)).astype(np.float32)
    qb, kb, vb = (W.f32_to_bf16_bits(x) for x in (qf, kf, vf))
    out_b = oracle.tree_attn(qb, kb, vb, "bf16", parents, P, 0.5)
    out_f = oracle.tree_attn(*(W.bf16_bits_to_f32(x).astype(np.float64) for x in (qb, kb, vb)),
                             "f64", parents, P, 0.5)
    np.testing.assert_array_equal(out_b, out_f)


# ---------------------------------------------------------------- builders
def _brute_topB(logq_modes, B, log_prior):
    """All prefixes up to depth L, best-mode score, keep the B-1 best."""
    Km, L, V = logq_modes.shape
    scored = []
    for d in range(1, L + 1):
        for seq in itertools.product(range(V), repeat=d):
            s = max(log_prior[k] + sum(logq_modes[k, j, seq[j]] for j in range(d)) for k in range(Km))
            scored.append((-s, d, seq))
    scored.sort()
    return {seq for _, _, seq in scored[:B - 1]}


def _tree_prefixes(parents, tokens):
    seqs = [()] * len(parents)
    for i in range(1, len(parents)):
        seqs[i] = seqs[parents[i]] + (int(tokens[i]),)
    return seqs


@pytest.mark.parametrize("seed", range(40))
def test_best_first_builder_is_exact_topB(seed):
    """Top-B prefixes of a product (CAST Thm. 1 / App. C builder): the set is
    prefix-closed, in topological order, and equals brute force."""
    rng = np.random.default_rng(seed)
    L, V = int(rng.integers(1, 4)), int(rng.integers(2, 6))
    B = int(rng.integers(2, min(20, sum(V ** d for d in range(1, L + 1))) + 2))
    q = softmax(rng.standard_normal((L, V)) * 2, axis=1)
    parents, tokens = W.best_first_tree(q, B)
    seqs = _tree_prefixes(parents, tokens)
    assert all(parents[i] < i for i in range(1, len(parents)))
    want = _brute_topB(np.log(q)[None], B, np.zeros(1))
    assert set(seqs[1:]) == want


@pytest.mark.parametrize("seed", range(60))
def test_merged_heap_is_exact_topB_under_best_mode_score(seed):
    """Multi-Future Drafting Prop. 6: the merged heap returns the B distinct
    prefixes with the largest best-mode score; with one mode it is the
    best-first builder node for node."""
    rng = np.random.default_rng(1000 + seed)
    Km, L, V = int(rng.integers(1, 5)), int(rng.integers(1, 4)), int(rng.integers(2, 5))
    B = int(rng.integers(2, min(25, sum(V ** d for d in range(1, L + 1))) + 2))
    qs = softmax(rng.standard_normal((Km, L, V)) * 2, axis=2)
    prior = np.log(softmax(rng.standard_normal(Km))) if seed % 2 else np.full(Km, -np.log(Km))
    parents, tokens = W.merged_heap_tree(qs, B, prior)
    seqs = _tree_prefixes(parents, tokens)
    assert len(set(seqs)) == len(seqs)
    assert set(seqs[1:]) == _brute_topB(np.log(qs), B, prior)
    if Km == 1:
        p1, t1 = W.best_first_tree(qs[0], B)
        np.testing.assert_array_equal(p1, parents)
        np.testing.assert_array_equal(t1[1:], tokens[1:])
