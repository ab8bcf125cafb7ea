"""Independent routes to the verification law, for pinning the oracle.

Nothing here is imported by the product.  These comparators follow the
pages' *procedures*, not the exit-law formulas the oracle evaluates:

* ``exact_law``: the target-flow definition of the exit node ("Where Draft
  Trees Lose Target Mass", Sec. 3.1): follow target tokens through matching
  children; the deepest matched node is the exit node and the token that
  leaves the tree is the bonus token.  Probabilities are accumulated over all
  token sequences, so no P, rho or w is used.
* ``mc_predraw``: predraw-and-follow (App. A.4.1): one independent target
  draw per node, follow the matching child, else stop and emit the draw.
* ``mc_seqres``: exact sequential residual verification (App. A.4.2):
  children tested one by one in a random order with residual renormalisation.
"""
from __future__ import annotations

import numpy as np
from scipy.special import softmax


def children_of(parents: np.ndarray) -> list[list[int]]:
    ch = [[] for _ in range(len(parents))]
    for u in range(1, len(parents)):
        ch[int(parents[u])].append(u)
    return ch


def node_probs(logits: np.ndarray, inv_temperature: float = 1.0) -> np.ndarray:
    """p_v over the vocabulary for every row, by the library softmax in fp64."""
    return softmax(np.asarray(logits, np.float64) * inv_temperature, axis=-1)


def exact_law(parents: np.ndarray, tokens: np.ndarray, p: np.ndarray) -> np.ndarray:
    """Joint law J[v, a] = Pr(exit node v, bonus token a) by target flow."""
    B, V = p.shape
    ch = children_of(parents)
    child_by_token = [{int(tokens[u]): u for u in ch[v]} for v in range(B)]
    J = np.zeros((B, V))
    stack = [(0, 1.0)]
    while stack:
        v, mass = stack.pop()
        for a in range(V):
            pa = mass * p[v, a]
            if pa == 0.0:
                continue
            u = child_by_token[v].get(a)
            if u is None:
                J[v, a] += pa          # the continuation leaves the tree at v
            else:
                stack.append((u, pa))  # it follows the drafted child
    return J


def _draw(rng: np.random.Generator, probs: np.ndarray, n: int) -> np.ndarray:
    c = np.cumsum(probs)
    return np.minimum(np.searchsorted(c, rng.random(n) * c[-1], side="right"), len(probs) - 1)


def mc_predraw(parents, tokens, p, n, rng) -> np.ndarray:
    """Histogram over (exit node, bonus) of n predraw-and-follow runs."""
    B, V = p.shape
    ch = children_of(parents)
    draws = np.stack([_draw(rng, p[v], n) for v in range(B)])    # R_v for every node
    node = np.zeros(n, np.int64)
    active = np.ones(n, bool)
    out_v = np.zeros(n, np.int64)
    out_y = np.zeros(n, np.int64)
    while active.any():
        idx = np.nonzero(active)[0]
        cur = node[idx]
        r = draws[cur, idx]
        nxt = np.full(len(idx), -1)
        for v in np.unique(cur):
            sel = cur == v
            for u in ch[v]:
                nxt[sel & (r == tokens[u])] = u
        stop = nxt < 0
        out_v[idx[stop]] = cur[stop]
        out_y[idx[stop]] = r[stop]
        node[idx[~stop]] = nxt[~stop]
        active[idx[stop]] = False
    H = np.zeros((B, V))
    np.add.at(H, (out_v, out_y), 1.0)
    return H


def mc_seqres(parents, tokens, p, n, rng) -> np.ndarray:
    """Histogram of n exact sequential-residual runs, children tested in a
    fresh random order at every visit."""
    B, V = p.shape
    ch = children_of(parents)
    H = np.zeros((B, V))
    for _ in range(n):
        v = 0
        while True:
            order = list(rng.permutation(ch[v])) if ch[v] else []
            g = p[v].copy()
            moved = False
            for u in order:
                x = tokens[u]
                if rng.random() < g[x]:
                    v = u
                    moved = True
                    break
                rest = 1.0 - g[x]
                g[x] = 0.0
                if rest > 0:
                    g = g / rest
            if moved:
                continue
            y = _draw(rng, g, 1)[0]
            H[v, y] += 1
            break
    return H


def chi2_pvalue(counts: np.ndarray, probs: np.ndarray, min_expected: float = 5.0) -> float:
    """Pearson chi-square goodness of fit, cells with small expectation pooled."""
    from scipy.stats import chi2
    counts = np.asarray(counts, np.float64).ravel()
    probs = np.asarray(probs, np.float64).ravel()
    n = counts.sum()
    exp = probs * n
    big = exp >= min_expected
    obs_c = list(counts[big])
    exp_c = list(exp[big])
    if (~big).any() and exp[~big].sum() > 0:
        obs_c.append(counts[~big].sum())
        exp_c.append(exp[~big].sum())
    obs_c = np.array(obs_c)
    exp_c = np.array(exp_c)
    stat = ((obs_c - exp_c) ** 2 / exp_c).sum()
    dof = max(1, len(obs_c) - 1)
    return float(chi2.sf(stat, dof))


def tv_distance(counts: np.ndarray, probs: np.ndarray) -> float:
    c = np.asarray(counts, np.float64).ravel()
    return 0.5 * float(np.abs(c / c.sum() - np.asarray(probs).ravel()).sum())


def mc_tv_floor(probs: np.ndarray, n: int, rng, reps: int = 50) -> float:
    """TV between the exact law and n-sample empirical draws from it: the
    Monte-Carlo floor a correct sampler sits at (the practice of "CAST" App. D.2,
    "Sampling distribution"), taken as the mean plus five standard deviations of
    the resampled TV so that a correct sampler fails with negligible odds."""
    p = np.asarray(probs).ravel()
    tvs = np.array([tv_distance(rng.multinomial(n, p / p.sum()), p) for _ in range(reps)])
    return float(tvs.mean() + 5.0 * tvs.std())
