"""Pins of the oracle's cache commit ("CAST: Cost-Aware Speculative Trees
from One-Pass Block Drafters", App. B Lemma 1 and App. C "Packed
verification"): after the commit, attention of the accepted path as an
ordinary causal chain over the compacted cache reproduces the packed tree
attention of those nodes; the prefix and the rows past the path keep their
contents; the root-only and full-chain cases are identities.  CPU only."""
import numpy as np
import pytest

import oracle
from tests import workloads as W


def _case(seed, R=2, B=23, Hq=4, Hkv=2, D=64, P=37, L=2):
    rng = np.random.default_rng(seed)
    parents = np.stack([W.random_tree(B, 100, rng)[0] for _ in range(R)]).astype(np.int32)
    q = rng.standard_normal((R, B, Hq, D)).astype(np.float32)
    k = rng.standard_normal((L, R, Hkv, P + B, D)).astype(np.float32)
    v = rng.standard_normal((L, R, Hkv, P + B, D)).astype(np.float32)
    return parents, q, k, v, P


def _path(par, node):
    p = [node]
    while p[-1] != 0:
        p.append(int(par[p[-1]]))
    return p[::-1]


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_committed_path_attends_like_the_packed_tree(seed):
    """Lemma 1: each packed node attends exactly to the prefix and its root
    path.  So for the accepted path, causal attention over the committed
    cache (a chain of A + 1 rows after the prefix) equals the tree attention
    of the same nodes over the packed cache, in every layer."""
    parents, q, k, v, P = _case(seed)
    R, B = parents.shape
    D = q.shape[-1]
    rng = np.random.default_rng(seed + 10)
    exit_node = np.array([int(rng.integers(0, B)) for _ in range(R)], np.int32)
    k2, v2, nl = oracle.commit_kv(k, v, parents, exit_node, P)
    for r in range(R):
        path = _path(parents[r], int(exit_node[r]))
        assert nl[r] == P + len(path)
        A1 = len(path)
        chain = np.array([-1] + list(range(A1 - 1)), np.int32)
        for layer in range(k.shape[0]):
            tree_out = oracle.tree_attn(q[r:r + 1], k[layer, r:r + 1], v[layer, r:r + 1], "f32",
                                        parents[r:r + 1], P, 1.0 / np.sqrt(D))[0, path]
            kc = np.ascontiguousarray(k2[layer, r:r + 1, :, :P + A1])
            vc = np.ascontiguousarray(v2[layer, r:r + 1, :, :P + A1])
            chain_out = oracle.tree_attn(np.ascontiguousarray(q[r:r + 1, path]), kc, vc, "f32",
                                         chain[None], P, 1.0 / np.sqrt(D))[0]
            np.testing.assert_allclose(chain_out, tree_out, rtol=0, atol=1e-12)


def test_prefix_and_tail_rows_are_untouched():
    parents, q, k, v, P = _case(7)
    exit_node = np.array([5, 17], np.int32)
    k2, v2, nl = oracle.commit_kv(k, v, parents, exit_node, P)
    np.testing.assert_array_equal(k2[:, :, :, :P], k[:, :, :, :P])
    for r in range(2):
        np.testing.assert_array_equal(k2[:, r, :, nl[r]:], k[:, r, :, nl[r]:])
        np.testing.assert_array_equal(v2[:, r, :, nl[r]:], v[:, r, :, nl[r]:])


def test_root_only_and_full_chain_are_identities():
    parents, q, k, v, P = _case(8, R=1)
    k2, v2, nl = oracle.commit_kv(k, v, parents, np.array([0], np.int32), P)
    assert nl[0] == P + 1
    np.testing.assert_array_equal(k2, k)
    B = parents.shape[1]
    chain = np.array([[-1] + list(range(B - 1))], np.int32)
    k2, v2, nl = oracle.commit_kv(k, v, chain, np.array([B - 1], np.int32), P)
    assert nl[0] == P + B
    np.testing.assert_array_equal(k2, k)
    np.testing.assert_array_equal(v2, v)
