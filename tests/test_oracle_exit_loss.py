"""Pins of the oracle's exit-guided draft-tree loss ("Where Draft Trees Lose
Target Mass: Exit-Guided Speculative Decoding", Sec. 5 Eq. 14 and App. C.2
Eq. 66-67) and of its gradient.  CPU only.

What fixes the oracle here, other than its own formula:
  * the one-child case is the library's cross entropy (torch), and a general
    tree is a weighted sum of library cross entropies of the right rows;
  * App. C.2's rearrangement (one library logsumexp per row times the row's
    summed weight, minus a gather) equals the per-node sum;
  * rows with one finite logit make every log-probability 0 or -inf, so a
    wrong depth-to-row mapping shows as an infinite loss;
  * constant rows give log V per node (closed form);
  * adding a constant to a row changes nothing but its logsumexp;
  * the gradient matches central finite differences of the loss.
"""
import numpy as np
import pytest
import scipy.special
import torch

import oracle
from tests import workloads as W


def _case(seed, R=3, B=19, V=41, extra_rows=1, scale=3.0):
    rng = np.random.default_rng(seed)
    trees = [W.random_tree(B, V, rng) for _ in range(R)]
    parents = np.stack([t[0] for t in trees]).astype(np.int32)
    tokens = np.stack([t[1] for t in trees]).astype(np.int32)
    H = max(int(W.depths_of(parents[r]).max()) for r in range(R)) + extra_rows
    z = (rng.standard_normal((R, H, V)) * scale).astype(np.float32)
    w = rng.uniform(0.0, 1.0, size=(R, B)).astype(np.float32)
    return z, parents, tokens, w


def _depths(parents):
    return np.stack([W.depths_of(p) for p in parents])


def test_single_child_is_library_cross_entropy():
    """B = 2 (root and one drafted child) with weight 1: Eq. 14 is the mean
    cross entropy of the depth-1 rows at the drafted tokens."""
    rng = np.random.default_rng(5)
    R, H, V = 6, 2, 300
    z = (rng.standard_normal((R, H, V)) * 4).astype(np.float32)
    parents = np.tile(np.array([-1, 0], np.int32), (R, 1))
    tokens = np.stack([[0, int(rng.integers(0, V))] for _ in range(R)]).astype(np.int32)
    w = np.ones((R, 2), np.float32)
    got = oracle.exit_loss(z, "f32", parents, tokens, w)
    zt = torch.from_numpy(z.astype(np.float64))
    want = torch.nn.functional.cross_entropy(zt[:, 0, :], torch.from_numpy(tokens[:, 1]).long())
    assert got.loss == pytest.approx(float(want), rel=1e-13)
    np.testing.assert_allclose(got.row_lse, torch.logsumexp(zt, dim=-1).numpy(), rtol=1e-14)
    np.testing.assert_array_equal(got.row_weight, np.array([[1.0, 0.0]] * R))


@pytest.mark.parametrize("seed", [0, 1])
def test_tree_is_weighted_library_cross_entropy(seed):
    z, parents, tokens, w = _case(seed)
    R, B = parents.shape
    d = _depths(parents)
    zt = torch.from_numpy(z.astype(np.float64))
    total = 0.0
    for r in range(R):
        rows = zt[r, d[r, 1:] - 1]                             # row of node v: position depth(v)
        ce = torch.nn.functional.cross_entropy(rows, torch.from_numpy(tokens[r, 1:]).long(),
                                               reduction="none")
        total += float((torch.from_numpy(w[r, 1:].astype(np.float64)) * ce).sum())
    got = oracle.exit_loss(z, "f32", parents, tokens, w)
    assert got.numerator == pytest.approx(total, rel=1e-12)
    assert got.loss == pytest.approx(total / (R * (B - 1)), rel=1e-12)


@pytest.mark.parametrize("seed", [2, 3])
def test_per_row_rearrangement(seed):
    """App. C.2 Eq. 67: sum_m (sum of the row's weights) * logsumexp(z_m)
    minus the weighted gather of the drafted tokens' logits."""
    z, parents, tokens, w = _case(seed, R=4, B=37, V=64)
    R, B = parents.shape
    H = z.shape[1]
    d = _depths(parents)
    z64 = z.astype(np.float64)
    omega = np.zeros((R, H))
    gather = 0.0
    for r in range(R):
        np.add.at(omega[r], d[r, 1:] - 1, w[r, 1:].astype(np.float64))
        gather += float(np.sum(w[r, 1:] * z64[r, d[r, 1:] - 1, tokens[r, 1:]]))
    lse = scipy.special.logsumexp(z64, axis=-1)
    num = float(np.sum(omega * lse)) - gather
    got = oracle.exit_loss(z, "f32", parents, tokens, w)
    assert got.numerator == pytest.approx(num, rel=1e-12)
    np.testing.assert_allclose(got.row_weight, omega, rtol=1e-14)
    np.testing.assert_allclose(got.row_lse, lse, rtol=1e-14)


@pytest.mark.filterwarnings("ignore::RuntimeWarning")
def test_certain_rows_pin_the_depth_mapping():
    """Row d - 1 puts all its mass on the token of the chain's depth-d node:
    every -log q is 0.  Reading the row of depth d - 1 or d + 1 instead would
    meet a -inf logit and give an infinite loss."""
    H, V = 6, 50
    B = H + 1
    parents = np.arange(-1, H, dtype=np.int32)[None]           # chain 0 <- 1 <- ... <- H
    tok = np.array([[7, 3, 11, 3, 40, 0, 29]], np.int32)
    z = np.full((1, H, V), -np.inf, np.float32)
    for dd in range(1, B):
        z[0, dd - 1, tok[0, dd]] = 2.5 * dd
    w = np.linspace(0.1, 0.9, B).astype(np.float32)[None]
    got = oracle.exit_loss(z, "f32", parents, tok, w)
    assert got.loss == 0.0
    assert np.all(got.grad == 0.0)
    np.testing.assert_allclose(got.row_lse[0], 2.5 * np.arange(1, B))
    # an all -inf row scored by a node has no normaliser: the loss is NaN
    z2 = z.copy()
    z2[0, 2, :] = -np.inf
    assert np.isnan(oracle.exit_loss(z2, "f32", parents, tok, w).loss)


def test_constant_rows_closed_form():
    z, parents, tokens, w = _case(7, R=2, B=15, V=33)
    R, H, V = z.shape
    B = parents.shape[1]
    const = np.random.default_rng(1).uniform(-5, 5, size=(R, H, 1)).astype(np.float32)
    zc = np.broadcast_to(const, z.shape).copy()
    got = oracle.exit_loss(zc, "f32", parents, tokens, w)
    want = np.log(V) * float(np.sum(w[:, 1:].astype(np.float64))) / (R * (B - 1))
    assert got.loss == pytest.approx(want, rel=1e-14)
    np.testing.assert_allclose(got.row_lse, const[..., 0].astype(np.float64) + np.log(V), rtol=1e-14)
    # gradient: each node adds w (1/V - [a = x_v]) / N to its row
    d = _depths(parents)
    w64 = w.astype(np.float64)
    g = np.zeros((R, H, V))
    for r in range(R):
        for v in range(1, B):
            g[r, d[r, v] - 1] += w64[r, v] / V
            g[r, d[r, v] - 1, tokens[r, v]] -= w64[r, v]
    np.testing.assert_allclose(got.grad, g / (R * (B - 1)), rtol=1e-12, atol=1e-17)


def test_row_shift_invariance():
    z, parents, tokens, w = _case(9)
    z = z.astype(np.float64)                   # f64 storage: the shift is exact
    shift = np.random.default_rng(2).integers(-20, 20, size=z.shape[:2] + (1,)).astype(np.float64)
    a = oracle.exit_loss(z, "f64", parents, tokens, w)
    b = oracle.exit_loss(z + shift, "f64", parents, tokens, w)
    assert b.loss == pytest.approx(a.loss, rel=1e-12)
    np.testing.assert_allclose(b.row_lse, a.row_lse + shift[..., 0], rtol=1e-13)
    np.testing.assert_allclose(b.grad, a.grad, rtol=1e-9, atol=1e-15)


def test_gradient_matches_finite_differences():
    z, parents, tokens, w = _case(11, R=2, B=9, V=7)
    z64 = z.astype(np.float64)
    got = oracle.exit_loss(z64, "f64", parents, tokens, w)
    h = 1e-6
    fd = np.zeros_like(z64)
    for idx in np.ndindex(z64.shape):
        zp, zm = z64.copy(), z64.copy()
        zp[idx] += h
        zm[idx] -= h
        fd[idx] = (oracle.exit_loss(zp, "f64", parents, tokens, w).loss
                   - oracle.exit_loss(zm, "f64", parents, tokens, w).loss) / (2 * h)
    np.testing.assert_allclose(got.grad, fd, atol=1e-8)
    # the gradient of a row sums to zero (softmax minus one-hot per node)
    np.testing.assert_allclose(got.grad.sum(axis=-1), 0.0, atol=1e-15)


def test_zero_weights_and_empty_trees():
    z, parents, tokens, w = _case(13)
    z[0, 0, :] = -np.inf                       # an impossible row under zero weight
    z[0, 0, 0] = 0.0
    got = oracle.exit_loss(z, "f32", parents, tokens, np.zeros_like(w))
    assert got.loss == 0.0 and np.all(got.grad == 0.0) and np.all(got.row_weight == 0.0)
    root_only = oracle.exit_loss(z[:, :1], "f32", parents[:, :1], tokens[:, :1], w[:, :1])
    assert root_only.loss == 0.0 and root_only.numerator == 0.0


def test_bf16_widening_and_depth_limit():
    z, parents, tokens, w = _case(15)
    bits = W.f32_to_bf16_bits(z)
    a = oracle.exit_loss(bits, "bf16", parents, tokens, w)
    b = oracle.exit_loss(W.bf16_bits_to_f32(bits), "f32", parents, tokens, w)
    assert a.loss == b.loss
    H = int(_depths(parents).max())
    with pytest.raises(oracle.OracleError):
        oracle.exit_loss(z[:, :H - 1], "f32", parents, tokens, w)
