"""GPU parity of tev_exit_loss (exit-guided draft-tree loss, "Where Draft Trees
Lose Target Mass", Sec. 5 Eq. 14 / App. C.2 Eq. 66-67) against the oracle,
through the C ABI.

Tolerances, from the kernel's arithmetic: every slab term is 2^(fma(z, log2 e,
-offset)) in f32 with |argument| < 64 for the terms that matter, so each term
carries a relative error below ~3e-6 (argument rounding, log2 e in f32, the
exp2 instruction); per-thread f32 sums of 32 terms and the wave and block
levels add below 3e-6 more.  A row's logsumexp is therefore within ~6e-6 in
absolute terms; the tests allow 2e-5.  The loss is a weighted mean of
(lse - z) with exact z: within 2e-5 times the mean weight, plus 1e-6 relative.
A gradient element is Omega/N * softmax - (listed weights)/N, the softmax
carrying the same ~6e-6 relative error: allowed 3e-5 of (|g| + 2 |one-hot
part|), plus 1e-12 of the largest element.
"""
import numpy as np
import pytest
import torch

import oracle
from draft_tree_verification_amd import tev
from tests import workloads as W
from tests import gpu_parity as GP

pytestmark = pytest.mark.gpu

LSE_ABS = 2e-5
LOSS_W = 2e-5
LOSS_REL = 1e-6
GRAD_REL = 3e-5


def _random_case(seed, R, B, H_extra, V, dtype, scale=3.0, wmode="uniform"):
    rng = np.random.default_rng(seed)
    trees = [W.random_tree(B, V, rng) for _ in range(R)]
    parents = np.stack([t[0] for t in trees]).astype(np.int32)
    tokens = np.stack([t[1] for t in trees]).astype(np.int32)
    H = max(int(W.depths_of(parents[r]).max()) for r in range(R)) + H_extra
    H = max(H, 1)
    z = (rng.standard_normal((R, H, V)) * scale).astype(np.float32)
    if wmode == "uniform":
        w = rng.uniform(0.0, 1.0, size=(R, B)).astype(np.float32)
    else:                                   # a third of the weights exactly zero
        w = rng.uniform(0.0, 1.0, size=(R, B)).astype(np.float32)
        w[rng.uniform(size=(R, B)) < 1 / 3] = 0.0
    zs = z if dtype == "f32" else W.f32_to_bf16_bits(z)
    return zs, parents, tokens, w


def _gpu(zs, dtype, parents, tokens, w, with_grad=True, out=None):
    res = tev.tev_exit_loss(tev.to_device_logits(zs, dtype), tev.to_device_i32(parents),
                            tev.to_device_i32(tokens), torch.from_numpy(w).cuda(),
                            with_grad=with_grad, out=out)
    torch.cuda.synchronize()
    return res


def _one_hot_part(parents, tokens, w, H, V):
    """sum of w(v)/N at (row of v, x_v): the part of the gradient subtracted."""
    R, B = parents.shape
    fix = np.zeros((R, H, V))
    for r in range(R):
        d = W.depths_of(parents[r])
        for v in range(1, B):
            if w[r, v] != 0.0:
                fix[r, d[v] - 1, tokens[r, v]] += float(w[r, v])
    return fix / max(R * (B - 1), 1)


def _compare(res, ref, parents, tokens, w, check_grad=True):
    R, B = parents.shape
    lse = res.row_lse.cpu().numpy()
    np.testing.assert_allclose(lse, ref.row_lse, rtol=1e-6, atol=LSE_ABS)
    np.testing.assert_allclose(res.row_weight.cpu().numpy(), ref.row_weight, rtol=1e-6, atol=0)
    loss = float(res.loss.cpu()[0])
    mean_w = float(np.sum(np.abs(w[:, 1:].astype(np.float64)))) / max(R * (B - 1), 1)
    assert abs(loss - ref.loss) <= LOSS_W * mean_w + LOSS_REL * abs(ref.loss), (loss, ref.loss)
    if check_grad and res.grad is not None:
        g = res.grad.cpu().numpy().astype(np.float64)
        H, V = g.shape[1:]
        fix = _one_hot_part(parents, tokens, w, H, V)
        tol = GRAD_REL * (np.abs(ref.grad) + 2 * fix) + 1e-12 * np.abs(ref.grad).max()
        bad = np.abs(g - ref.grad) > tol
        assert not bad.any(), (f"{int(bad.sum())} gradient elements off; worst "
                               f"{np.max(np.abs(g - ref.grad) - tol)}")


CASES = [
    dict(R=2, B=19, H_extra=1, V=20000, dtype="bf16"),       # 3 slabs, ragged tail
    dict(R=3, B=37, H_extra=0, V=8192, dtype="f32"),          # exactly one slab
    dict(R=1, B=64, H_extra=2, V=24577, dtype="f32"),         # odd V: scalar loads
    dict(R=2, B=50, H_extra=0, V=1001, dtype="bf16"),         # V * 2 not 16-aligned: scalar loads
    dict(R=4, B=256, H_extra=0, V=9000, dtype="bf16"),        # the largest tree
    dict(R=5, B=9, H_extra=3, V=40000, dtype="bf16", wmode="zeros"),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"R{c['R']}_B{c['B']}_V{c['V']}_{c['dtype']}")
def test_exit_loss_matches_oracle(case):
    GP.log(f"[exit_loss] {case}")
    zs, parents, tokens, w = _random_case(seed=21, **case)
    dtype = case["dtype"]
    ref = oracle.exit_loss(zs, dtype, parents, tokens, w)
    res = _gpu(zs, dtype, parents, tokens, w)
    _compare(res, ref, parents, tokens, w)
    flags = tev.tev_read_device_status(res.workspace, 3, parents.shape[0], parents.shape[1], zs.shape[-1])
    assert not np.any(flags)
    # the loss alone (no gradient output) gives the same loss and rows
    res2 = _gpu(zs, dtype, parents, tokens, w, with_grad=False)
    assert float(res2.loss.cpu()[0]) == float(res.loss.cpu()[0])
    assert torch.equal(res2.row_lse, res.row_lse)


def test_shared_tokens_at_one_depth_and_vocab_edges():
    """Nodes of one depth under different parents may carry the same token:
    the gradient subtracts each weight at that one element.  Tokens 0 and
    V - 1 exercise the first and last element of a row."""
    V, H = 20000, 3
    parents = np.array([[-1, 0, 0, 1, 2, 1, 2, 3, 4]], np.int32)
    tokens = np.array([[5, 0, V - 1, 7, 7, V - 1, 0, 3, 3]], np.int32)
    w = np.array([[0.9, 0.1, 0.2, 0.3, 0.25, 0.05, 0.4, 0.6, 0.7]], np.float32)
    rng = np.random.default_rng(4)
    z = (rng.standard_normal((1, H, V)) * 2).astype(np.float32)
    for dtype in ("f32", "bf16"):
        zs = z if dtype == "f32" else W.f32_to_bf16_bits(z)
        ref = oracle.exit_loss(zs, dtype, parents, tokens, w)
        _compare(_gpu(zs, dtype, parents, tokens, w), ref, parents, tokens, w)


def test_root_only_and_unscored_rows():
    zs, parents, tokens, w = _random_case(seed=3, R=2, B=1, H_extra=2, V=5000, dtype="bf16")
    res = _gpu(zs, "bf16", parents, tokens, w)
    assert float(res.loss.cpu()[0]) == 0.0
    assert torch.count_nonzero(res.grad).item() == 0
    ref = oracle.exit_loss(zs, "bf16", parents, tokens, w)
    np.testing.assert_allclose(res.row_lse.cpu().numpy(), ref.row_lse, rtol=1e-6, atol=LSE_ABS)


def test_flagged_examples():
    """A NaN logit or a node deeper than H flags the example: its rows, its
    gradient rows and the loss are NaN; other examples' rows are untouched."""
    zs, parents, tokens, w = _random_case(seed=8, R=3, B=20, H_extra=0, V=12000, dtype="f32")
    ref = oracle.exit_loss(zs, "f32", parents, tokens, w)
    bad = zs.copy()
    bad[1, 0, 777] = np.nan
    res = _gpu(bad, "f32", parents, tokens, w)
    flags = tev.tev_read_device_status(res.workspace, 3, 3, 20, 12000)
    assert flags[1] & tev.TEV_FLAG_NONFINITE and flags[0] == 0 and flags[2] == 0
    assert np.isnan(float(res.loss.cpu()[0]))
    assert torch.isnan(res.row_lse[1]).all() and torch.isnan(res.grad[1]).all()
    np.testing.assert_allclose(res.row_lse[0].cpu().numpy(), ref.row_lse[0], atol=LSE_ABS)
    # a node deeper than the rows given
    H = zs.shape[1]
    deep = _gpu(zs[:, : H - 1].copy(), "f32", parents, tokens, w)
    flags = tev.tev_read_device_status(deep.workspace, 3, 3, 20, 12000)
    d = np.array([W.depths_of(parents[r]).max() for r in range(3)])
    np.testing.assert_array_equal((flags & tev.TEV_FLAG_TREE) != 0, d > H - 1)
    assert np.isnan(float(deep.loss.cpu()[0]))


def test_workspace_reuse_and_repeatability():
    """Two calls in a row on one workspace (the second smaller) match the
    oracle, and a repeated call is bit-identical."""
    a = _random_case(seed=30, R=3, B=40, H_extra=1, V=30000, dtype="bf16")
    b = _random_case(seed=31, R=2, B=12, H_extra=0, V=9000, dtype="bf16")
    ws = torch.empty(tev.tev_exit_loss_workspace_bytes(3, 40, a[0].shape[1], 30000),
                     dtype=torch.uint8, device="cuda")
    ws.fill_(0xAB)
    outs = []
    for zs, parents, tokens, w in (a, b):
        res = tev.tev_exit_loss(tev.to_device_logits(zs, "bf16"), tev.to_device_i32(parents),
                                tev.to_device_i32(tokens), torch.from_numpy(w).cuda(), workspace=ws)
        torch.cuda.synchronize()
        _compare(res, oracle.exit_loss(zs, "bf16", parents, tokens, w), parents, tokens, w)
        outs.append(res)
    zs, parents, tokens, w = b
    again = tev.tev_exit_loss(tev.to_device_logits(zs, "bf16"), tev.to_device_i32(parents),
                              tev.to_device_i32(tokens), torch.from_numpy(w).cuda(), workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(again.loss, outs[1].loss) and torch.equal(again.grad, outs[1].grad)


def _workload_case(name, requests=None):
    """A named workload's tree, its own draft rows, and the GPU exit law's
    exit masses as the weights (the loss consumes w from the exit law)."""
    wl = W.make_config(name, with_attention=False, requests=requests)
    zs = W.draft_rows(name, requests=requests)
    law = tev.tev_exit_law(tev.to_device_logits(wl.logits, wl.dtype), tev.to_device_i32(wl.parents),
                           tev.to_device_i32(wl.tokens))
    w = law.exit_mass.cpu().numpy().astype(np.float32)
    return zs, wl.parents, wl.tokens, w, wl.dtype


def test_qwen3_4b_tree_with_exit_law_weights():
    """1 example, B=64 over 16 draft rows of V=151936 bf16 (the single-request
    workload), weights = the GPU exit law's w(v)."""
    zs, parents, tokens, w, dtype = _workload_case("qwen3_4b")
    GP.log(f"[exit_loss] qwen3_4b R=1 B=64 H={zs.shape[1]} V={zs.shape[2]}")
    assert abs(float(np.sum(w)) - 1.0) < 1e-4          # the exit law sums to one
    ref = oracle.exit_loss(zs, dtype, parents, tokens, w)
    _compare(_gpu(zs, dtype, parents, tokens, w), ref, parents, tokens, w)


def test_batched_full_size_in_groups():
    """The 32-example batched workload at full size, in the launch the bench
    times: loss and every row's logsumexp against the oracle run on groups of
    4 examples (numerators add up across groups); the gradient of the first
    group's rows, rescaled from the group's node count to the batch's."""
    zs, parents, tokens, w, dtype = _workload_case("batched")
    R, H, V = zs.shape
    B = parents.shape[1]
    GP.log(f"[exit_loss] batched R={R} B={B} H={H} V={V}")
    res = _gpu(zs, dtype, parents, tokens, w)
    lse = res.row_lse.cpu().numpy()
    num = 0.0
    for g0 in range(0, R, 4):
        sl = slice(g0, g0 + 4)
        ref = oracle.exit_loss(zs[sl], dtype, parents[sl], tokens[sl], w[sl])
        num += ref.numerator
        np.testing.assert_allclose(lse[sl], ref.row_lse, rtol=1e-6, atol=LSE_ABS)
        np.testing.assert_allclose(res.row_weight[sl].cpu().numpy(), ref.row_weight, rtol=1e-6)
        if g0 == 0:
            scale = 4 / R                                  # group N = 4 (B-1), batch N = R (B-1)
            g = res.grad[sl].cpu().numpy().astype(np.float64)
            gref = ref.grad * scale
            fix = _one_hot_part(parents[sl], tokens[sl], w[sl], H, V) * scale
            tol = GRAD_REL * (np.abs(gref) + 2 * fix) + 1e-12 * np.abs(gref).max()
            assert not (np.abs(g - gref) > tol).any()
    loss_ref = num / (R * (B - 1))
    mean_w = float(np.sum(w[:, 1:].astype(np.float64))) / (R * (B - 1))
    assert abs(float(res.loss.cpu()[0]) - loss_ref) <= LOSS_W * mean_w + LOSS_REL * abs(loss_ref)


def _sweep_cases(n=16, seed=3104):
    rng = np.random.default_rng(seed)
    cases = []
    while len(cases) < n:
        c = dict(R=int(rng.integers(1, 7)), B=int(rng.choice([1, 2, 9, 33, 64, 65, 128, 256])),
                 H_extra=int(rng.integers(0, 3)),
                 V=int(rng.choice([int(rng.integers(300, 5000)), int(rng.integers(5000, 40000)), 8192, 8193])),
                 dtype="f32" if rng.random() < 0.4 else "bf16", scale=float(rng.choice([0.5, 3.0, 8.0])),
                 wmode=str(rng.choice(["uniform", "zeros"])))
        if c["R"] * (16 + c["H_extra"]) * c["V"] > 4_000_000:
            continue
        c["seed"] = int(rng.integers(1, 1 << 30))
        cases.append(c)
    return cases


SWEEP = _sweep_cases()


@pytest.mark.parametrize("case", SWEEP, ids=[f"sweep{i}" for i in range(len(SWEEP))])
def test_exit_loss_sweep(case):
    GP.log(f"[exit_loss] {case}")
    zs, parents, tokens, w = _random_case(**case)
    dtype = case["dtype"]
    ref = oracle.exit_loss(zs, dtype, parents, tokens, w)
    res = _gpu(zs, dtype, parents, tokens, w)
    _compare(res, ref, parents, tokens, w)
    flags = tev.tev_read_device_status(res.workspace, 3, parents.shape[0], parents.shape[1], zs.shape[-1])
    assert not np.any(flags)
