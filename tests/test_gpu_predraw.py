"""GPU parity of tev_predraw (predraw-and-follow verification, "Where Draft
Trees Lose Target Mass", App. A.4.1) against the oracle, through the C ABI:
every node's draw bit-exact outside the 1e-6 band of its bin, and the walk's
exit node and bonus token equal wherever no draw on the walked path is in the
band."""
import numpy as np
import pytest
import torch

import oracle
from draft_tree_verification_amd import tev
from tests import workloads as W
from tests import gpu_parity as GP

pytestmark = pytest.mark.gpu


def _uniforms(seed, R, n, B):
    k = np.random.default_rng(seed).integers(0, 1 << 24, size=(R, n, B))
    return (k.astype(np.float64) * 2.0 ** -24).astype(np.float32)


def _check(wl, n=64, seed=0):
    lg, par, tok, _ = GP.device_inputs(wl)
    res = tev.tev_exit_law(lg, par, tok, wl.inv_temperature)
    u = _uniforms(seed, wl.R, n, wl.B)
    nd, en, bt = tev.tev_predraw(lg, par, tok, res.workspace, torch.from_numpy(u).cuda(),
                                 wl.inv_temperature)
    torch.cuda.synchronize()
    nd, en, bt = nd.cpu().numpy(), en.cpu().numpy(), bt.cpu().numpy()
    ora = oracle.predraw(wl.logits, wl.dtype, wl.parents, wl.tokens, u, wl.inv_temperature)
    # node draws: equal wherever the node's uniform is not within 1e-6 of a
    # boundary of its bin (the oracle's per-node band, from its row CDF)
    same = nd == ora.node_draw
    mism = np.argwhere(~same & ~ora.node_band)
    assert len(mism) == 0, (f"{len(mism)} node draws differ outside the band; first "
                            f"{[(tuple(i), nd[tuple(i)], ora.node_draw[tuple(i)]) for i in mism[:5]]}")
    ok = ~ora.band
    np.testing.assert_array_equal(en[ok], ora.exit_node[ok])
    np.testing.assert_array_equal(bt[ok], ora.bonus_token[ok])
    # every emitted (exit, bonus) is a valid outcome of the walk over the GPU's own draws
    for r in range(wl.R):
        for d in range(n):
            v = 0
            while True:
                nxt = [u_ for u_ in range(1, wl.B) if wl.parents[r, u_] == v and wl.tokens[r, u_] == nd[r, d, v]]
                if not nxt:
                    break
                v = nxt[0]
            assert en[r, d] == v and bt[r, d] == nd[r, d, v]
    return int(ora.node_band.sum()), int((~ok).sum())


CASES = [
    dict(name="f32_small", R=2, B=24, V=3000, dtype="f32", tree="random"),
    dict(name="bf16_ragged", R=2, B=37, V=20008, dtype="bf16", tree="best_first"),
    dict(name="bf16_unaligned", R=1, B=30, V=20003, dtype="bf16", tree="random"),
    dict(name="chain_max_nodes", R=1, B=256, V=9000, dtype="f32", tree="chain"),
    dict(name="root_only", R=3, B=1, V=12000, dtype="bf16", tree="random"),
]


@pytest.mark.parametrize("case", CASES, ids=[c["name"] for c in CASES])
def test_predraw_small(case):
    c = dict(case)
    name = c.pop("name")
    GP.log(f"[predraw] {name} {c}")
    wl = W.make_custom(name, with_attention=False, n_uniform=1, **c)
    diff, band = _check(wl)
    GP.log(f"[predraw] {name} ok: {diff} node draws in the band, {band} walks excluded")


def test_predraw_qwen3_4b():
    GP.log("[predraw] workload qwen3_4b")
    wl = W.make_config("qwen3_4b", with_attention=False, n_uniform=1)
    diff, band = _check(wl, n=16, seed=1)
    GP.log(f"[predraw] qwen3_4b ok: {diff} node draws in the band, {band} walks excluded")


def test_predraw_flags_invalid_requests():
    wl = W.make_custom("bad", R=2, B=12, V=9000, dtype="bf16", tree="random", with_attention=False,
                       n_uniform=1)
    wl.logits[1, 3, 5] = 0x7FC0   # a NaN logit in request 1
    lg, par, tok, _ = GP.device_inputs(wl)
    res = tev.tev_exit_law(lg, par, tok)
    u = torch.from_numpy(_uniforms(3, 2, 8, 12)).cuda()
    nd, en, bt = tev.tev_predraw(lg, par, tok, res.workspace, u)
    torch.cuda.synchronize()
    assert np.all(nd[1].cpu().numpy() == -1) and np.all(en[1].cpu().numpy() == -1)
    assert np.all(en[0].cpu().numpy() >= 0)


def _sweep_cases(n=16, seed=3102):
    rng = np.random.default_rng(seed)
    cases = []
    while len(cases) < n:
        R = int(rng.integers(1, 7))
        B = int(rng.choice([1, 2, 9, 33, 64, 65, 128]))
        V = int(rng.choice([int(rng.integers(500, 5000)), int(rng.integers(5000, 40000)), 4097, 8191]))
        tree = str(rng.choice(["random", "chain", "star", "best_first"] if B >= 3 else ["random"]))
        dtype = "f32" if rng.random() < 0.3 else "bf16"
        if R * B * V > 8_000_000:
            continue
        cases.append(dict(name=f"sweep{len(cases)}", R=R, B=B, V=V, tree=tree, dtype=dtype,
                          seed=int(rng.integers(1, 1 << 30))))
    return cases


SWEEP = _sweep_cases()


@pytest.mark.parametrize("case", SWEEP, ids=[c["name"] for c in SWEEP])
def test_predraw_sweep(case):
    c = dict(case)
    name = c.pop("name")
    GP.log(f"[predraw] {name} {c}")
    wl = W.make_custom(name, with_attention=False, n_uniform=1, **c)
    _check(wl, n=16, seed=c["seed"])
