"""GPU parity of tev_exit_law and tev_sample against the CPU oracle (called
through the C ABI).  Small cases span several 4096-token chunks and a ragged
tail; the named workloads run at full size."""
import numpy as np
import pytest
import torch

import oracle
from draft_tree_verification_amd import tev
from tests import workloads as W
from tests import gpu_parity as GP

pytestmark = pytest.mark.gpu


SMALL = [
    dict(name="random_f32_ragged", R=3, B=37, V=20000, dtype="f32", tree="random"),
    dict(name="random_bf16_ragged", R=2, B=45, V=20008, dtype="bf16", tree="random"),
    dict(name="random_bf16_unaligned", R=2, B=30, V=20003, dtype="bf16", tree="random"),
    dict(name="random_f32_unaligned", R=1, B=20, V=9001, dtype="f32", tree="random"),
    dict(name="star_bf16_max_nodes", R=1, B=256, V=30000, dtype="bf16", tree="star"),
    dict(name="chain_f32_max_depth", R=1, B=256, V=9000, dtype="f32", tree="chain"),
    dict(name="best_first_bf16", R=2, B=64, V=17000, dtype="bf16", tree="best_first"),
    dict(name="root_only", R=2, B=1, V=12000, dtype="f32", tree="random"),
    dict(name="temperature", R=1, B=40, V=16384, dtype="bf16", tree="random", inv_temperature=0.6),
    dict(name="small_vocab", R=4, B=9, V=37, dtype="f32", tree="random"),
]


@pytest.mark.parametrize("case", SMALL, ids=[c["name"] for c in SMALL])
def test_small_cases(case):
    c = dict(case)
    name = c.pop("name")
    GP.log(f"[exit-law] {name} {c}")
    wl = W.make_custom(name, with_attention=False, n_uniform=1024, **c)
    rep = GP.check_exit_law_and_draws(wl)
    GP.log(f"[exit-law] {name} ok {rep}")


@pytest.mark.parametrize("name", ["tiny", "qwen3_4b", "qwen3_8b_wide", "mixture"])
def test_named_workloads(name):
    GP.log(f"[exit-law] workload {name}")
    wl = W.make_config(name, with_attention=False)
    rep = GP.check_exit_law_and_draws(wl)
    GP.log(f"[exit-law] {name} ok {rep}")


def test_batched_workload():
    GP.log("[exit-law] workload batched (32 requests)")
    wl = W.make_config("batched", with_attention=False)
    rep = GP.check_exit_law_and_draws(wl, cdf_nodes=2)
    GP.log(f"[exit-law] batched ok {rep}")


def test_children_cover_whole_vocabulary():
    """rho(root) = 0 exactly: the root is never drawn, its residual unused."""
    V = 6
    par = np.array([[-1, 0, 0, 0, 0, 0, 0, 1]], np.int32)
    tok = np.array([[0, 0, 1, 2, 3, 4, 5, 2]], np.int32)
    lg = np.random.default_rng(0).standard_normal((1, 8, V)).astype(np.float32)
    wl = W.Workload("cover", 0, 1, 8, V, "f32", lg, par, tok, W.uniforms_for(3, 0, 2048)[None],
                    1, 1, 64, 0)
    g = GP.run_exit_law(wl)
    assert g["w"][0, 0] == 0.0 and g["rho"][0, 0] == 0.0
    assert np.all(g["exit"] != 0)
    GP.check_exit_law_and_draws(wl)


def test_neg_inf_logits():
    wl = W.make_custom("neginf", R=1, B=20, V=20000, dtype="bf16", tree="random",
                       with_attention=False, n_uniform=512)
    lg = W.bf16_bits_to_f32(wl.logits)
    lg[0, :, 5000:12000] = -np.inf                   # whole chunks and partial chunks
    lg[0, 3, :] = np.where(np.arange(20000) % 7 == 0, lg[0, 3], -np.inf)
    wl.logits = W.f32_to_bf16_bits(lg)
    GP.check_exit_law_and_draws(wl)


@pytest.mark.parametrize("kind", ["nan", "posinf", "all_neginf"])
def test_nonfinite_rows_are_flagged(kind):
    wl = W.make_custom("bad", R=3, B=10, V=9000, dtype="f32", tree="random", with_attention=False,
                       n_uniform=16)
    if kind == "nan":
        wl.logits[1, 4, 8500] = np.nan
    elif kind == "posinf":
        wl.logits[1, 2, 17] = np.inf
    else:
        wl.logits[1, 7, :] = -np.inf
    g = GP.run_exit_law(wl)
    assert g["flags"][1] & tev.TEV_FLAG_NONFINITE
    assert g["flags"][0] == 0 and g["flags"][2] == 0
    assert np.all(np.isnan(g["rho"][1])) and np.isnan(g["cov"][1])
    assert np.all(g["exit"][1] == -1) and np.all(g["bonus"][1] == -1)
    # the other requests are unaffected
    ora = oracle.exit_law(wl.logits[[0, 2]], "f32", wl.parents[[0, 2]], wl.tokens[[0, 2]])
    GP.assert_close_rel("w", g["w"][[0, 2]], ora.exit_mass)


@pytest.mark.parametrize("kind", ["parent_order", "root_parent", "token_range", "dup_sibling"])
def test_invalid_trees_are_flagged(kind):
    wl = W.make_custom("badtree", R=2, B=12, V=9000, dtype="bf16", tree="random",
                       with_attention=False, n_uniform=16)
    p, t = wl.parents, wl.tokens
    if kind == "parent_order":
        p[1, 4] = 9
    elif kind == "root_parent":
        p[1, 0] = 0
    elif kind == "token_range":
        t[1, 5] = 9000
    else:
        kids = np.nonzero(p[1] == p[1, 3])[0]
        kids = kids[kids != 3]
        if len(kids) == 0:
            p[1, 3] = 0
            kids = np.nonzero(p[1] == 0)[0]
            kids = kids[kids != 3]
        t[1, 3] = t[1, kids[0]]
    g = GP.run_exit_law(wl)
    assert g["flags"][1] & tev.TEV_FLAG_TREE, g["flags"]
    assert g["flags"][0] == 0
    assert np.all(np.isnan(g["w"][1])) and np.all(g["exit"][1] == -1)


def test_determinism_bitwise():
    wl = W.make_custom("det", R=2, B=64, V=40000, dtype="bf16", tree="best_first",
                       with_attention=False, n_uniform=256)
    a = GP.run_exit_law(wl)
    b = GP.run_exit_law(wl)
    for key in ("rho", "reach", "w", "cov", "exit", "bonus"):
        np.testing.assert_array_equal(a[key], b[key])
    ca = tev.tev_export_exit_cdf(a["res"].workspace, wl.R, wl.B, wl.V)
    cb = tev.tev_export_exit_cdf(b["res"].workspace, wl.R, wl.B, wl.V)
    np.testing.assert_array_equal(ca, cb)


def test_workspace_reuse_across_calls():
    """One zero-filled workspace serves consecutive calls: every call leaves
    its completion counters at zero again."""
    import torch
    wls = [W.make_custom(f"reuse{i}", R=2, B=33, V=30000, dtype="bf16", tree="random", seed=200 + i,
                         with_attention=False, n_uniform=128) for i in range(3)]
    ws = torch.zeros(tev.tev_exit_law_workspace_bytes(2, 33, 30000), dtype=torch.uint8, device="cuda")
    for wl in wls * 2:
        lg, par, tok, uni = GP.device_inputs(wl)
        res = tev.tev_exit_law(lg, par, tok, 1.0, workspace=ws)
        en, bt = tev.tev_sample(lg, par, tok, res.workspace, uni)
        torch.cuda.synchronize()
        ora = oracle.exit_law(wl.logits, wl.dtype, wl.parents, wl.tokens)
        GP.assert_close_rel("w", res.exit_mass.cpu().numpy(), ora.exit_mass)
        GP.assert_close_rel("C", res.coverage.cpu().numpy(), ora.coverage)
        dr = oracle.sample(wl.logits, wl.dtype, wl.parents, wl.tokens, ora.exit_mass, wl.uniforms)
        ok = ~(dr.band_exit | dr.band_bonus)
        assert np.array_equal(en.cpu().numpy()[ok], dr.exit_node[ok])
        assert np.array_equal(bt.cpu().numpy()[ok], dr.bonus_token[ok])


def _value_cases(n=16, seed=3105):
    """Seeded value ranges: logit spread from nearly flat to a few tokens
    holding all the mass, drafted children boosted or not, temperatures
    either side of 1, and one row with a single finite logit."""
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        cases.append(dict(name=f"values{i}", R=int(rng.integers(1, 5)),
                          B=int(rng.choice([2, 9, 33, 64, 128])),
                          V=int(rng.choice([int(rng.integers(100, 4096)), int(rng.integers(4096, 30000)), 8192])),
                          dtype="f32" if rng.random() < 0.4 else "bf16",
                          tree=str(rng.choice(["random", "chain", "star", "best_first"])),
                          logit_sigma=float(rng.choice([0.1, 1.0, 3.0, 20.0, 60.0])),
                          child_boost=float(rng.choice([0.0, 4.0, 20.0])),
                          inv_temperature=float(rng.choice([0.25, 0.6, 1.0, 1.9])),
                          seed=int(rng.integers(1, 1 << 30))))
    return cases


VALUES = _value_cases()


@pytest.mark.parametrize("case", VALUES, ids=[c["name"] for c in VALUES])
def test_value_sweep(case):
    c = dict(case)
    name = c.pop("name")
    GP.log(f"[exit-law] {name} {c}")
    wl = W.make_custom(name, with_attention=False, n_uniform=1024, **c)
    # one node's row keeps a single finite logit (a one-hot target row)
    lg = wl.logits.astype(np.float32) if wl.dtype == "f32" else W.bf16_bits_to_f32(wl.logits)
    rng = np.random.default_rng(c["seed"])
    r, v = int(rng.integers(0, wl.R)), int(rng.integers(0, wl.B))
    keep = int(rng.integers(0, wl.V))
    lg[r, v, :] = np.where(np.arange(wl.V) == keep, lg[r, v, keep], -np.inf)
    wl.logits = lg if wl.dtype == "f32" else W.f32_to_bf16_bits(lg)
    rep = GP.check_exit_law_and_draws(wl)
    GP.log(f"[exit-law] {name} ok {rep}")
