"""GPU parity of tev_verify_round (one call for the whole round) through the
C ABI: its attention output, exit law and draws against the CPU oracle under
the same acceptance rules as the separate calls, and its exit law and draws
bit-equal to those of tev_exit_law + tev_sample on the same inputs (the round
runs the same arithmetic, only packed into fewer launches)."""
import numpy as np
import pytest
import torch

import oracle
from draft_tree_verification_amd import tev
from tests import workloads as W
from tests import gpu_parity as GP

pytestmark = pytest.mark.gpu


def _dev(wl, a):
    if wl.dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(a, np.float32)).cuda()


def _run_round(wl, n_uniform=None):
    q, k, v = _dev(wl, wl.q), _dev(wl, wl.k), _dev(wl, wl.v)
    lg, par, tok, uni = GP.device_inputs(wl)
    res = tev.tev_verify_round(q, k, v, lg, par, tok, uni, wl.P, wl.scale, wl.inv_temperature)
    torch.cuda.synchronize()
    flags = tev.tev_read_device_status(res.workspace, 2, wl.R, wl.B, wl.V)
    return res, flags, (lg, par, tok, uni)


def _check_round(wl, rows=None):
    res, flags, (lg, par, tok, uni) = _run_round(wl)
    assert np.all(flags == 0), flags
    # attention against the oracle
    ref = oracle.tree_attn(wl.q, wl.k, wl.v, wl.dtype, wl.parents, wl.P, wl.scale, rows=rows)
    got = res.attn_out.cpu().numpy().reshape(-1, wl.D)
    got = got if rows is None else got[rows]
    err = GP.attn_row_errors(got, ref)
    assert err.max() <= GP.TOL_REL, f"attention row error {err.max():.3e}"
    # exit law and draws: bit-equal to the separate calls ...
    el = tev.tev_exit_law(lg, par, tok, wl.inv_temperature)
    en, bt = tev.tev_sample(lg, par, tok, el.workspace, uni, wl.inv_temperature)
    torch.cuda.synchronize()
    for name, a, b in (("rho", res.rho, el.rho), ("reach", res.reach, el.reach),
                       ("exit_mass", res.exit_mass, el.exit_mass), ("coverage", res.coverage, el.coverage),
                       ("exit_node", res.exit_node, en), ("bonus_token", res.bonus_token, bt)):
        np.testing.assert_array_equal(a.cpu().numpy(), b.cpu().numpy(), err_msg=name)
    # ... and within the bar of the oracle
    ora = oracle.exit_law(wl.logits, wl.dtype, wl.parents, wl.tokens, wl.inv_temperature)
    GP.assert_close_rel("exit_mass", res.exit_mass.cpu().numpy(), ora.exit_mass)
    GP.assert_close_rel("coverage", res.coverage.cpu().numpy(), ora.coverage)
    GP.assert_close_rel("reach", res.reach.cpu().numpy(), ora.reach)
    dr = oracle.sample(wl.logits, wl.dtype, wl.parents, wl.tokens, ora.exit_mass, wl.uniforms,
                       wl.inv_temperature)
    ok = ~(dr.band_exit | dr.band_bonus)
    assert np.array_equal(res.exit_node.cpu().numpy()[ok], dr.exit_node[ok])
    assert np.array_equal(res.bonus_token.cpu().numpy()[ok], dr.bonus_token[ok])
    return float(err.max())


SMALL = [
    dict(name="bf16_d128", R=2, B=37, V=20000, Hq=8, Hkv=2, D=128, P=300, tree="random"),
    dict(name="bf16_d64_best_first", R=1, B=64, V=17000, Hq=6, Hkv=3, D=64, P=517, tree="best_first"),
    dict(name="bf16_max_nodes", R=1, B=256, V=9000, Hq=4, Hkv=2, D=128, P=1024, tree="random"),
    dict(name="bf16_root_only", R=2, B=1, V=5000, Hq=4, Hkv=2, D=128, P=200, tree="random"),
    dict(name="f32_small", R=2, B=16, V=3000, Hq=4, Hkv=4, D=64, P=128, tree="random", dtype="f32"),
    # the reach workgroups beside the attention for up to 7 and from 8
    # requests on (the attention plan leaves that many CUs), and logit rows
    # that are not whole 16-byte vectors
    dict(name="bf16_r7", R=7, B=20, V=12000, Hq=4, Hkv=2, D=64, P=100, tree="random"),
    dict(name="bf16_r9", R=9, B=20, V=12000, Hq=4, Hkv=2, D=64, P=100, tree="random"),
    dict(name="bf16_odd_vocab", R=2, B=30, V=9001, Hq=4, Hkv=2, D=128, P=150, tree="random"),
]


@pytest.mark.parametrize("case", SMALL, ids=[c["name"] for c in SMALL])
def test_round_small(case):
    c = dict(case)
    name = c.pop("name")
    dtype = c.pop("dtype", "bf16")
    GP.log(f"[round] {name} {c} {dtype}")
    wl = W.make_custom(name, dtype=dtype, n_uniform=512, **c)
    err = _check_round(wl)
    GP.log(f"[round] {name} ok, attention row error {err:.3e}")


def _sweep_cases(n=48, seed=2026):
    """Seeded random shapes across the launch plans: requests, tree size and
    kind, vocabulary (odd sizes included), GQA ratio, head_dim, prefix length
    around the 64-key stages and split boundaries (P = 0 included); sized so
    that the oracle's attention stays within a few GFLOP per case."""
    rng = np.random.default_rng(seed)
    cases = []
    while len(cases) < n:
        R = int(rng.integers(1, 13))
        B = int(rng.choice([1, 2, 3, 17, 40, 64, 65, 127, 128, 200, 256]))
        G = int(rng.choice([1, 2, 3, 4, 5, 8]))
        Hkv = int(rng.choice([1, 2, 4]))
        D = int(rng.choice([64, 128]))
        P = int(rng.choice([0, 1, 31, 63, 64, 65, 255, 513, 1500, 2048, 4097]))
        V = int(rng.integers(2000, 30001))
        tree = str(rng.choice(["random", "chain", "star", "best_first"] if B >= 3 else ["random"]))
        dtype = "f32" if rng.random() < 0.2 else "bf16"
        if R * B > 1200 or G * Hkv > 32 or R * B * G * Hkv * (P + B) * D > 1e9:
            continue
        cases.append(dict(name=f"sweep{len(cases)}", R=R, B=B, V=V, Hq=G * Hkv, Hkv=Hkv, D=D, P=P,
                          tree=tree, dtype=dtype, seed=int(rng.integers(1, 1 << 30))))
    return cases


SWEEP = _sweep_cases()


@pytest.mark.parametrize("case", SWEEP, ids=[c["name"] for c in SWEEP])
def test_round_sweep(case):
    c = dict(case)
    name = c.pop("name")
    GP.log(f"[round] {name} {c}")
    wl = W.make_custom(name, n_uniform=512, **c)
    err = _check_round(wl)
    GP.log(f"[round] {name} ok, attention row error {err:.3e}")


NAMED = ["tiny", "qwen3_4b", "qwen3_8b_wide", "mixture", "batched"]


@pytest.mark.parametrize("name", NAMED)
def test_round_named(name):
    """Every named workload at full size through the call the benchmark times
    (each runs its own attention plan and reach batching: at qwen3_8b_wide
    two query tiles per wave with four reach batches, at batched 32 requests
    with eight CUs left to the reach).  rho, P, w and C of every node, 4096
    uniform pairs per request with the exit and residual CDF deviations, and
    every attention row (at batched, every row of the first and the last
    request); the exit law and draws also bit-equal to tev_exit_law +
    tev_sample on the same inputs."""
    GP.log(f"[round] workload {name} (full size, 4096 uniform pairs per request)")
    wl = W.make_config(name, n_uniform=4096)
    res, flags, (lg, par, tok, uni) = _run_round(wl)
    assert np.all(flags == 0), flags
    GP.log(f"[round] {name}: round done, comparing the exit law")
    el = tev.tev_exit_law(lg, par, tok, wl.inv_temperature)
    en, bt = tev.tev_sample(lg, par, tok, el.workspace, uni, wl.inv_temperature)
    torch.cuda.synchronize()
    for nm, a, b in (("rho", res.rho, el.rho), ("reach", res.reach, el.reach),
                     ("exit_mass", res.exit_mass, el.exit_mass), ("coverage", res.coverage, el.coverage),
                     ("exit_node", res.exit_node, en), ("bonus_token", res.bonus_token, bt)):
        np.testing.assert_array_equal(a.cpu().numpy(), b.cpu().numpy(), err_msg=nm)
    ora = oracle.exit_law(wl.logits, wl.dtype, wl.parents, wl.tokens, wl.inv_temperature)
    rep = {k: GP.assert_close_rel(k, getattr(res, a).cpu().numpy(), getattr(ora, b))
           for k, a, b in (("rho", "rho", "rho"), ("reach", "reach", "reach"),
                           ("exit_mass", "exit_mass", "exit_mass"), ("coverage", "coverage", "coverage"))}
    rep.update(GP.check_draws_and_cdfs(wl, lg, par, tok, res.workspace, res.exit_node.cpu().numpy(),
                                       res.bonus_token.cpu().numpy(), ora,
                                       cdf_nodes=2 if wl.R > 1 else 3))
    GP.log(f"[round] {name}: exit law and draws ok {rep}; comparing attention")
    rows = GP.request_rows(wl, sorted({0, wl.R - 1})) if name == "batched" else None
    ref = oracle.tree_attn(wl.q, wl.k, wl.v, wl.dtype, wl.parents, wl.P, wl.scale, rows=rows)
    got = res.attn_out.cpu().numpy().reshape(-1, wl.D)
    got = got if rows is None else got[rows]
    err = GP.attn_row_errors(got, ref)
    assert err.max() <= GP.TOL_REL, f"attention row error {err.max():.3e} at row {int(np.argmax(err))}"
    GP.log(f"[round] {name} ok: {len(err)} attention rows, max row error {err.max():.3e}")


DRAW_CASES = [c["name"] for c in SMALL if c.get("dtype", "bf16") == "bf16"] + \
    [n for n in NAMED if n != "tiny"]


@pytest.mark.parametrize("name", DRAW_CASES)
@pytest.mark.parametrize("n_draws", [1, 4])
def test_round_draws_in_reach(name, n_draws):
    """With at most four draws per request the round makes them in the reach
    workgroup beside the attention: exit nodes and bonus tokens bit-equal to
    tev_sample after tev_exit_law on the same inputs, and equal to the
    oracle's outside the 1e-6 band."""
    small = {c["name"]: c for c in SMALL}
    if name in small:
        c = dict(small[name])
        c.pop("name")
        wl = W.make_custom(name, dtype=c.pop("dtype", "bf16"), n_uniform=n_draws, **c)
    else:
        wl = W.make_config(name, n_uniform=n_draws)
    GP.log(f"[round] draws in the reach workgroup: {name}, {n_draws} per request")
    res, flags, (lg, par, tok, uni) = _run_round(wl)
    assert np.all(flags == 0), flags
    el = tev.tev_exit_law(lg, par, tok, wl.inv_temperature)
    en, bt = tev.tev_sample(lg, par, tok, el.workspace, uni, wl.inv_temperature)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(res.exit_node.cpu().numpy(), en.cpu().numpy(), err_msg="exit_node")
    np.testing.assert_array_equal(res.bonus_token.cpu().numpy(), bt.cpu().numpy(), err_msg="bonus_token")
    ora = oracle.exit_law(wl.logits, wl.dtype, wl.parents, wl.tokens, wl.inv_temperature)
    dr = oracle.sample(wl.logits, wl.dtype, wl.parents, wl.tokens, ora.exit_mass, wl.uniforms,
                       wl.inv_temperature)
    ok = ~(dr.band_exit | dr.band_bonus)
    assert np.array_equal(res.exit_node.cpu().numpy()[ok], dr.exit_node[ok])
    assert np.array_equal(res.bonus_token.cpu().numpy()[ok], dr.bonus_token[ok])


def test_round_invalid_tree_is_flagged():
    wl = W.make_custom("round_bad", R=2, B=12, V=9000, dtype="bf16", tree="random", Hq=4, Hkv=2,
                       D=128, P=64, n_uniform=16)
    wl.parents[1, 5] = 7
    res, flags, _ = _run_round(wl)
    assert flags[1] & tev.TEV_FLAG_TREE and flags[0] == 0
    assert np.all(np.isnan(res.exit_mass[1].cpu().numpy()))
    assert np.all(res.exit_node[1].cpu().numpy() == -1)
    assert np.all(np.isnan(res.attn_out[1].cpu().numpy()))
    assert np.all(np.isfinite(res.attn_out[0].cpu().numpy()))


def test_round_timed_matches_round():
    """tev_verify_round_timed (events at the launch boundaries, as bench.py
    times the round) writes exactly what tev_verify_round writes, and its
    events are recorded in launch order."""
    wl = W.make_custom("round_timed", R=1, B=40, V=30000, dtype="bf16", tree="random", Hq=8, Hkv=2,
                       D=128, P=600, n_uniform=4)
    q, k, v = _dev(wl, wl.q), _dev(wl, wl.k), _dev(wl, wl.v)
    lg, par, tok, uni = GP.device_inputs(wl)
    args = (q, k, v, lg, par, tok, uni, wl.P, wl.scale, wl.inv_temperature)
    ref = tev.tev_verify_round(*args)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
    for e in ev:
        e.record()
    got = tev.tev_verify_round(*args, events=ev)
    torch.cuda.synchronize()
    for name in ("attn_out", "rho", "reach", "exit_mass", "coverage", "exit_node", "bonus_token"):
        np.testing.assert_array_equal(getattr(got, name).cpu().numpy(), getattr(ref, name).cpu().numpy(),
                                      err_msg=name)
    gaps = [ev[i].elapsed_time(ev[i + 1]) for i in range(3)]
    assert all(g >= 0.0 for g in gaps), gaps
