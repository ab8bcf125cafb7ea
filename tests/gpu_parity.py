"""Shared helpers of the GPU parity tests: run a workload through the C ABI
(via the binding) and through the CPU oracle, and compare under the
acceptance rules:

* rho, P, w, C: |x - x_ref| <= 2e-3 |x_ref| + 1e-9 (fp32 outputs of an fp64
  pipeline; the 1e-9 floor covers masses too small to move a 2^-24-grid
  uniform across a bin outside the band);
* exit node and bonus token: equal to the oracle's for every draw whose
  uniforms are not within 1e-6 of a boundary of the chosen bin (the oracle's
  band flags), given identical uniforms;
* the GPU's normalised exit CDF and residual CDFs within 1e-6 of the
  oracle's at every index -- the bound that makes index agreement outside the
  band a guarantee rather than luck;
* attention: per query row, max_d |o - o_ref| <= 2e-3 max_d |o_ref|.
"""
from __future__ import annotations

import sys

import numpy as np
import torch

import oracle
from draft_tree_verification_amd import tev

TOL_REL = 2e-3
TOL_ABS = 1e-9
CDF_TOL = 1e-6


def log(msg: str):
    print(msg, flush=True)
    sys.stdout.flush()


def device_inputs(wl):
    lg = tev.to_device_logits(wl.logits, wl.dtype)
    par = tev.to_device_i32(wl.parents)
    tok = tev.to_device_i32(wl.tokens)
    uni = torch.from_numpy(np.ascontiguousarray(wl.uniforms, np.float32)).cuda()
    return lg, par, tok, uni


def assert_close_rel(name, got, ref, rel=TOL_REL, abs_=TOL_ABS):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    err = np.abs(got - ref)
    bound = rel * np.abs(ref) + abs_
    bad = ~(err <= bound)
    if bad.any():
        idx = np.argwhere(bad)[:5]
        raise AssertionError(f"{name}: {bad.sum()} of {bad.size} outside tolerance; first "
                             f"{[(tuple(i), got[tuple(i)], ref[tuple(i)]) for i in idx]}")
    return float((err / (np.abs(ref) + 1e-30)).max()) if err.size else 0.0


def run_exit_law(wl, inv_temperature=None):
    s = wl.inv_temperature if inv_temperature is None else inv_temperature
    lg, par, tok, uni = device_inputs(wl)
    res = tev.tev_exit_law(lg, par, tok, s)
    en, bt = tev.tev_sample(lg, par, tok, res.workspace, uni, s)
    torch.cuda.synchronize()
    return dict(lg=lg, par=par, tok=tok, uni=uni, res=res,
                rho=res.rho.cpu().numpy(), reach=res.reach.cpu().numpy(),
                w=res.exit_mass.cpu().numpy(), cov=res.coverage.cpu().numpy(),
                exit=en.cpu().numpy(), bonus=bt.cpu().numpy(),
                flags=tev.tev_read_device_status(res.workspace, 0, wl.R, wl.B, wl.V))


def check_exit_law_and_draws(wl, cdf_nodes: int = 3, inv_temperature=None, nthreads=0):
    """Full comparison of exit law, draws and CDFs for a workload."""
    s = wl.inv_temperature if inv_temperature is None else inv_temperature
    g = run_exit_law(wl, s)
    assert np.all(g["flags"] == 0), g["flags"]
    ora = oracle.exit_law(wl.logits, wl.dtype, wl.parents, wl.tokens, s, nthreads=nthreads)
    report = {}
    report["rho"] = assert_close_rel("rho", g["rho"], ora.rho)
    report["reach"] = assert_close_rel("reach", g["reach"], ora.reach)
    report["exit_mass"] = assert_close_rel("exit_mass", g["w"], ora.exit_mass)
    report["coverage"] = assert_close_rel("coverage", g["cov"], ora.coverage)
    dr = oracle.sample(wl.logits, wl.dtype, wl.parents, wl.tokens, ora.exit_mass, wl.uniforms, s,
                       nthreads=nthreads)
    ok_e = ~dr.band_exit
    ok_b = ok_e & ~dr.band_bonus
    mism_e = np.argwhere(ok_e & (g["exit"] != dr.exit_node))
    assert len(mism_e) == 0, f"exit node mismatches at {mism_e[:5].tolist()}"
    mism_b = np.argwhere(ok_b & (g["bonus"] != dr.bonus_token))
    assert len(mism_b) == 0, (f"bonus mismatches at {mism_b[:5].tolist()}: gpu "
                              f"{g['bonus'][tuple(mism_b[0])]} oracle {dr.bonus_token[tuple(mism_b[0])]}")
    report["band_excluded"] = int((~ok_b).sum())
    report["draws"] = int(ok_b.size)
    # CDF deviation: exit CDF of every request
    cdf_gpu = tev.tev_export_exit_cdf(g["res"].workspace, wl.R, wl.B, wl.V)
    cum = np.cumsum(ora.exit_mass, axis=1)
    cdf_ref = cum / cum[:, -1:]
    report["exit_cdf_dev"] = float(np.abs(cdf_gpu - cdf_ref).max())
    assert report["exit_cdf_dev"] < CDF_TOL, report
    # residual CDFs of the most drawn nodes (and a leaf if any) of request 0..
    dev = 0.0
    for r in range(min(wl.R, 2)):
        counts = np.bincount(dr.exit_node[r], minlength=wl.B)
        nodes = list(np.argsort(-counts)[:cdf_nodes])
        for v in nodes:
            if ora.exit_mass[r, v] <= 0:
                continue
            ref = oracle.residual_cdf(wl.logits[r], wl.dtype, wl.parents[r], wl.tokens[r], int(v), s)
            got = tev.tev_export_residual_cdf(g["lg"], g["par"], g["tok"], g["res"].workspace, r,
                                              int(v), s).cpu().numpy()
            dev = max(dev, float(np.abs(got - ref).max()))
    report["residual_cdf_dev"] = dev
    assert dev < CDF_TOL, report
    return report


def attn_row_errors(got: np.ndarray, ref: np.ndarray) -> np.ndarray:
    """Row-normwise relative error: max_d |o - o_ref| / max_d |o_ref| per row."""
    got = got.reshape(-1, got.shape[-1]).astype(np.float64)
    ref = ref.reshape(-1, ref.shape[-1])
    return np.abs(got - ref).max(axis=1) / np.maximum(np.abs(ref).max(axis=1), 1e-30)


def run_attn(wl):
    dt = torch.bfloat16 if wl.dtype == "bf16" else torch.float32
    def dev(a):
        if wl.dtype == "bf16":
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()
        return torch.from_numpy(np.ascontiguousarray(a, np.float32)).cuda()
    q, k, v = dev(wl.q), dev(wl.k), dev(wl.v)
    assert q.dtype == dt
    par = tev.to_device_i32(wl.parents)
    ws = torch.zeros(max(1, tev.tev_tree_attn_workspace_bytes(wl.R, wl.B, wl.Hq, wl.Hkv, wl.D, wl.P)),
                     dtype=torch.uint8, device="cuda")
    out = tev.tev_tree_attn(q, k, v, par, wl.P, wl.scale, workspace=ws)
    torch.cuda.synchronize()
    flags = tev.tev_read_device_status(ws, 1, wl.R)
    return out.cpu().numpy(), flags


def check_attn(wl, rows: np.ndarray | None = None, nthreads=0):
    got, flags = run_attn(wl)
    assert np.all(flags == 0), flags
    ref = oracle.tree_attn(wl.q, wl.k, wl.v, wl.dtype, wl.parents, wl.P, wl.scale, rows=rows,
                           nthreads=nthreads)
    g = got.reshape(-1, wl.D) if rows is None else got.reshape(-1, wl.D)[rows]
    err = attn_row_errors(g, ref)
    worst = int(np.argmax(err))
    assert err.max() <= TOL_REL, f"row error {err.max():.3e} at row {worst if rows is None else rows[worst]}"
    return float(err.max())


def request_rows(wl, requests) -> np.ndarray:
    """Flat query-row indices ((r * B + i) * Hq + h) of every row of the given requests."""
    per = wl.B * wl.Hq
    return np.concatenate([np.arange(r * per, (r + 1) * per, dtype=np.int64) for r in requests])


def check_draws_and_cdfs(wl, lg, par, tok, ws, exit_node, bonus, ora, cdf_nodes=3, s=None,
                         nthreads=0):
    """Draws of one round (exit_node, bonus [R][n]) against the oracle's on the
    same uniforms outside the band, and the GPU's exit CDF (every request) and
    residual CDFs (the most drawn nodes of up to two requests) within 1e-6 of
    the oracle's, read from the exit-law workspace ``ws``."""
    s = wl.inv_temperature if s is None else s
    dr = oracle.sample(wl.logits, wl.dtype, wl.parents, wl.tokens, ora.exit_mass, wl.uniforms, s,
                       nthreads=nthreads)
    ok_e = ~dr.band_exit
    ok_b = ok_e & ~dr.band_bonus
    mism_e = np.argwhere(ok_e & (exit_node != dr.exit_node))
    assert len(mism_e) == 0, f"exit node mismatches at {mism_e[:5].tolist()}"
    mism_b = np.argwhere(ok_b & (bonus != dr.bonus_token))
    assert len(mism_b) == 0, (f"bonus mismatches at {mism_b[:5].tolist()}: gpu "
                              f"{bonus[tuple(mism_b[0])]} oracle {dr.bonus_token[tuple(mism_b[0])]}")
    rep = {"band_excluded": int((~ok_b).sum()), "draws": int(ok_b.size)}
    cdf_gpu = tev.tev_export_exit_cdf(ws, wl.R, wl.B, wl.V)
    cum = np.cumsum(ora.exit_mass, axis=1)
    rep["exit_cdf_dev"] = float(np.abs(cdf_gpu - cum / cum[:, -1:]).max())
    assert rep["exit_cdf_dev"] < CDF_TOL, rep
    dev = 0.0
    for r in sorted({0, wl.R - 1}):
        counts = np.bincount(dr.exit_node[r], minlength=wl.B)
        for v in list(np.argsort(-counts)[:cdf_nodes]):
            if ora.exit_mass[r, v] <= 0:
                continue
            ref = oracle.residual_cdf(wl.logits[r], wl.dtype, wl.parents[r], wl.tokens[r], int(v), s)
            got = tev.tev_export_residual_cdf(lg, par, tok, ws, r, int(v), s).cpu().numpy()
            dev = max(dev, float(np.abs(got - ref).max()))
    rep["residual_cdf_dev"] = dev
    assert dev < CDF_TOL, rep
    return rep
