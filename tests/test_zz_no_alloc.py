"""tev_verify_round_noalloc (the round on the library's own device scratch,
for callers that cannot allocate) against tev_verify_round with a caller
workspace, through the C ABI: every output bit-equal, on two calls in a row
whose second input is smaller than the first (the scratch keeps the first
call's contents), and on the fp32 path."""
import numpy as np
import pytest
import torch

from draft_tree_verification_amd import tev
from tests import gpu_parity as GP
from tests import workloads as W

pytestmark = pytest.mark.gpu

FIELDS = ("attn_out", "rho", "reach", "exit_mass", "coverage", "exit_node", "bonus_token")


def _dev(wl, a):
    if wl.dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(a, np.float32)).cuda()


def _compare(wl):
    q, k, v = _dev(wl, wl.q), _dev(wl, wl.k), _dev(wl, wl.v)
    lg, par, tok, uni = GP.device_inputs(wl)
    args = (q, k, v, lg, par, tok, uni, wl.P, wl.scale, wl.inv_temperature)
    need = tev.tev_verify_round_workspace_bytes(wl.R, wl.B, wl.V, wl.Hq, wl.Hkv, wl.D, wl.P)
    assert 0 < need <= tev.NOALLOC_SCRATCH_BYTES
    got = tev.tev_verify_round_noalloc(*args)
    ref = tev.tev_verify_round(*args)
    torch.cuda.synchronize()
    for name in FIELDS:
        np.testing.assert_array_equal(getattr(got, name).cpu().numpy(), getattr(ref, name).cpu().numpy(),
                                      err_msg=name)
    assert np.isfinite(got.coverage.cpu().numpy()).all()
    return need


def test_noalloc_round_two_calls_second_smaller():
    big = W.make_config("qwen3_4b", n_uniform=64)
    small = W.make_custom("noalloc_small", R=2, B=37, V=20000, dtype="bf16", tree="random", Hq=8,
                          Hkv=2, D=128, P=300, n_uniform=32)
    GP.log("[noalloc] call 1: qwen3_4b (1 x 64 nodes, V=151936, P=4096)")
    n1 = _compare(big)
    GP.log("[noalloc] call 2: 2 x 37 nodes, V=20000, P=300")
    n2 = _compare(small)
    assert n2 < n1
    GP.log(f"[noalloc] ok: scratch use {n1} then {n2} bytes of {tev.NOALLOC_SCRATCH_BYTES}")


def test_noalloc_round_f32_and_flags():
    """The fp32 path (three calls in order) and a request flagged by the
    device (invalid tree): NaN / -1 outputs for it, as with a workspace."""
    wl = W.make_config("tiny", n_uniform=256)
    GP.log("[noalloc] tiny (fp32)")
    _compare(wl)
    bad = W.make_custom("noalloc_bad", R=2, B=12, V=9000, dtype="bf16", tree="random", Hq=4, Hkv=2,
                        D=128, P=64, n_uniform=16)
    bad.parents[1, 5] = 7
    q, k, v = _dev(bad, bad.q), _dev(bad, bad.k), _dev(bad, bad.v)
    lg, par, tok, uni = GP.device_inputs(bad)
    got = tev.tev_verify_round_noalloc(q, k, v, lg, par, tok, uni, bad.P, bad.scale)
    torch.cuda.synchronize()
    assert np.all(np.isnan(got.exit_mass[1].cpu().numpy()))
    assert np.all(got.exit_node[1].cpu().numpy() == -1)
    assert np.all(np.isfinite(got.exit_mass[0].cpu().numpy()))
    GP.log("[noalloc] fp32 and flags ok")
