"""GPU parity of tev_commit_kv (in-place KV-cache commit after verification)
against the oracle's commit, through the C ABI: every byte of the committed
caches, every layer, bf16 and f32, shallow and deep paths, batches that span
several staging rounds, and invalid exit nodes."""
import numpy as np
import pytest
import torch

import oracle
from draft_tree_verification_amd import tev
from tests import workloads as W
from tests import gpu_parity as GP

pytestmark = pytest.mark.gpu


def _run(dtype, R, B, L, Hkv, D, P, tree, exit_fn, seed):
    rng = np.random.default_rng(seed)
    if tree == "chain":
        parents = np.tile(np.array([-1] + list(range(B - 1)), np.int32), (R, 1))
    else:
        parents = np.stack([W.random_tree(B, 100, rng)[0] for _ in range(R)]).astype(np.int32)
    exit_node = np.array([exit_fn(parents[r], rng) for r in range(R)], np.int32)
    shape = (L, R, Hkv, P + B, D)
    if dtype == "bf16":
        kk = W.f32_to_bf16_bits(rng.standard_normal(shape).astype(np.float32))
        vv = W.f32_to_bf16_bits(rng.standard_normal(shape).astype(np.float32))
        to = lambda a: torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
        back = lambda t: t.view(torch.int16).cpu().numpy().view(np.uint16)
    else:
        kk = rng.standard_normal(shape).astype(np.float32)
        vv = rng.standard_normal(shape).astype(np.float32)
        to = lambda a: torch.from_numpy(a).cuda()
        back = lambda t: t.cpu().numpy()
    k_d, v_d = to(kk), to(vv)
    nl = tev.tev_commit_kv(k_d, v_d, tev.to_device_i32(parents), tev.to_device_i32(exit_node), P)
    torch.cuda.synchronize()
    return kk, vv, parents, exit_node, back(k_d), back(v_d), nl.cpu().numpy()


CASES = [
    dict(dtype="bf16", R=2, B=37, L=3, Hkv=4, D=128, P=100, tree="random"),
    dict(dtype="f32", R=3, B=20, L=2, Hkv=2, D=64, P=0, tree="random"),
    dict(dtype="bf16", R=1, B=256, L=2, Hkv=2, D=128, P=64, tree="chain"),   # 256 rows: several batches
    dict(dtype="f32", R=1, B=256, L=1, Hkv=1, D=128, P=8, tree="chain"),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"{c['dtype']}_B{c['B']}_{c['tree']}_D{c['D']}")
def test_commit_matches_oracle(case):
    GP.log(f"[commit] {case}")
    deepest = lambda par, rng: int(np.argmax(W.depths_of(par)))
    for fn in (deepest, lambda par, rng: int(rng.integers(0, len(par))), lambda par, rng: 0):
        kk, vv, par, en, kg, vg, nl = _run(seed=3, exit_fn=fn, **case)
        k2, v2, nl2 = oracle.commit_kv(kk, vv, par, en, case["P"])
        np.testing.assert_array_equal(nl, nl2)
        np.testing.assert_array_equal(kg, k2)
        np.testing.assert_array_equal(vg, v2)


def test_commit_rejects_invalid_exit_node():
    kk, vv, par, en, kg, vg, nl = _run("bf16", 2, 10, 1, 2, 128, 16, "random",
                                       lambda par, rng: 12, seed=4)   # out of range
    assert np.all(nl == -1)
    np.testing.assert_array_equal(kg, kk)
    np.testing.assert_array_equal(vg, vv)


def _sweep_cases(n=16, seed=3103):
    rng = np.random.default_rng(seed)
    cases = []
    while len(cases) < n:
        c = dict(dtype="f32" if rng.random() < 0.4 else "bf16", R=int(rng.integers(1, 7)),
                 B=int(rng.choice([1, 2, 17, 64, 65, 130, 256])), L=int(rng.integers(1, 5)),
                 Hkv=int(rng.choice([1, 2, 4, 8])), D=int(rng.choice([64, 128])),
                 P=int(rng.choice([0, 1, 63, 64, 500, 2049])), tree=str(rng.choice(["random", "chain"])))
        if c["L"] * c["R"] * c["Hkv"] * (c["P"] + c["B"]) * c["D"] > 6_000_000:
            continue
        c["seed"] = int(rng.integers(1, 1 << 30))
        cases.append(c)
    return cases


SWEEP = _sweep_cases()


@pytest.mark.parametrize("case", SWEEP, ids=[f"sweep{i}" for i in range(len(SWEEP))])
def test_commit_sweep(case):
    GP.log(f"[commit] {case}")
    deepest = lambda par, rng: int(np.argmax(W.depths_of(par)))
    for fn in (deepest, lambda par, rng: int(rng.integers(0, len(par)))):
        kk, vv, par, en, kg, vg, nl = _run(exit_fn=fn, **case)
        k2, v2, nl2 = oracle.commit_kv(kk, vv, par, en, case["P"])
        np.testing.assert_array_equal(nl, nl2)
        np.testing.assert_array_equal(kg, k2)
        np.testing.assert_array_equal(vg, v2)
