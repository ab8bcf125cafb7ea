"""The whole verification stage on the GPU, call after call, against the
oracle run the same way: the tree built from draft rows (tev_build_tree), one
round on it (tev_verify_round: attention, exit law, TEV's draws) and the
cache commit of the drawn exit node's path (tev_commit_kv).  Each step's
inputs on the oracle side come from the oracle's previous step (the GPU's
tree and draws must equal the oracle's for the chain to continue), so the
chain shows the calls fit together the way the pages' round uses them
("CAST" App. C "The round"; "Where Draft Trees Lose Target Mass", App. D.1)."""
import numpy as np
import pytest
import torch

import oracle
from draft_tree_verification_amd import tev
from tests import workloads as W
from tests import gpu_parity as GP

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("dtype,R,L,V,K,B,Hq,Hkv,D,P", [
    ("f32", 2, 4, 3000, 8, 24, 4, 2, 64, 100),
    ("bf16", 3, 8, 20000, 16, 64, 8, 2, 128, 256),
])
def test_build_verify_commit_chain(dtype, R, L, V, K, B, Hq, Hkv, D, P):
    GP.log(f"[stage] {dtype} R={R} L={L} V={V} K={K} B={B}")
    rng = np.random.default_rng(B + V)
    z = (rng.standard_normal((R, L, V)) * 3.0).astype(np.float32)
    roots = rng.integers(0, V, size=R).astype(np.int32)
    zs = z if dtype == "f32" else W.f32_to_bf16_bits(z)
    # 1. the tree
    t = tev.tev_build_tree(tev.to_device_logits(zs, dtype), K, B, tev.to_device_i32(roots))
    torch.cuda.synchronize()
    ref_t = oracle.build_tree(zs, dtype, K, B, roots)
    assert not ref_t.near_tie.any()
    np.testing.assert_array_equal(t.parents.cpu().numpy(), ref_t.parents)
    np.testing.assert_array_equal(t.tokens.cpu().numpy(), ref_t.tokens)
    parents, tokens = ref_t.parents, ref_t.tokens
    # 2. target logits for that tree (drafted children boosted), Q/K/V, uniforms
    lg = rng.standard_normal((R, B, V)).astype(np.float32) * 3.0
    for r in range(R):
        for u in range(1, B):
            lg[r, parents[r, u], tokens[r, u]] += 4.0
    lgs = lg if dtype == "f32" else W.f32_to_bf16_bits(lg)
    q, k, v = W.make_attention(B + V, R, B, Hq, Hkv, D, P, dtype)
    uni = np.stack([W.uniforms_for(7, r, 1) for r in range(R)])
    to = lambda a: tev.to_device_logits(a, dtype)
    res = tev.tev_verify_round(to(q), to(k), to(v), to(lgs), t.parents, t.tokens,
                               torch.from_numpy(uni).cuda(), P, 1.0 / np.sqrt(D), 1.0)
    torch.cuda.synchronize()
    law = oracle.exit_law(lgs, dtype, parents, tokens)
    dr = oracle.sample(lgs, dtype, parents, tokens, law.exit_mass, uni)
    en = res.exit_node.cpu().numpy()[:, 0]
    bt = res.bonus_token.cpu().numpy()[:, 0]
    for r in range(R):
        if not (dr.band_exit[r, 0] or dr.band_bonus[r, 0]):
            assert en[r] == dr.exit_node[r, 0] and bt[r] == dr.bonus_token[r, 0]
    ref_o = oracle.tree_attn(q, k, v, dtype, parents, P, 1.0 / np.sqrt(D))
    err = GP.attn_row_errors(res.attn_out.cpu().numpy().reshape(-1, D), ref_o)
    assert err.max() <= 2e-3
    # 3. commit the drawn exit node's path (the oracle's draw) in place
    exit_nodes = dr.exit_node[:, 0].astype(np.int32)
    kd, vd = to(k), to(v)
    nl = tev.tev_commit_kv(kd, vd, t.parents, tev.to_device_i32(exit_nodes), P)
    torch.cuda.synchronize()
    k2, v2, nl2 = oracle.commit_kv(k[None], v[None], parents, exit_nodes, P)
    np.testing.assert_array_equal(nl.cpu().numpy(), nl2)
    back = (lambda x: x.cpu().numpy()) if dtype == "f32" else (lambda x: x.view(torch.int16).cpu().numpy().view(np.uint16))
    np.testing.assert_array_equal(back(kd), k2[0])
    np.testing.assert_array_equal(back(vd), v2[0])
