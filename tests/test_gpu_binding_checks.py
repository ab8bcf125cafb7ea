"""The Python binding refuses device tensors of the wrong element type or
size before anything is launched (the C ABI takes bare pointers and cannot see
sizes, so a short output buffer would otherwise be written past its end)."""
import numpy as np
import pytest
import torch

from draft_tree_verification_amd import tev
from tests import workloads as W

pytestmark = pytest.mark.gpu


def _case():
    rng = np.random.default_rng(0)
    p, t = W.random_tree(16, 500, rng)
    par = tev.to_device_i32(p[None])
    tok = tev.to_device_i32(t[None])
    lg = torch.randn(1, 16, 500, device="cuda")
    return par, tok, lg


def test_index_inputs_must_be_int32_of_the_right_size():
    par, tok, lg = _case()
    with pytest.raises(TypeError):
        tev.tev_exit_law(lg, par.to(torch.int64), tok)
    with pytest.raises(ValueError):
        tev.tev_exit_law(lg, par[:, :8].contiguous(), tok)
    z = torch.randn(1, 4, 500, device="cuda")
    with pytest.raises(ValueError):
        tev.tev_build_tree(z, 8, 16, root_tokens=torch.zeros(2, dtype=torch.int32, device="cuda"))
    with pytest.raises(ValueError):
        tev.tev_exit_loss(z, par, tok, torch.ones(1, 15, device="cuda"))


def test_short_output_buffers_are_refused():
    par, tok, lg = _case()
    law = tev.tev_exit_law(lg, par, tok)
    torch.cuda.synchronize()
    uni = torch.rand(1, 3, 2, device="cuda")
    short = (torch.empty(1, 2, dtype=torch.int32, device="cuda"), torch.empty(1, 2, dtype=torch.int32, device="cuda"))
    with pytest.raises(ValueError):
        tev.tev_sample(lg, par, tok, law.workspace, uni, out=short)
    z = torch.randn(1, 4, 500, device="cuda")
    built = tev.tev_build_tree(z, 8, 16)
    with pytest.raises(ValueError):
        tev.tev_build_tree(z, 8, 32, out=built)          # a tree of 16 nodes cannot take 32
    k = torch.zeros(1, 2, 10 + 16, 64, device="cuda")
    with pytest.raises(ValueError):
        tev.tev_commit_kv(k, k.clone(), par, torch.zeros(1, dtype=torch.int32, device="cuda"), 10,
                          out=torch.empty(0, dtype=torch.int32, device="cuda"))
