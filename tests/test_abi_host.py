"""Host-side checks of the C ABI: the library loads, exports every function
include/tev.h declares, and rejects bad arguments with the documented status
before touching a GPU.  CPU only (no kernel is launched)."""
import ctypes
import os
import re

import numpy as np
import pytest

from draft_tree_verification_amd import tev
from tests import workloads as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_functions():
    with open(os.path.join(ROOT, "include", "tev.h")) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(tev_[a-z_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    L = tev.lib()
    names = _declared_functions()
    assert len(names) >= 10
    for n in names:
        assert hasattr(L, n), n
    assert set(names) == set(tev.EXPORTED)


def test_status_strings():
    for code in range(9):
        assert tev.tev_status_str(code) != "unknown status"
    assert tev.tev_status_str(99) == "unknown status"


def test_host_tree_validation():
    rng = np.random.default_rng(0)
    p, t = W.random_tree(40, 100, rng)
    assert tev.tev_validate_tree_host(p, t, 100) == 0
    bad = p.copy(); bad[0] = 0
    assert tev.tev_validate_tree_host(bad, t, 100) == 4
    bad = p.copy(); bad[5] = 7
    assert tev.tev_validate_tree_host(bad, t, 100) == 4
    bad_t = t.copy(); bad_t[3] = 100
    assert tev.tev_validate_tree_host(p, bad_t, 100) == 4
    # duplicate sibling tokens
    p2 = np.array([-1, 0, 0], np.int32); t2 = np.array([0, 5, 5], np.int32)
    assert tev.tev_validate_tree_host(p2, t2, 10) == 4
    assert tev.tev_validate_tree_host(np.zeros(300, np.int32), np.zeros(300, np.int32), 10) == 2


def test_argument_errors_return_before_any_launch():
    L = tev.lib()
    fake = ctypes.c_void_p(0x1000)   # never dereferenced: every call below fails its checks
    null = None
    s = ctypes.c_void_p(0)
    # null pointers
    assert L.tev_exit_law(null, 1, fake, fake, 1, 4, 10, 1.0, fake, fake, fake, fake, fake, 1 << 20, s) == 1
    # bad sizes
    assert L.tev_exit_law(fake, 1, fake, fake, 1, 0, 10, 1.0, fake, fake, fake, fake, fake, 1 << 20, s) == 2
    assert L.tev_exit_law(fake, 1, fake, fake, 1, 257, 10, 1.0, fake, fake, fake, fake, fake, 1 << 20, s) == 2
    # dtype
    assert L.tev_exit_law(fake, 7, fake, fake, 1, 4, 10, 1.0, fake, fake, fake, fake, fake, 1 << 20, s) == 3
    # temperature
    assert L.tev_exit_law(fake, 1, fake, fake, 1, 4, 10, 0.0, fake, fake, fake, fake, fake, 1 << 20, s) == 8
    assert L.tev_exit_law(fake, 1, fake, fake, 1, 4, 10, float("nan"), fake, fake, fake, fake, fake, 1 << 20, s) == 8
    # workspace too small
    need = L.tev_exit_law_workspace_bytes(1, 4, 10)
    assert need > 0
    assert L.tev_exit_law(fake, 1, fake, fake, 1, 4, 10, 1.0, fake, fake, fake, fake, fake, need - 1, s) == 5
    # sampler
    assert L.tev_sample(fake, 1, fake, fake, 1, 4, 10, 1.0, fake, need, fake, 0, fake, fake, s) == 2
    assert L.tev_sample(fake, 1, fake, fake, 1, 4, 10, 1.0, fake, need - 1, fake, 5, fake, fake, s) == 5
    assert L.tev_sample(fake, 1, fake, fake, 1, 4, 10, 1.0, null, need, fake, 5, fake, fake, s) == 1
    # attention
    need_a = L.tev_tree_attn_workspace_bytes(1, 4, 8, 2, 128, 100)
    assert need_a > 0
    assert L.tev_tree_attn_workspace_bytes(1, 4, 8, 3, 128, 100) == 0
    assert L.tev_tree_attn(fake, fake, fake, 1, fake, 1, 4, 8, 3, 128, 100, 0.1, fake, fake, need_a, s) == 2
    assert L.tev_tree_attn(fake, fake, fake, 1, fake, 1, 4, 8, 2, 96, 100, 0.1, fake, fake, need_a, s) == 6
    assert L.tev_tree_attn(fake, fake, fake, 1, fake, 1, 4, 8, 2, 128, 100, 0.1, fake, fake, need_a - 1, s) == 5
    assert L.tev_tree_attn(fake, fake, fake, 1, fake, 1, 4, 8, 2, 128, 100, float("inf"), fake, fake, need_a, s) == 8
    assert L.tev_tree_attn(fake, fake, fake, 1, null, 1, 4, 8, 2, 128, 100, 0.1, fake, fake, need_a, s) == 1
    assert L.tev_tree_attn(fake, fake, fake, 5, fake, 1, 4, 8, 2, 128, 100, 0.1, fake, fake, need_a, s) == 3
    # scale must be > 0 (every dtype): zero or negative scales are refused
    for bad_scale in (0.0, -0.0, -0.1):
        for dt in (0, 1):
            assert L.tev_tree_attn(fake, fake, fake, dt, fake, 1, 4, 8, 2, 128, 100, bad_scale, fake, fake,
                                   need_a, s) == 8, (bad_scale, dt)
    # one head's K / V extent must stay below 2^31 bytes: (P + B) D e < 2^31
    B = 4
    p_max_bf16 = (1 << 31) // (128 * 2) - B - 1     # (P + B) 256 = 2^31 - 256: accepted
    ws_big = 1 << 62
    assert L.tev_tree_attn(fake, fake, fake, 1, fake, 1, B, 8, 2, 128, p_max_bf16 + 1, 0.1, fake, fake,
                           ws_big, s) == 2                                          # exactly 2^31
    assert L.tev_tree_attn(fake, fake, fake, 0, fake, 1, B, 8, 2, 128, (1 << 31) // 512 - B, 0.1, fake,
                           fake, ws_big, s) == 2                                    # f32: 2^31
    # the same limits through the whole round
    need_r = L.tev_verify_round_workspace_bytes(1, 4, 1000, 8, 2, 128, 100)
    assert need_r > 0
    args = lambda dt, P, sc, ws: (fake, fake, fake, fake, dt, fake, fake, 1, 4, 1000, 8, 2, 128, P, sc, 1.0,
                                  fake, 1, fake, fake, fake, fake, fake, fake, fake, fake, ws, s)
    assert L.tev_verify_round(*args(1, 100, 0.0, need_r)) == 8
    assert L.tev_verify_round(*args(1, 100, -1.0, need_r)) == 8
    assert L.tev_verify_round(*args(1, p_max_bf16 + 1, 0.1, ws_big)) == 2
    assert L.tev_verify_round(*args(1, 100, 0.1, need_r - 1)) == 5
    # the round on the library's scratch: a request whose workspace would
    # exceed the scratch array is refused before anything touches the GPU
    big = L.tev_verify_round_workspace_bytes(64, 256, 1 << 20, 8, 2, 128, 100)
    assert big > tev.NOALLOC_SCRATCH_BYTES
    na = lambda R, B, V: (fake, fake, fake, fake, 1, fake, fake, R, B, V, 8, 2, 128, 100, 0.1, 1.0, fake, 1,
                          fake, fake, fake, fake, fake, fake, fake, s)
    assert L.tev_verify_round_noalloc(*na(64, 256, 1 << 20)) == 5
    assert L.tev_verify_round_noalloc(*na(1, 0, 1000)) == 2
    assert L.tev_verify_round_noalloc(fake, fake, null, fake, 1, fake, fake, 1, 4, 1000, 8, 2, 128, 100, 0.1,
                                      1.0, fake, 1, fake, fake, fake, fake, fake, fake, fake, s) == 1
    # exit-guided loss
    need_l = L.tev_exit_loss_workspace_bytes(2, 9, 4, 1000)
    assert need_l > 0 and L.tev_exit_loss_workspace_bytes(2, 9, 1025, 1000) == 0
    assert L.tev_exit_loss(null, 1, fake, fake, fake, 2, 9, 4, 1000, fake, fake, fake, null, fake, need_l, s) == 1
    assert L.tev_exit_loss(fake, 2, fake, fake, fake, 2, 9, 4, 1000, fake, fake, fake, null, fake, need_l, s) == 3
    assert L.tev_exit_loss(fake, 1, fake, fake, fake, 2, 9, 0, 1000, fake, fake, fake, null, fake, need_l, s) == 2
    assert L.tev_exit_loss(fake, 1, fake, fake, fake, 2, 9, 4, 1000, fake, fake, fake, null, fake, need_l - 1, s) == 5
    # tree builder
    need_t = L.tev_build_tree_workspace_bytes(1, 16, 151936, 64)
    assert need_t > 0
    assert L.tev_build_tree_workspace_bytes(1, 17, 151936, 64) == 0       # L > 16
    assert L.tev_build_tree_workspace_bytes(1, 16, 151936, 129) == 0      # K > 128
    assert L.tev_build_tree_workspace_bytes(1, 16, 600000, 8) == 0        # more than 64 slabs
    assert L.tev_build_tree(null, 1, null, 1, 16, 151936, 64, 64, fake, fake, fake, fake, need_t, s) == 1
    assert L.tev_build_tree(fake, 1, null, 1, 2, 151936, 3, 14, fake, fake, fake, fake, need_t, s) == 2  # 3 + 9 < 13
    assert L.tev_build_tree(fake, 1, null, 1, 16, 151936, 64, 257, fake, fake, fake, fake, need_t, s) == 2
    assert L.tev_build_tree(fake, 1, null, 1, 16, 151936, 64, 64, fake, fake, fake, fake, need_t - 1, s) == 5
    # merged heap over modes
    need_m = L.tev_build_tree_modes_workspace_bytes(1, 8, 16, 151936, 128, 256)
    assert need_m > 0
    assert L.tev_build_tree_modes_workspace_bytes(1, 9, 16, 151936, 128, 256) == 0   # M > 8
    assert L.tev_build_tree_modes(fake, 1, null, null, 1, 8, 16, 151936, 128, 256, fake, fake, fake, fake,
                                  need_m - 1, s) == 5
    assert L.tev_build_tree_modes(fake, 1, null, null, 1, 2, 1, 151936, 3, 8, fake, fake, fake, fake,
                                  need_m, s) == 2                                   # 2 x 3 < 7 prefixes
    assert L.tev_build_tree_modes(null, 1, null, null, 1, 8, 16, 151936, 128, 256, fake, fake, fake, fake,
                                  need_m, s) == 1
    # exports
    assert L.tev_export_residual_cdf(fake, 1, fake, fake, 1, 4, 10, 1.0, fake, need, 1, 0, fake, s) == 2
    assert L.tev_read_device_status(null, 0, 1, 4, 10, fake, s) == 1


def test_workspace_sizes_grow_with_problem():
    L = tev.lib()
    a = L.tev_exit_law_workspace_bytes(1, 64, 151936)
    b = L.tev_exit_law_workspace_bytes(32, 64, 151936)
    assert 0 < a < b
    assert L.tev_exit_law_workspace_bytes(1, 64, 0) == 0
