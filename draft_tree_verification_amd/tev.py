"""Python binding of libtev (include/tev.h): argument marshalling only.

Every step of the verification path runs in the HIP kernels of libtev; this
module only checks tensor shapes, allocates outputs and workspaces through
torch, and passes raw device pointers and the current HIP stream to the C ABI.
There is no CPU fallback: if libtev.so is missing or cannot be loaded, every
call raises.

Function names follow the C ABI: tev_exit_law, tev_sample, tev_tree_attn, ...
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "_build", "libtev.so")

TEV_F32, TEV_BF16 = 0, 1
TEV_FLAG_NONFINITE, TEV_FLAG_TREE = 1, 2
TEV_MAX_NODES = 256
STATUS_NAMES = {0: "TEV_OK", 1: "TEV_ERR_NULL", 2: "TEV_ERR_SHAPE", 3: "TEV_ERR_DTYPE",
                4: "TEV_ERR_TREE", 5: "TEV_ERR_WORKSPACE", 6: "TEV_ERR_UNSUPPORTED",
                7: "TEV_ERR_HIP", 8: "TEV_ERR_VALUE"}

EXPORTED = ["tev_exit_law_workspace_bytes", "tev_exit_law", "tev_sample",
            "tev_tree_attn_workspace_bytes", "tev_tree_attn", "tev_validate_tree_host",
            "tev_read_device_status", "tev_status_str", "tev_export_exit_cdf",
            "tev_export_residual_cdf", "tev_verify_round_workspace_bytes", "tev_verify_round",
            "tev_verify_round_timed", "tev_predraw", "tev_commit_kv",
            "tev_exit_loss_workspace_bytes", "tev_exit_loss", "tev_build_tree_workspace_bytes",
            "tev_build_tree", "tev_build_tree_modes_workspace_bytes", "tev_build_tree_modes",
            "tev_verify_round_noalloc"]


class TevError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn} returned {STATUS_NAMES.get(status, status)}")
        self.status = status


_lib = None


def lib() -> ctypes.CDLL:
    """Load libtev.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with __graft_entry__.build()")
        L = ctypes.CDLL(LIB_PATH)
        vp, i, f, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
        L.tev_exit_law_workspace_bytes.argtypes = [i, i, i]
        L.tev_exit_law_workspace_bytes.restype = sz
        L.tev_exit_law.argtypes = [vp, i, vp, vp, i, i, i, f, vp, vp, vp, vp, vp, sz, vp]
        L.tev_sample.argtypes = [vp, i, vp, vp, i, i, i, f, vp, sz, vp, i, vp, vp, vp]
        L.tev_predraw.argtypes = [vp, i, vp, vp, i, i, i, f, vp, sz, vp, i, vp, vp, vp, vp]
        L.tev_commit_kv.argtypes = [vp, vp, i, vp, vp, i, i, i, i, i, i, vp, vp]
        L.tev_exit_loss_workspace_bytes.argtypes = [i, i, i, i]
        L.tev_exit_loss_workspace_bytes.restype = sz
        L.tev_exit_loss.argtypes = [vp, i, vp, vp, vp, i, i, i, i, vp, vp, vp, vp, vp, sz, vp]
        L.tev_build_tree_workspace_bytes.argtypes = [i, i, i, i]
        L.tev_build_tree_workspace_bytes.restype = sz
        L.tev_build_tree.argtypes = [vp, i, vp, i, i, i, i, i, vp, vp, vp, vp, sz, vp]
        L.tev_build_tree_modes_workspace_bytes.argtypes = [i, i, i, i, i, i]
        L.tev_build_tree_modes_workspace_bytes.restype = sz
        L.tev_build_tree_modes.argtypes = [vp, i, vp, vp, i, i, i, i, i, i, vp, vp, vp, vp, sz, vp]
        L.tev_tree_attn_workspace_bytes.argtypes = [i, i, i, i, i, i]
        L.tev_tree_attn_workspace_bytes.restype = sz
        L.tev_tree_attn.argtypes = [vp, vp, vp, i, vp, i, i, i, i, i, i, f, vp, vp, sz, vp]
        L.tev_validate_tree_host.argtypes = [vp, vp, i, i]
        L.tev_read_device_status.argtypes = [vp, i, i, i, i, vp, vp]
        L.tev_status_str.argtypes = [i]
        L.tev_status_str.restype = ctypes.c_char_p
        L.tev_export_exit_cdf.argtypes = [vp, i, i, i, vp, vp]
        L.tev_export_residual_cdf.argtypes = [vp, i, vp, vp, i, i, i, f, vp, sz, i, i, vp, vp]
        L.tev_verify_round_workspace_bytes.argtypes = [i, i, i, i, i, i, i]
        L.tev_verify_round_workspace_bytes.restype = sz
        L.tev_verify_round.argtypes = [vp, vp, vp, vp, i, vp, vp, i, i, i, i, i, i, i, f, f, vp, i,
                                       vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
        L.tev_verify_round_timed.argtypes = L.tev_verify_round.argtypes + [vp]
        L.tev_verify_round_noalloc.argtypes = [vp, vp, vp, vp, i, vp, vp, i, i, i, i, i, i, i, f, f, vp, i,
                                               vp, vp, vp, vp, vp, vp, vp, vp]
        for fn in ("tev_exit_law", "tev_sample", "tev_predraw", "tev_commit_kv", "tev_exit_loss", "tev_build_tree",
                   "tev_build_tree_modes",
                   "tev_tree_attn", "tev_validate_tree_host", "tev_verify_round", "tev_verify_round_timed",
                   "tev_verify_round_noalloc",
                   "tev_read_device_status", "tev_export_exit_cdf", "tev_export_residual_cdf"):
            getattr(L, fn).restype = ctypes.c_int
        _lib = L
    return _lib


def _p(t: torch.Tensor | None):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _check(fn: str, st: int):
    if st != 0:
        raise TevError(fn, st)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return TEV_BF16
    if t.dtype == torch.float32:
        return TEV_F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _dev_i32(x, shape, device) -> torch.Tensor:
    t = torch.as_tensor(x, dtype=torch.int32, device=device).reshape(shape).contiguous()
    return t


def _need_cuda(*ts: torch.Tensor):
    for t in ts:
        if not t.is_cuda:
            raise ValueError("tensors must live on the GPU")
        if not t.is_contiguous():
            raise ValueError("tensors must be contiguous")


def _need(t: torch.Tensor, dtype: torch.dtype, numel: int, name: str):
    """A device tensor the kernels index by the call's sizes: the right element
    type and exactly the right number of elements (the C ABI cannot see sizes)."""
    _need_cuda(t)
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if t.numel() != numel:
        raise ValueError(f"{name} must hold {numel} elements, got {t.numel()}")


# ---------------------------------------------------------------- exit law
@dataclass
class ExitLawResult:
    rho: torch.Tensor        # float32 [R][B]
    reach: torch.Tensor      # float32 [R][B]
    exit_mass: torch.Tensor  # float32 [R][B]
    coverage: torch.Tensor   # float32 [R]
    workspace: torch.Tensor  # uint8, private state read by tev_sample


def tev_exit_law_workspace_bytes(R: int, B: int, V: int) -> int:
    return int(lib().tev_exit_law_workspace_bytes(R, B, V))


def tev_exit_law(logits: torch.Tensor, parents: torch.Tensor, tokens: torch.Tensor,
                 inv_temperature: float = 1.0, workspace: torch.Tensor | None = None,
                 out: ExitLawResult | None = None) -> ExitLawResult:
    """Exit law of every request: logits [R][B][V] (bf16 or f32) on the GPU,
    parents/tokens int32 [R][B] on the GPU."""
    if logits.dim() == 2:
        logits = logits.unsqueeze(0)
    _need_cuda(logits)
    R, B, V = logits.shape
    _need(parents, torch.int32, R * B, "parents")
    _need(tokens, torch.int32, R * B, "tokens")
    dev = logits.device
    L = lib()
    need = tev_exit_law_workspace_bytes(R, B, V)
    if out is None:
        if workspace is None:
            workspace = torch.zeros(max(need, 1), dtype=torch.uint8, device=dev)
        out = ExitLawResult(torch.empty((R, B), dtype=torch.float32, device=dev),
                            torch.empty((R, B), dtype=torch.float32, device=dev),
                            torch.empty((R, B), dtype=torch.float32, device=dev),
                            torch.empty((R,), dtype=torch.float32, device=dev), workspace)
    for t, nm in ((out.rho, "rho"), (out.reach, "reach"), (out.exit_mass, "exit_mass")):
        _need(t, torch.float32, R * B, nm)
    _need(out.coverage, torch.float32, R, "coverage")
    st = L.tev_exit_law(_p(logits), _dtype_code(logits), _p(parents), _p(tokens), R, B, V,
                        float(inv_temperature), _p(out.rho), _p(out.reach), _p(out.exit_mass),
                        _p(out.coverage), _p(out.workspace), out.workspace.numel(), _stream())
    _check("tev_exit_law", st)
    return out


def tev_sample(logits: torch.Tensor, parents: torch.Tensor, tokens: torch.Tensor,
               workspace: torch.Tensor, uniforms: torch.Tensor, inv_temperature: float = 1.0,
               out: tuple[torch.Tensor, torch.Tensor] | None = None):
    """TEV's exit-node and bonus-token draws; uniforms float32 [R][n][2]."""
    if logits.dim() == 2:
        logits = logits.unsqueeze(0)
    _need_cuda(logits, workspace, uniforms)
    R, B, V = logits.shape
    _need(parents, torch.int32, R * B, "parents")
    _need(tokens, torch.int32, R * B, "tokens")
    n = uniforms.shape[-2]
    if uniforms.dtype != torch.float32 or uniforms.numel() != R * n * 2:
        raise ValueError("uniforms must be float32 [R][n][2]")
    if out is None:
        out = (torch.empty((R, n), dtype=torch.int32, device=logits.device),
               torch.empty((R, n), dtype=torch.int32, device=logits.device))
    _need(out[0], torch.int32, R * n, "exit_node")
    _need(out[1], torch.int32, R * n, "bonus_token")
    st = lib().tev_sample(_p(logits), _dtype_code(logits), _p(parents), _p(tokens), R, B, V,
                          float(inv_temperature), _p(workspace), workspace.numel(), _p(uniforms),
                          n, _p(out[0]), _p(out[1]), _stream())
    _check("tev_sample", st)
    return out


def tev_predraw(logits: torch.Tensor, parents: torch.Tensor, tokens: torch.Tensor,
                workspace: torch.Tensor, uniforms: torch.Tensor, inv_temperature: float = 1.0,
                out: tuple[torch.Tensor, torch.Tensor, torch.Tensor] | None = None):
    """Predraw-and-follow verification; uniforms float32 [R][n][B].
    Returns (node_draw [R][n][B], exit_node [R][n], bonus_token [R][n]), int32."""
    if logits.dim() == 2:
        logits = logits.unsqueeze(0)
    _need_cuda(logits, workspace, uniforms)
    R, B, V = logits.shape
    _need(parents, torch.int32, R * B, "parents")
    _need(tokens, torch.int32, R * B, "tokens")
    n = uniforms.shape[-2]
    if uniforms.dtype != torch.float32 or uniforms.numel() != R * n * B:
        raise ValueError("uniforms must be float32 [R][n][B]")
    if out is None:
        out = (torch.empty((R, n, B), dtype=torch.int32, device=logits.device),
               torch.empty((R, n), dtype=torch.int32, device=logits.device),
               torch.empty((R, n), dtype=torch.int32, device=logits.device))
    _need(out[0], torch.int32, R * n * B, "node_draw")
    _need(out[1], torch.int32, R * n, "exit_node")
    _need(out[2], torch.int32, R * n, "bonus_token")
    st = lib().tev_predraw(_p(logits), _dtype_code(logits), _p(parents), _p(tokens), R, B, V,
                           float(inv_temperature), _p(workspace), workspace.numel(), _p(uniforms),
                           n, _p(out[0]), _p(out[1]), _p(out[2]), _stream())
    _check("tev_predraw", st)
    return out


def tev_commit_kv(k: torch.Tensor, v: torch.Tensor, parents: torch.Tensor, exit_node: torch.Tensor,
                  P: int, out: torch.Tensor | None = None) -> torch.Tensor:
    """In-place cache commit: k, v [L][R][Hkv][P+B][D] (or [R][Hkv][P+B][D] for
    one layer); exit_node int32 [R].  Returns new_len int32 [R]."""
    _need_cuda(k, v, parents, exit_node)
    if k.dim() == 4:
        k, v = k.unsqueeze(0), v.unsqueeze(0)
    L, R, Hkv, nkv, D = k.shape
    B = nkv - P
    if v.shape != k.shape or v.dtype != k.dtype or B < 1:
        raise ValueError("k/v [L][R][Hkv][P+B][D]")
    _need(parents, torch.int32, R * B, "parents")
    _need(exit_node, torch.int32, R, "exit_node")
    if out is None:
        out = torch.empty((R,), dtype=torch.int32, device=k.device)
    _need(out, torch.int32, R, "new_len")
    st = lib().tev_commit_kv(_p(k), _p(v), _dtype_code(k), _p(parents), _p(exit_node), R, B, L, Hkv,
                             D, int(P), _p(out), _stream())
    _check("tev_commit_kv", st)
    return out


# ---------------------------------------------------------------- exit-guided loss
@dataclass
class ExitLossResult:
    loss: torch.Tensor        # float32 [1]
    row_lse: torch.Tensor     # float32 [R][H]
    row_weight: torch.Tensor  # float32 [R][H]
    grad: torch.Tensor | None  # float32 [R][H][V] or None
    workspace: torch.Tensor   # uint8; its first R words are the flag words


def tev_exit_loss_workspace_bytes(R: int, B: int, H: int, V: int) -> int:
    return int(lib().tev_exit_loss_workspace_bytes(R, B, H, V))


def tev_exit_loss(draft_logits: torch.Tensor, parents: torch.Tensor, tokens: torch.Tensor,
                  weights: torch.Tensor, with_grad: bool = True,
                  workspace: torch.Tensor | None = None,
                  out: ExitLossResult | None = None) -> ExitLossResult:
    """Exit-guided draft-tree loss: draft_logits [R][H][V] (bf16 or f32),
    parents/tokens int32 [R][B], weights float32 [R][B], all on the GPU."""
    _need_cuda(draft_logits)
    R, H, V = draft_logits.shape
    B = parents.shape[-1]
    _need(parents, torch.int32, R * B, "parents")
    _need(tokens, torch.int32, R * B, "tokens")
    _need(weights, torch.float32, R * B, "weights")
    dev = draft_logits.device
    if out is None:
        if workspace is None:
            workspace = torch.empty(max(tev_exit_loss_workspace_bytes(R, B, H, V), 1),
                                    dtype=torch.uint8, device=dev)
        out = ExitLossResult(torch.empty(1, dtype=torch.float32, device=dev),
                             torch.empty((R, H), dtype=torch.float32, device=dev),
                             torch.empty((R, H), dtype=torch.float32, device=dev),
                             torch.empty((R, H, V), dtype=torch.float32, device=dev)
                             if with_grad else None, workspace)
    _need(out.loss, torch.float32, 1, "loss")
    _need(out.row_lse, torch.float32, R * H, "row_lse")
    _need(out.row_weight, torch.float32, R * H, "row_weight")
    if out.grad is not None:
        _need(out.grad, torch.float32, R * H * V, "grad")
    st = lib().tev_exit_loss(_p(draft_logits), _dtype_code(draft_logits), _p(parents), _p(tokens),
                             _p(weights), R, B, H, V, _p(out.loss), _p(out.row_lse),
                             _p(out.row_weight), _p(out.grad), _p(out.workspace),
                             out.workspace.numel(), _stream())
    _check("tev_exit_loss", st)
    return out


# ---------------------------------------------------------------- tree builder
@dataclass
class BuiltTree:
    parents: torch.Tensor    # int32 [R][B]
    tokens: torch.Tensor     # int32 [R][B]
    scores: torch.Tensor     # float64 [R][B]
    workspace: torch.Tensor  # uint8; its first R words are the flag words


def tev_build_tree_workspace_bytes(R: int, L: int, V: int, K: int) -> int:
    return int(lib().tev_build_tree_workspace_bytes(R, L, V, K))


def tev_build_tree(draft_logits: torch.Tensor, K: int, B: int, root_tokens: torch.Tensor | None = None,
                   workspace: torch.Tensor | None = None, out: BuiltTree | None = None) -> BuiltTree:
    """Best-first draft tree: draft_logits [R][L][V] (bf16 or f32) on the GPU,
    K tokens kept per position, B nodes (root included)."""
    _need_cuda(draft_logits)
    R, L, V = draft_logits.shape
    if root_tokens is not None:
        _need(root_tokens, torch.int32, R, "root_tokens")
    dev = draft_logits.device
    if out is None:
        if workspace is None:
            workspace = torch.empty(max(tev_build_tree_workspace_bytes(R, L, V, K), 1), dtype=torch.uint8,
                                    device=dev)
        out = BuiltTree(torch.empty((R, B), dtype=torch.int32, device=dev),
                        torch.empty((R, B), dtype=torch.int32, device=dev),
                        torch.empty((R, B), dtype=torch.float64, device=dev), workspace)
    _need(out.parents, torch.int32, R * B, "parents")
    _need(out.tokens, torch.int32, R * B, "tokens")
    _need(out.scores, torch.float64, R * B, "scores")
    st = lib().tev_build_tree(_p(draft_logits), _dtype_code(draft_logits), _p(root_tokens), R, L, V, K, B,
                              _p(out.parents), _p(out.tokens), _p(out.scores), _p(out.workspace),
                              out.workspace.numel(), _stream())
    _check("tev_build_tree", st)
    return out


def tev_build_tree_modes_workspace_bytes(R: int, M: int, L: int, V: int, K: int, B: int) -> int:
    return int(lib().tev_build_tree_modes_workspace_bytes(R, M, L, V, K, B))


def tev_build_tree_modes(draft_logits: torch.Tensor, K: int, B: int, log_prior: torch.Tensor | None = None,
                         root_tokens: torch.Tensor | None = None, workspace: torch.Tensor | None = None,
                         out: BuiltTree | None = None) -> BuiltTree:
    """Merged heap over M draft modes: draft_logits [R][M][L][V] (bf16 or
    f32), log_prior float32 [R][M] or None (uniform)."""
    _need_cuda(draft_logits)
    R, M, L, V = draft_logits.shape
    if log_prior is not None:
        _need(log_prior, torch.float32, R * M, "log_prior")
    if root_tokens is not None:
        _need(root_tokens, torch.int32, R, "root_tokens")
    dev = draft_logits.device
    if out is None:
        if workspace is None:
            workspace = torch.empty(max(tev_build_tree_modes_workspace_bytes(R, M, L, V, K, B), 1),
                                    dtype=torch.uint8, device=dev)
        out = BuiltTree(torch.empty((R, B), dtype=torch.int32, device=dev),
                        torch.empty((R, B), dtype=torch.int32, device=dev),
                        torch.empty((R, B), dtype=torch.float64, device=dev), workspace)
    _need(out.parents, torch.int32, R * B, "parents")
    _need(out.tokens, torch.int32, R * B, "tokens")
    _need(out.scores, torch.float64, R * B, "scores")
    st = lib().tev_build_tree_modes(_p(draft_logits), _dtype_code(draft_logits), _p(log_prior), _p(root_tokens),
                                    R, M, L, V, K, B, _p(out.parents), _p(out.tokens), _p(out.scores),
                                    _p(out.workspace), out.workspace.numel(), _stream())
    _check("tev_build_tree_modes", st)
    return out


# ---------------------------------------------------------------- attention
def tev_tree_attn_workspace_bytes(R, B, Hq, Hkv, D, P) -> int:
    return int(lib().tev_tree_attn_workspace_bytes(R, B, Hq, Hkv, D, P))


def tev_tree_attn(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, parents: torch.Tensor,
                  P: int, scale: float | None = None, workspace: torch.Tensor | None = None,
                  out: torch.Tensor | None = None) -> torch.Tensor:
    """q [R][B][Hq][D], k/v [R][Hkv][P+B][D] (bf16 or f32) -> float32 [R][B][Hq][D]."""
    _need_cuda(q, k, v)
    R, B, Hq, D = q.shape
    Hkv = k.shape[1]
    if k.shape != (R, Hkv, P + B, D) or v.shape != k.shape or k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("k/v must be [R][Hkv][P+B][D] with q's dtype")
    _need(parents, torch.int32, R * B, "parents")
    if scale is None:
        scale = 1.0 / float(np.sqrt(D))
    need = tev_tree_attn_workspace_bytes(R, B, Hq, Hkv, D, P)
    if workspace is None:
        workspace = torch.zeros(max(need, 1), dtype=torch.uint8, device=q.device)
    if out is None:
        out = torch.empty((R, B, Hq, D), dtype=torch.float32, device=q.device)
    _need(out, torch.float32, R * B * Hq * D, "out")
    st = lib().tev_tree_attn(_p(q), _p(k), _p(v), _dtype_code(q), _p(parents), R, B, Hq, Hkv, D,
                             int(P), float(scale), _p(out), _p(workspace), workspace.numel(),
                             _stream())
    _check("tev_tree_attn", st)
    return out


# ---------------------------------------------------------------- whole round
@dataclass
class RoundResult:
    attn_out: torch.Tensor     # float32 [R][B][Hq][D]
    rho: torch.Tensor          # float32 [R][B]
    reach: torch.Tensor        # float32 [R][B]
    exit_mass: torch.Tensor    # float32 [R][B]
    coverage: torch.Tensor     # float32 [R]
    exit_node: torch.Tensor    # int32 [R][n]
    bonus_token: torch.Tensor  # int32 [R][n]
    workspace: torch.Tensor    # uint8; its head is an exit-law workspace


def tev_verify_round_workspace_bytes(R, B, V, Hq, Hkv, D, P) -> int:
    return int(lib().tev_verify_round_workspace_bytes(R, B, V, Hq, Hkv, D, P))


def tev_verify_round(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, logits: torch.Tensor,
                     parents: torch.Tensor, tokens: torch.Tensor, uniforms: torch.Tensor, P: int,
                     scale: float | None = None, inv_temperature: float = 1.0,
                     workspace: torch.Tensor | None = None,
                     out: RoundResult | None = None, events=None) -> RoundResult:
    """Tree attention, exit law and draws of one round (the three calls'
    arguments; q/k/v and logits share one dtype).  events: optional four
    recorded-once torch.cuda.Event objects, re-recorded at the launch
    boundaries (tev_verify_round_timed)."""
    if logits.dim() == 2:
        logits = logits.unsqueeze(0)
    _need_cuda(q, k, v, logits, uniforms)
    R, B, Hq, D = q.shape
    _need(parents, torch.int32, R * B, "parents")
    _need(tokens, torch.int32, R * B, "tokens")
    Hkv = k.shape[1]
    V = logits.shape[-1]
    if k.shape != (R, Hkv, P + B, D) or v.shape != k.shape or k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("k/v must be [R][Hkv][P+B][D] with q's dtype")
    if logits.shape != (R, B, V) or logits.dtype != q.dtype:
        raise ValueError("logits must be [R][B][V] with q's dtype")
    n = uniforms.shape[-2]
    if uniforms.dtype != torch.float32 or uniforms.numel() != R * n * 2:
        raise ValueError("uniforms must be float32 [R][n][2]")
    if scale is None:
        scale = 1.0 / float(np.sqrt(D))
    dev = q.device
    if out is None:
        if workspace is None:
            need = tev_verify_round_workspace_bytes(R, B, V, Hq, Hkv, D, P)
            workspace = torch.zeros(max(need, 1), dtype=torch.uint8, device=dev)
        f32 = dict(dtype=torch.float32, device=dev)
        out = RoundResult(torch.empty((R, B, Hq, D), **f32), torch.empty((R, B), **f32),
                          torch.empty((R, B), **f32), torch.empty((R, B), **f32),
                          torch.empty((R,), **f32),
                          torch.empty((R, n), dtype=torch.int32, device=dev),
                          torch.empty((R, n), dtype=torch.int32, device=dev), workspace)
    _need(out.attn_out, torch.float32, R * B * Hq * D, "attn_out")
    for t, nm in ((out.rho, "rho"), (out.reach, "reach"), (out.exit_mass, "exit_mass")):
        _need(t, torch.float32, R * B, nm)
    _need(out.coverage, torch.float32, R, "coverage")
    _need(out.exit_node, torch.int32, R * n, "exit_node")
    _need(out.bonus_token, torch.int32, R * n, "bonus_token")
    args = [_p(q), _p(k), _p(v), _p(logits), _dtype_code(q), _p(parents), _p(tokens), R, B, V, Hq,
            Hkv, D, int(P), float(scale), float(inv_temperature), _p(uniforms), n, _p(out.attn_out),
            _p(out.rho), _p(out.reach), _p(out.exit_mass), _p(out.coverage), _p(out.exit_node),
            _p(out.bonus_token), _p(out.workspace), out.workspace.numel(), _stream()]
    if events is None:
        st = lib().tev_verify_round(*args)
        _check("tev_verify_round", st)
    else:
        handles = (ctypes.c_void_p * 4)(*[ctypes.c_void_p(e.cuda_event) for e in events])
        st = lib().tev_verify_round_timed(*args, ctypes.cast(handles, ctypes.c_void_p))
        _check("tev_verify_round_timed", st)
    return out


NOALLOC_SCRATCH_BYTES = 32 << 20   # TEV_NOALLOC_SCRATCH_BYTES in include/tev.h


def tev_verify_round_noalloc(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, logits: torch.Tensor,
                             parents: torch.Tensor, tokens: torch.Tensor, uniforms: torch.Tensor, P: int,
                             scale: float | None = None, inv_temperature: float = 1.0,
                             out: RoundResult | None = None) -> RoundResult:
    """tev_verify_round on the library's own device scratch (no workspace
    argument; the C call allocates nothing).  ``out`` may carry preallocated
    outputs; its workspace field is ignored and returned as None."""
    if logits.dim() == 2:
        logits = logits.unsqueeze(0)
    _need_cuda(q, k, v, logits, uniforms)
    R, B, Hq, D = q.shape
    _need(parents, torch.int32, R * B, "parents")
    _need(tokens, torch.int32, R * B, "tokens")
    Hkv = k.shape[1]
    V = logits.shape[-1]
    if k.shape != (R, Hkv, P + B, D) or v.shape != k.shape or k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("k/v must be [R][Hkv][P+B][D] with q's dtype")
    if logits.shape != (R, B, V) or logits.dtype != q.dtype:
        raise ValueError("logits must be [R][B][V] with q's dtype")
    n = uniforms.shape[-2]
    if uniforms.dtype != torch.float32 or uniforms.numel() != R * n * 2:
        raise ValueError("uniforms must be float32 [R][n][2]")
    if scale is None:
        scale = 1.0 / float(np.sqrt(D))
    dev = q.device
    if out is None:
        f32 = dict(dtype=torch.float32, device=dev)
        out = RoundResult(torch.empty((R, B, Hq, D), **f32), torch.empty((R, B), **f32),
                          torch.empty((R, B), **f32), torch.empty((R, B), **f32),
                          torch.empty((R,), **f32),
                          torch.empty((R, n), dtype=torch.int32, device=dev),
                          torch.empty((R, n), dtype=torch.int32, device=dev), None)
    _need(out.attn_out, torch.float32, R * B * Hq * D, "attn_out")
    for t, nm in ((out.rho, "rho"), (out.reach, "reach"), (out.exit_mass, "exit_mass")):
        _need(t, torch.float32, R * B, nm)
    _need(out.coverage, torch.float32, R, "coverage")
    _need(out.exit_node, torch.int32, R * n, "exit_node")
    _need(out.bonus_token, torch.int32, R * n, "bonus_token")
    st = lib().tev_verify_round_noalloc(
        _p(q), _p(k), _p(v), _p(logits), _dtype_code(q), _p(parents), _p(tokens), R, B, V, Hq, Hkv, D,
        int(P), float(scale), float(inv_temperature), _p(uniforms), n, _p(out.attn_out), _p(out.rho),
        _p(out.reach), _p(out.exit_mass), _p(out.coverage), _p(out.exit_node), _p(out.bonus_token),
        _stream())
    _check("tev_verify_round_noalloc", st)
    return RoundResult(out.attn_out, out.rho, out.reach, out.exit_mass, out.coverage, out.exit_node,
                       out.bonus_token, None)


# ---------------------------------------------------------------- helpers
def tev_validate_tree_host(parents: np.ndarray, tokens: np.ndarray, V: int) -> int:
    p = np.ascontiguousarray(parents, dtype=np.int32)
    t = np.ascontiguousarray(tokens, dtype=np.int32)
    return int(lib().tev_validate_tree_host(p.ctypes.data_as(ctypes.c_void_p),
                                            t.ctypes.data_as(ctypes.c_void_p), int(p.shape[0]), int(V)))


def tev_read_device_status(workspace: torch.Tensor, kind: int, R: int, B: int = 1, V: int = 1) -> np.ndarray:
    flags = np.zeros(R, np.uint32)
    st = lib().tev_read_device_status(_p(workspace), kind, R, B, V,
                                      flags.ctypes.data_as(ctypes.c_void_p), _stream())
    _check("tev_read_device_status", st)
    return flags


def tev_status_str(status: int) -> str:
    return lib().tev_status_str(int(status)).decode()


def tev_export_exit_cdf(workspace: torch.Tensor, R: int, B: int, V: int) -> np.ndarray:
    cdf = np.empty((R, B), np.float64)
    st = lib().tev_export_exit_cdf(_p(workspace), R, B, V, cdf.ctypes.data_as(ctypes.c_void_p), _stream())
    _check("tev_export_exit_cdf", st)
    return cdf


def tev_export_residual_cdf(logits: torch.Tensor, parents: torch.Tensor, tokens: torch.Tensor,
                            workspace: torch.Tensor, r: int, node: int,
                            inv_temperature: float = 1.0) -> torch.Tensor:
    if logits.dim() == 2:
        logits = logits.unsqueeze(0)
    R, B, V = logits.shape
    cdf = torch.empty(V, dtype=torch.float64, device=logits.device)
    st = lib().tev_export_residual_cdf(_p(logits), _dtype_code(logits), _p(parents), _p(tokens),
                                       R, B, V, float(inv_temperature), _p(workspace),
                                       workspace.numel(), int(r), int(node), _p(cdf), _stream())
    _check("tev_export_residual_cdf", st)
    return cdf


# ---------------------------------------------------------------- tensors from host arrays
def to_device_logits(a: np.ndarray, dtype: str, device="cuda") -> torch.Tensor:
    """float32 array or uint16 bf16 bit patterns -> device tensor of that dtype."""
    if dtype == "bf16":
        t = torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(device)


def to_device_i32(a: np.ndarray, device="cuda") -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(device)
