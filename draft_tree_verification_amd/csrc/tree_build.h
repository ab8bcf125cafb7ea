// tree_build.h -- workspace layout and launcher of the best-first draft-tree
// builder (tree_build.hip).  Not part of the public ABI.
#pragma once

#include "tev_internal.h"

namespace tev {

constexpr int TB_THREADS = 256;                    // slab pass: one slab per workgroup
constexpr int TB_EPT = 32;
constexpr int TB_SLAB = TB_THREADS * TB_EPT;       // 8192 logits
constexpr int TB_MAX_L = 16;                       // draft positions
constexpr int TB_MAX_K = 128;                      // retained tokens per position
constexpr int TB_MAX_SLABS = 64;                   // one slab list per lane in the row merge
constexpr int TB_MAX_MODES = 8;                    // draft modes of the merged heap

inline int tb_slabs(int V) { return (V + TB_SLAB - 1) / TB_SLAB; }

// Builder workspace, M = R * L draft rows, ns slabs per row:
//   status  u32 [R]          device flag bits of the request (TEV_FLAG_*)
//   flag    u32 [M][ns]      a NaN or +inf logit in the slab
//   slab_m  f32 [M][ns]      slab maximum
//   slab_s  f64 [M][ns]      sum over the slab of exp(z - slab maximum)
//   cand    u64 [M][ns][K]   the slab's K best keys, best first (0 = none);
//                            key = (order-preserving bits of z) << 32 | ~token
//   top     u64 [M][K]       the row's K best keys, best first
//   lse     f64 [M]          the row's logsumexp
//   row_flag u32 [M]         TEV_FLAG_NONFINITE for a NaN / +inf logit or an all -inf row
struct TreeWs {
    size_t status, flag, slab_m, slab_s, cand, top, lse, row_flag, total;
};

inline TreeWs tree_ws_layout(int R, int L, int V, int K) {
    const size_t M = (size_t)R * L, mns = M * (size_t)tb_slabs(V);
    TreeWs W{};
    size_t o = 0;
    W.status = o; o = align_up(o + 4 * (size_t)R, 256);
    W.flag = o;   o = align_up(o + 4 * mns, 256);
    W.slab_m = o; o = align_up(o + 4 * mns, 256);
    W.slab_s = o; o = align_up(o + 8 * mns, 256);
    W.cand = o;   o = align_up(o + 8 * mns * (size_t)K, 256);
    W.top = o;    o = align_up(o + 8 * M * (size_t)K, 256);
    W.lse = o;    o = align_up(o + 8 * M, 256);
    W.row_flag = o; o = align_up(o + 4 * M, 256);
    W.total = o;
    return W;
}

// Several draft modes: the per-mode part above for R * M (request, mode)
// pairs, then the modes' emitted streams.  The request flag words come first
// (the per-mode part keeps its own per-mode ones).
//   status    u32 [R]
//   base      TreeWs of R * M requests
//   stream    40-byte records [R * M][B]: key, rank sequence, parent, token, depth
//   stream_n  i32 [R * M]    nodes each mode emitted (root included)
struct TreeModesWs {
    size_t status, base_off, stream, stream_n, total;
    TreeWs base;
};

inline TreeModesWs tree_modes_ws_layout(int R, int M, int L, int V, int K, int B) {
    TreeModesWs W{};
    size_t o = 0;
    W.status = o;   o = align_up(o + 4 * (size_t)R, 256);
    W.base_off = o;
    W.base = tree_ws_layout(R * M, L, V, K);
    o = align_up(o + W.base.total, 256);
    W.stream = o;   o = align_up(o + 40 * (size_t)R * M * B, 256);
    W.stream_n = o; o = align_up(o + 4 * (size_t)R * M, 256);
    W.total = o;
    return W;
}

// M = 1: the single-mode search writes the tree; M > 1: per-mode streams and
// the merge.  log_prior [R][M] or NULL (then every key adds lp_default).
hipError_t launch_build_tree(const void *draft_logits, int dtype, bool vec, const float *log_prior,
                             double lp_default, const int32_t *root_tokens, int R, int M, int L, int V, int K,
                             int B, int32_t *parents, int32_t *tokens, double *scores, char *ws, hipStream_t st);

}  // namespace tev
