// exit_loss.h -- workspace layout and launcher of the exit-guided draft-tree
// loss (exit_loss.hip).  Not part of the public ABI.
#pragma once

#include "tev_internal.h"

namespace tev {

// Logits per slab: a workgroup of LOSS_THREADS threads reduces one slab of one
// draft row, each thread holding LOSS_EPT elements in registers.
constexpr int LOSS_THREADS = 256;
constexpr int LOSS_EPT = 32;
constexpr int LOSS_SLAB = LOSS_THREADS * LOSS_EPT;   // 8192
constexpr int LOSS_MAX_H = 1024;                     // draft positions per example
constexpr int LOSS_ROW_THREADS = 1024;               // per-example pass: one wave per row

inline int loss_slabs(int V) { return (V + LOSS_SLAB - 1) / LOSS_SLAB; }

// Exit-loss workspace, M = R * H draft rows, ns slabs per row:
//   status  u32 [R]      device flag bits of the example (TEV_FLAG_*)
//   slab_m  f32 [M][ns]  slab offset in log2 units (floor of max logit * log2 e)
//   slab_s  f32 [M][ns]  sum over the slab of 2^(z log2 e - slab_m)
//   lse2    f64 [M]      logsumexp of the row in log2 units
//   omega   f64 [M]      summed weight of the row's nonzero-weight nodes
//   num     f64 [R]      the example's share of the loss numerator
//   ent_n   i32 [M]      number of nonzero-weight nodes scored by the row
//   ent_tok i32 [M][B]   their tokens, in node order
//   ent_w   f32 [M][B]   their weights
struct LossWs {
    size_t status, slab_m, slab_s, lse2, omega, num, ent_n, ent_tok, ent_w, total;
};

inline LossWs loss_ws_layout(int R, int B, int H, int V) {
    const size_t M = (size_t)R * H, mns = M * (size_t)loss_slabs(V);
    LossWs L{};
    size_t o = 0;
    L.status = o;  o = align_up(o + 4 * (size_t)R, 256);
    L.slab_m = o;  o = align_up(o + 4 * mns, 256);
    L.slab_s = o;  o = align_up(o + 4 * mns, 256);
    L.lse2 = o;    o = align_up(o + 8 * M, 256);
    L.omega = o;   o = align_up(o + 8 * M, 256);
    L.num = o;     o = align_up(o + 8 * (size_t)R, 256);
    L.ent_n = o;   o = align_up(o + 4 * M, 256);
    L.ent_tok = o; o = align_up(o + 4 * M * B, 256);
    L.ent_w = o;   o = align_up(o + 4 * M * B, 256);
    L.total = o;
    return L;
}

// vec: 16-byte loads of the draft logits and 16-byte stores of the gradient
// (rows of V * element size a multiple of 16 bytes, aligned pointers).
hipError_t launch_exit_loss(const void *draft_logits, int dtype, bool vec, const int32_t *parents,
                            const int32_t *tokens, const float *weights, int R, int B, int H, int V,
                            float *loss, float *row_lse, float *row_weight, float *grad, char *ws,
                            hipStream_t st);

}  // namespace tev
