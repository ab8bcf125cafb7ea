// tev_internal.h -- workspace layouts and launcher declarations shared by the
// HIP translation units of libtev.  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/tev.h"

namespace tev {

constexpr float kInf = __builtin_inff();

// The vocabulary pass splits every logit row into chunks of CHUNK tokens; one
// wavefront (64 lanes) reduces one (row, chunk) pair on its own, each lane
// holding EPT = 64 elements in registers.  A workgroup of VOCAB_THREADS
// threads runs four such independent waves on consecutive chunks of a row.
constexpr int CHUNK = 4096;
constexpr int VOCAB_THREADS = 256;
constexpr int WAVES_PER_WG = VOCAB_THREADS / 64;
constexpr int EPT = CHUNK / 64;   // 64 elements per lane

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }
inline int n_chunks(int V) { return (V + CHUNK - 1) / CHUNK; }

// Exit-law workspace, per request r, node v, chunk c (nc chunks per row):
//   status  u32 [R]          device flag bits of the request (TEV_FLAG_*)
//   flags   u32 [R][B][nc]   per-(row, chunk) flags from the vocabulary pass
//   part_m  f32 [R][B][nc]   chunk offset M_c in log2 units (floor of max logit * sL)
//   part_r  f64 [R][B][nc]   chunk residual sum  sum_{a in c, a not child} 2^(l_a sL - M_c)
//   part_c  f64 [R][B][nc]   chunk child sum     sum_{a in c, a child}     2^(l_a sL - M_c)
//   row_m   f32 [R][B]       row offset M_v = max_c M_c
//   rcum    f64 [R][B][nc]   running residual sum over chunks, units 2^(-M_v)
//   wcum    f64 [R][B]       running exit mass over nodes in index order
//   cterm   f32 [R][B][2]    node u's own term 2^(l sL - M_c) in its parent's
//                            row and that chunk's offset M_c (u > 0)
struct ExitWs {
    size_t status, flags, part_m, part_r, part_c, row_m, rcum, wcum, cterm, total;
};

inline ExitWs exit_ws_layout(int R, int B, int V) {
    const size_t rb = (size_t)R * B, rbc = rb * (size_t)n_chunks(V);
    ExitWs L{};
    size_t o = 0;
    L.status = o; o = align_up(o + 4 * (size_t)R, 256);
    L.flags = o;  o = align_up(o + 4 * rbc, 256);
    L.part_m = o; o = align_up(o + 4 * rbc, 256);
    L.part_r = o; o = align_up(o + 8 * rbc, 256);
    L.part_c = o; o = align_up(o + 8 * rbc, 256);
    L.row_m = o;  o = align_up(o + 4 * rb, 256);
    L.rcum = o;   o = align_up(o + 8 * rbc, 256);
    L.wcum = o;   o = align_up(o + 8 * rb, 256);
    L.cterm = o;  o = align_up(o + 8 * rb, 256);
    L.total = o;
    return L;
}

// Tree-attention workspace:
//   status  u32 [R]
//   part_o  f16 [S][R*Hkv][G*B][D]  split outputs o_s / l_s in units of 2^u_s
//   part_ml f32 [S][R*Hkv][G*B][4]  running max m_s (log2 units), sum l_s, u_s
struct AttnPlan {
    int nqt, nw;          // query tiles (16 rows) per wave, waves per workgroup
    int rows_per_wg;      // nw * nqt * 16
    int row_blocks;       // ceil(G*B / rows_per_wg)
    int splits;           // prefix splits
    int keys_per_split;   // multiple of 32
};

struct AttnWs {
    size_t status, part_o, part_ml, total;
};

// reserve: CUs the attention leaves free for other workgroups of the same
// launch (the fused round runs the reach beside it).  The stand-alone call
// keeps one free as well: with whole-block splits the last split, which also
// holds the masked tree keys, then gets the short remainder of the prefix.
AttnPlan attn_plan(int R, int B, int Hq, int Hkv, int D, int P, int reserve = 1);

inline AttnWs attn_ws_layout(int R, int B, int Hq, int Hkv, int D, int P, int reserve = 1) {
    AttnPlan pl = attn_plan(R, B, Hq, Hkv, D, P, reserve);
    const int G = Hq / Hkv;
    const size_t rows = (size_t)R * Hkv * G * B;
    AttnWs L{};
    size_t o = 0;
    L.status = o; o = align_up(o + 4 * (size_t)R, 256);
    const size_t S = pl.splits > 1 ? (size_t)pl.splits : 0;
    L.part_o = o;  o = align_up(o + 2 * S * rows * D, 256);
    L.part_ml = o; o = align_up(o + 16 * S * rows, 256);
    L.total = o;
    return L;
}

// Verification-round workspace: the exit-law workspace, then the attention
// workspace of the plan that leaves the reach its CUs.
struct RoundWs {
    size_t exit, attn, total;
    int reserve;
};

inline int round_reserve(int R) { return R < 8 ? (R > 1 ? R : 1) : 8; }

inline RoundWs round_ws_layout(int R, int B, int V, int Hq, int Hkv, int D, int P) {
    RoundWs L{};
    L.reserve = round_reserve(R);
    L.exit = 0;
    L.attn = align_up(exit_ws_layout(R, B, V).total, 256);
    L.total = L.attn + attn_ws_layout(R, B, Hq, Hkv, D, P, L.reserve).total;
    return L;
}

// ---- launchers (return hipGetLastError() of the launches) ----
hipError_t launch_vocab(const void *logits, int dtype, bool vec, const int32_t *parents,
                        const int32_t *tokens, int R, int B, int V, float sL, char *ws,
                        hipStream_t st);
hipError_t launch_exit_law(const void *logits, int dtype, bool vec, const int32_t *parents,
                           const int32_t *tokens, int R, int B, int V, float sL, float *rho,
                           float *reach, float *exit_mass, float *coverage, char *ws,
                           hipStream_t st);
hipError_t launch_sample(const void *logits, int dtype, bool vec, const int32_t *parents,
                         const int32_t *tokens, int R, int B, int V, float sL, const char *ws,
                         const float *uniforms, int n_draws, int32_t *exit_node,
                         int32_t *bonus_token, hipStream_t st);
hipError_t launch_predraw(const void *logits, int dtype, bool vec, const int32_t *parents,
                          const int32_t *tokens, int R, int B, int V, float sL, const char *ws,
                          const float *uniforms, int n_draws, int32_t *node_draw,
                          int32_t *exit_node, int32_t *bonus_token, hipStream_t st);
hipError_t launch_commit_kv(void *k, void *v, int dtype, const int32_t *parents,
                            const int32_t *exit_node, int R, int B, int L, int Hkv, int D, int P,
                            int32_t *new_len, hipStream_t st);
hipError_t launch_residual_cdf(const void *logits, int dtype, bool vec, const int32_t *parents,
                               const int32_t *tokens, int R, int B, int V, float sL,
                               const char *ws, int r, int node, double *cdf, hipStream_t st);
hipError_t launch_tree_attn(const void *q, const void *k, const void *v, int dtype,
                            const int32_t *parents, int R, int B, int Hq, int Hkv, int D, int P,
                            float scale, float *out, char *ws, hipStream_t st);

hipError_t launch_round(const void *q, const void *k, const void *v, const void *logits, int dtype,
                        bool vec, const int32_t *parents, const int32_t *tokens, int R, int B,
                        int V, int Hq, int Hkv, int D, int P, float scale, float sL,
                        const float *uniforms, int n_draws, float *attn_out, float *rho,
                        float *reach, float *exit_mass, float *coverage, int32_t *exit_node,
                        int32_t *bonus_token, char *ws, hipStream_t st,
                        void *const *events = nullptr);

}  // namespace tev
