// round.hip -- one whole verification round in three launches on gfx950.
//
// The round computes exactly what tev_tree_attn, tev_exit_law and tev_sample
// compute one after the other (tree attention: "CAST: Cost-Aware Speculative
// Trees from One-Pass Block Drafters", App. B Lemma 1 and App. C; exit law and
// draws: "Where Draft Trees Lose Target Mass: Exit-Guided Speculative
// Decoding", Sec. 3 Eq. 1-2, Sec. 3.1 Eq. 4, Sec. 3.2 Eq. 6-7, App. B
// Algorithm 1), but packs the work so that the single-workgroup steps run
// beside the wide ones instead of after them:
//
//   1. k_vocab                       -- the logit stream (all CUs);
//   2. k_round_attn = attention workgroups + one reach workgroup per request:
//      the attention plan leaves that many CUs free, and the reach needs only
//      the vocabulary pass, finished by the stream order.  With at most
//      DRAWS_IN_REACH draws per request the reach workgroup also makes them,
//      right after the exit CDF (the same arithmetic as a draw workgroup);
//   3. k_round_tail = the split combine of the attention, and the draw
//      workgroups when there are more draws (they need the reach, the
//      combine the attention, both done).  No launch when neither is left.
//
// Workgroups of one launch never wait for each other, so no cross-workgroup
// synchronisation is involved; the roles only share the launch.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "exit_law_dev.h"
#include "tev_internal.h"
#include "tree_attn_dev.h"

namespace tev {
namespace {

// Launch 2: workgroups [0, attn_grid) are attention tasks, the next R are the
// reach of request b - attn_grid (512 threads, NB batches of rows).
constexpr int DRAWS_IN_REACH = 4;

template <int D, int NQT, int NB>
__global__ __launch_bounds__(NT) void k_round_attn(AttnArgs a, ReachArgs ra, int attn_grid,
                                                   SampleArgs<uint16_t> sa, int reach_draws, int vec) {
    const int b = (int)blockIdx.x;
    if (b >= attn_grid) {
        const int r = b - attn_grid;
        reach_wg<NB, NT>(ra, r);
        if (reach_draws) {
            __syncthreads();   // the exit CDF, residual sums and status of request r
            for (int n = 0; n < sa.n_draws; n++) {
                if (vec) sample_wg<uint16_t, true, NT>(sa, n, r);
                else sample_wg<uint16_t, false, NT>(sa, n, r);
            }
        }
        return;
    }
    const int task = xcd_task(b, a.n_wg);
    if (task >= a.n_wg) return;
    attn_mfma_wg<D, NQT>(a, task);
}

struct CombineArgs {
    const uint16_t *part_o;
    const float *part_ml;
    int splits, Hkv, G, B, Hq;
    size_t rows_all;
    const unsigned *status;
    float *out;
};

// Launch 3: workgroups [0, R * n_draws) draw (request b / n_draws, draw
// b % n_draws), the rest combine the attention splits.
template <int D, typename T, bool VEC>
__global__ __launch_bounds__(VOCAB_THREADS) void k_round_tail(SampleArgs<T> sa, int sbx, int n_sample,
                                                            CombineArgs ca) {
    const int b = (int)blockIdx.x;
    if (b < n_sample) {
        sample_wg<T, VEC>(sa, b % sbx, b / sbx);   // sbx = draws per request
        return;
    }
    attn_combine_wg<D>(ca.part_o, ca.part_ml, ca.splits, ca.Hkv, ca.G, ca.B, ca.Hq, ca.rows_all,
                       ca.status, ca.out, b - n_sample);
}

struct RoundDraws {
    SampleArgs<uint16_t> sa;
    int in_reach, vec;
};

template <int D, int NQT, int NB>
void launch_round_attn(const AttnArgs &a, const ReachArgs &ra, int attn_grid, int R,
                       const RoundDraws &rd, hipStream_t st) {
    k_round_attn<D, NQT, NB><<<dim3((unsigned)(attn_grid + R)), NT, 0, st>>>(a, ra, attn_grid, rd.sa,
                                                                             rd.in_reach, rd.vec);
}

template <int D, int NQT>
void round_attn_nb(const AttnArgs &a, const ReachArgs &ra, int attn_grid, int R, int B,
                   const RoundDraws &rd, hipStream_t st) {
    const int nb = reach_batches(B, NT);
    if (nb <= 2) launch_round_attn<D, NQT, 2>(a, ra, attn_grid, R, rd, st);
    else if (nb <= 4) launch_round_attn<D, NQT, 4>(a, ra, attn_grid, R, rd, st);
    else launch_round_attn<D, NQT, 8>(a, ra, attn_grid, R, rd, st);
}

// n_draws draw workgroups per request, then the combine workgroups of the
// split partials (none without splits; no launch when neither is left).
template <int D, typename T, bool VEC>
void launch_round_tail(const SampleArgs<T> &sa, int R, int n_draws, const CombineArgs &ca,
                       hipStream_t st) {
    static_assert(SAMPLE_THREADS == VOCAB_THREADS, "draw and combine workgroups share a launch");
    const int n_combine = ca.splits > 1 ? (int)((ca.rows_all + 3) / 4) : 0;
    const int sbx = n_draws;
    const int n_sample = R * sbx;
    if (n_sample + n_combine == 0) return;
    k_round_tail<D, T, VEC><<<dim3((unsigned)(n_sample + n_combine)), VOCAB_THREADS, 0, st>>>(
        sa, sbx, n_sample, ca);
}

template <int D, typename T>
void round_tail_vec(bool vec, const SampleArgs<T> &sa, int R, int n_draws, const CombineArgs &ca,
                    hipStream_t st) {
    if (vec) launch_round_tail<D, T, true>(sa, R, n_draws, ca, st);
    else launch_round_tail<D, T, false>(sa, R, n_draws, ca, st);
}

}  // namespace

hipError_t launch_round(const void *q, const void *k, const void *v, const void *logits, int dtype,
                        bool vec, const int32_t *parents, const int32_t *tokens, int R, int B,
                        int V, int Hq, int Hkv, int D, int P, float scale, float sL,
                        const float *uniforms, int n_draws, float *attn_out, float *rho,
                        float *reach, float *exit_mass, float *coverage, int32_t *exit_node,
                        int32_t *bonus_token, char *ws, hipStream_t st, void *const *events) {
    const RoundWs RL = round_ws_layout(R, B, V, Hq, Hkv, D, P);
    // optional caller events at the launch boundaries (profiling)
    auto mark = [&](int i) {
        if (events && events[i]) (void)hipEventRecord((hipEvent_t)events[i], st);
    };
    char *ws_e = ws + RL.exit;
    char *ws_a = ws + RL.attn;
    if (dtype != TEV_BF16) {
        // fp32 attention runs on the vector ALU path: the three calls in
        // order (events: before the exit law, after it, after the attention,
        // after the draws)
        mark(0);
        hipError_t e = launch_exit_law(logits, dtype, vec, parents, tokens, R, B, V, sL, rho, reach,
                                       exit_mass, coverage, ws_e, st);
        mark(1);
        if (e == hipSuccess)
            e = launch_tree_attn(q, k, v, dtype, parents, R, B, Hq, Hkv, D, P, scale, attn_out, ws_a, st);
        mark(2);
        if (e == hipSuccess)
            e = launch_sample(logits, dtype, vec, parents, tokens, R, B, V, sL, ws_e, uniforms,
                              n_draws, exit_node, bonus_token, st);
        mark(3);
        return e;
    }

    // 1. the vocabulary pass
    mark(0);
    hipError_t e = launch_vocab(logits, dtype, vec, parents, tokens, R, B, V, sL, ws_e, st);
    if (e != hipSuccess) return e;
    mark(1);

    // 2. attention + reach
    const AttnPlan pl = attn_plan(R, B, Hq, Hkv, D, P, RL.reserve);
    const AttnWs AL = attn_ws_layout(R, B, Hq, Hkv, D, P, RL.reserve);
    uint16_t *part_o = (uint16_t *)(ws_a + AL.part_o);
    float *part_ml = (float *)(ws_a + AL.part_ml);
    unsigned *astatus = (unsigned *)(ws_a + AL.status);
    const int n_wg = pl.row_blocks * pl.splits * R * Hkv;
    const int attn_grid = 8 * ((n_wg + 7) / 8);
    const float c_log2 = (float)((double)scale * 1.4426950408889634);
    const AttnArgs a{(const uint16_t *)q, (const uint16_t *)k, (const uint16_t *)v, parents, B, Hq, Hkv,
                     P, c_log2, pl.row_blocks, pl.splits, pl.keys_per_split, n_wg, attn_out, part_o,
                     part_ml, astatus};
    const ReachArgs ra{parents, tokens, B, V, n_chunks(V), sL, exit_ptrs(ws_e, R, B, V), rho, reach,
                       exit_mass, coverage};
    const SampleArgs<uint16_t> sa = sample_args((const uint16_t *)logits, parents, tokens, R, B, V, sL,
                                                ws_e, uniforms, n_draws, exit_node, bonus_token);
    const RoundDraws rd{sa, n_draws <= DRAWS_IN_REACH ? 1 : 0, vec ? 1 : 0};
    if (D == 64 && pl.nqt == 1) round_attn_nb<64, 1>(a, ra, attn_grid, R, B, rd, st);
    else if (D == 64) round_attn_nb<64, 2>(a, ra, attn_grid, R, B, rd, st);
    else if (pl.nqt == 1) round_attn_nb<128, 1>(a, ra, attn_grid, R, B, rd, st);
    else round_attn_nb<128, 2>(a, ra, attn_grid, R, B, rd, st);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    mark(2);

    // 3. split combine, and the draws left to a launch of their own
    const int G = Hq / Hkv;
    const size_t rows_all = (size_t)R * Hkv * G * B;
    const CombineArgs ca{part_o, part_ml, pl.splits, Hkv, G, B, Hq, rows_all, astatus, attn_out};
    const int tail_draws = rd.in_reach ? 0 : n_draws;
    if (D == 64) round_tail_vec<64, uint16_t>(vec, sa, R, tail_draws, ca, st);
    else round_tail_vec<128, uint16_t>(vec, sa, R, tail_draws, ca, st);
    e = hipGetLastError();
    mark(3);
    return e;
}

}  // namespace tev
