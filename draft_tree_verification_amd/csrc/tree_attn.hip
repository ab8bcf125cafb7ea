// tree_attn.hip -- one layer of ancestor-masked tree attention on gfx950.
//
// What is computed ("CAST: Cost-Aware Speculative Trees from One-Pass Block
// Drafters", App. B Lemma 1; App. C "Packed verification"): query (r, i, h)
// attends to the P cached prefix rows and to the rows of its own root path
// (itself included) of kv head g = h / G, G = Hq / Hkv; cache row P + j holds
// tree node j.
//
// k_attn_mfma (bf16): one workgroup of eight waves serves up to 128 NQT query
// rows of one (request, kv head) -- the G*B rows (node i, head g*G + hh) share
// that head's K/V, so the GQA group times the tree makes the products dense --
// over one split of the prefix; the last split also takes the B tree rows
// under the ancestor mask.  Each wave owns 16 NQT rows for every 64-key stage
// of the split.  K and V stages sit row-major in LDS, double buffered, while
// the next stages' global loads are in flight.  Scores are formed transposed,
//   S^T (16 keys x 16 queries per tile) = K (16 x D) . Q^T (D x 16),
// with v_mfma_f32_16x16x32_bf16, so each lane holds one query column; its
// online-softmax probabilities, converted to fp16, are exactly the B operand of
//   O^T (D x 16) += V^T (D x 32 keys) . P^T (32 keys x 16),
// (v_mfma_f32_16x16x32_f16, V in fp16 under a per-workgroup power-of-two
// scale) whose V^T operand comes straight from the row-major V stage through
// the transposing LDS read, in the key order the score tiles leave in
// registers.  Tree rows are masked by a per-node ancestor bitmap in LDS (one
// bit per node).  Partial results of split prefixes are merged by
// k_attn_combine.
//
// k_attn_alu (fp32): one wave per query row, lanes over head_dim, online
// softmax in fp32 over blocks of keys -- a plain vector-ALU kernel for fp32
// inputs.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "tev_internal.h"
#include "tree_attn_dev.h"
#include "wave_ops.h"

namespace tev {
namespace {

// ----------------------------------------------------------------------------
// fp32 vector-ALU kernel: grid (ceil(B*Hq/4), R), 256 threads, wave = one row.
// Keys are taken in blocks of ALU_KB (the prefix rows, then the root path of
// node i walked upward through the parents in LDS): the K and V loads of a
// block are issued together (64 values per lane: 32 keys at head_dim 64, 16
// at 128), then the block's scores update the online softmax at once.
// ----------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void k_attn_alu(const float *__restrict__ q,
                                                  const float *__restrict__ k,
                                                  const float *__restrict__ v,
                                                  const int32_t *__restrict__ parents, int B,
                                                  int Hq, int Hkv, int P, float scale,
                                                  float *__restrict__ out,
                                                  unsigned *__restrict__ status) {
    constexpr int PER = D / 64;
    constexpr int ALU_KB = 32 / PER;   // keys per block
    const int r = blockIdx.y;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    __shared__ int s_par[256];
    __shared__ int s_bad;
    const bool ok = load_parents(parents + (size_t)r * B, B, s_par, &s_bad);
    if (blockIdx.x == 0 && threadIdx.x == 0) status[r] = ok ? 0u : TEV_FLAG_TREE;
    const int flat = blockIdx.x * 4 + wave;
    if (flat >= B * Hq) return;
    const int i = flat / Hq, h = flat % Hq;
    const int G = Hq / Hkv, g = h / G;
    float *o = out + (((size_t)r * B + i) * Hq + h) * D;
    if (!ok) {
#pragma unroll
        for (int p = 0; p < PER; p++) o[lane + 64 * p] = __builtin_nanf("");
        return;
    }
    const float *qp = q + (((size_t)r * B + i) * Hq + h) * D;
    const size_t kvrows = (size_t)P + B;
    const float *kb = k + ((size_t)r * Hkv + g) * kvrows * D;
    const float *vb = v + ((size_t)r * Hkv + g) * kvrows * D;
    float qv[PER], acc[PER];
#pragma unroll
    for (int p = 0; p < PER; p++) { qv[p] = qp[lane + 64 * p]; acc[p] = 0.f; }
    float m = -kInf, l = 0.f;
    int j = i;   // next node of the root path (walked upward), -1 when done
    for (int t0 = 0;; t0 += ALU_KB) {
        int rows[ALU_KB];
#pragma unroll
        for (int u = 0; u < ALU_KB; u++) {
            const int t = t0 + u;
            if (t < P) {
                rows[u] = t;
            } else if (j >= 0) {
                rows[u] = P + j;
                j = s_par[j];
            } else {
                rows[u] = -1;
            }
        }
        if (rows[0] < 0) break;
        float kx[ALU_KB][PER], vx[ALU_KB][PER];
#pragma unroll
        for (int u = 0; u < ALU_KB; u++)
#pragma unroll
            for (int p = 0; p < PER; p++) {
                const size_t off = (size_t)max(rows[u], 0) * D + lane + 64 * p;
                kx[u][p] = kb[off];
                vx[u][p] = vb[off];
            }
        float sc[ALU_KB];
        float bm = -kInf;
#pragma unroll
        for (int u = 0; u < ALU_KB; u++) {
            float dot = 0.f;
#pragma unroll
            for (int p = 0; p < PER; p++) dot = fmaf(qv[p], kx[u][p], dot);
            sc[u] = rows[u] >= 0 ? wave_sum_f(dot) * scale : -kInf;
            bm = fmaxf(bm, sc[u]);
        }
        const float mn = fmaxf(m, bm);
        const float alpha = expf(m - mn);
        l *= alpha;
#pragma unroll
        for (int p = 0; p < PER; p++) acc[p] *= alpha;
#pragma unroll
        for (int u = 0; u < ALU_KB; u++) {
            const float pr = rows[u] >= 0 ? expf(sc[u] - mn) : 0.f;
            l += pr;
#pragma unroll
            for (int p = 0; p < PER; p++) acc[p] = fmaf(pr, vx[u][p], acc[p]);
        }
        m = mn;
        if (rows[ALU_KB - 1] < 0) break;
    }
#pragma unroll
    for (int p = 0; p < PER; p++) o[lane + 64 * p] = acc[p] / l;
}

template <int D, int NQT>
__global__ __launch_bounds__(NT) void k_attn_mfma(AttnArgs a) {
    const int task = xcd_task((int)blockIdx.x, a.n_wg);
    if (task >= a.n_wg) return;
    attn_mfma_wg<D, NQT>(a, task);
}

template <int D>
__global__ __launch_bounds__(256) void k_attn_combine(const uint16_t *__restrict__ part_o,
                                                      const float *__restrict__ part_ml,
                                                      int splits, int Hkv, int G, int B, int Hq,
                                                      size_t rows_all,
                                                      const unsigned *__restrict__ status,
                                                      float *__restrict__ out) {
    attn_combine_wg<D>(part_o, part_ml, splits, Hkv, G, B, Hq, rows_all, status, out, (int)blockIdx.x);
}

template <int D, int NQT>
hipError_t mfma_impl(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                     const int32_t *parents, int R, int B, int Hq, int Hkv, int P, float scale,
                     float *out, char *ws, const AttnPlan &pl, hipStream_t st) {
    const AttnWs L = attn_ws_layout(R, B, Hq, Hkv, D, P);
    const float c_log2 = (float)((double)scale * 1.4426950408889634);
    uint16_t *part_o = (uint16_t *)(ws + L.part_o);
    float *part_ml = (float *)(ws + L.part_ml);
    unsigned *status = (unsigned *)(ws + L.status);
    const int n_wg = pl.row_blocks * pl.splits * R * Hkv;
    const int grid = 8 * ((n_wg + 7) / 8);
    const AttnArgs a{q, k, v, parents, B, Hq, Hkv, P, c_log2, pl.row_blocks, pl.splits,
                     pl.keys_per_split, n_wg, out, part_o, part_ml, status};
    k_attn_mfma<D, NQT><<<dim3(grid), NT, 0, st>>>(a);
    if (pl.splits > 1) {
        const int G = Hq / Hkv;
        const size_t rows_all = (size_t)R * Hkv * G * B;
        k_attn_combine<D><<<dim3((unsigned)((rows_all + 3) / 4)), 256, 0, st>>>(
            part_o, part_ml, pl.splits, Hkv, G, B, Hq, rows_all, status, out);
    }
    return hipGetLastError();
}

}  // namespace

AttnPlan attn_plan(int R, int B, int Hq, int Hkv, int D, int P, int reserve) {
    (void)D;
    AttnPlan p{};
    const int G = Hq / Hkv;
    const int rows = G * B;
    // Query tiles per wave (a workgroup serves 8 waves x 16 nqt rows): two
    // once the rows fill them, except for a few kv heads of at most 256 rows,
    // where two row blocks of 128 give more parallelism than more prefix
    // splits (measured at 1 request, 32/8 heads, B = 64, P = 4096).
    p.nqt = (rows > NW * 16 && !(rows <= 2 * NW * 16 && (long)R * Hkv < 32)) ? 2 : 1;
    p.nw = NW;
    p.rows_per_wg = NW * p.nqt * 16;
    p.row_blocks = (rows + p.rows_per_wg - 1) / p.rows_per_wg;
    const long base = (long)R * Hkv * p.row_blocks;
    // At most one workgroup per free CU (256 CUs less the reserve), each split
    // keeping >= 128 prefix keys so that per-split fixed costs stay small.
    long want = (256 - reserve) / base;
    long maxs = P / 128;
    if (maxs < 1) maxs = 1;
    if (maxs > MAX_SPLITS) maxs = MAX_SPLITS;
    int S = (int)(want < maxs ? want : maxs);
    if (S < 1) S = 1;
    int kps = 0;
    if (S > 1) {
        kps = (P + S - 1) / S;
        kps = (kps + 31) / 32 * 32;
        S = (P + kps - 1) / kps;
    }
    p.splits = S;
    p.keys_per_split = S > 1 ? kps : 0;
    return p;
}

hipError_t launch_tree_attn(const void *q, const void *k, const void *v, int dtype,
                            const int32_t *parents, int R, int B, int Hq, int Hkv, int D, int P,
                            float scale, float *out, char *ws, hipStream_t st) {
    const AttnWs L = attn_ws_layout(R, B, Hq, Hkv, D, P);
    if (dtype == TEV_F32) {
        const dim3 grid((unsigned)((B * Hq + 3) / 4), (unsigned)R);
        if (D == 64)
            k_attn_alu<64><<<grid, 256, 0, st>>>((const float *)q, (const float *)k, (const float *)v,
                                                 parents, B, Hq, Hkv, P, scale, out, (unsigned *)(ws + L.status));
        else
            k_attn_alu<128><<<grid, 256, 0, st>>>((const float *)q, (const float *)k, (const float *)v,
                                                  parents, B, Hq, Hkv, P, scale, out, (unsigned *)(ws + L.status));
        return hipGetLastError();
    }
    const AttnPlan pl = attn_plan(R, B, Hq, Hkv, D, P);
    const uint16_t *qb = (const uint16_t *)q, *kb = (const uint16_t *)k, *vb = (const uint16_t *)v;
#define TEV_ATTN_CASE(DD, QQ) \
    if (D == DD && pl.nqt == QQ) return mfma_impl<DD, QQ>(qb, kb, vb, parents, R, B, Hq, Hkv, P, scale, out, ws, pl, st);
    TEV_ATTN_CASE(64, 1) TEV_ATTN_CASE(64, 2)
    TEV_ATTN_CASE(128, 1) TEV_ATTN_CASE(128, 2)
#undef TEV_ATTN_CASE
    return hipErrorInvalidValue;
}

}  // namespace tev
