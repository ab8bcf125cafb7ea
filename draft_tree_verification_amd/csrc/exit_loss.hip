// exit_loss.hip -- the exit-guided draft-tree loss and its gradient on gfx950.
//
// What is computed ("Where Draft Trees Lose Target Mass: Exit-Guided
// Speculative Decoding", Sec. 5 Eq. 14, evaluated as App. C.2 Eq. 66-67):
// for R examples with trees of B nodes, position-wise draft logits z [R][H][V]
// (row (r, d - 1) scores every node of depth d, d = 1..H) and detached node
// weights w [R][B] (the exit masses w(v)),
//   L = sum_r sum_{v >= 1, w(v) != 0} w(v) (lse(z_{r,d(v)}) - z_{r,d(v),x_v}) / (R (B - 1))
//   dL/dz_m = (Omega_m softmax(z_m) - sum_{v in m} w(v) e_{x_v}) / (R (B - 1)),
// Omega_m the summed weight of row m's nodes.  One logsumexp per row serves
// all of the row's nodes; the nodes only add a gather (App. C.2).
//
// Launches (all HBM streams except the per-example pass):
//   k_loss_slabs  grid (ns, R*H), 256 threads: one 8192-logit slab of one row
//                 per workgroup, 32 logits per thread in registers; writes the
//                 slab's integer log2 offset (floor of max * log2 e) and its
//                 f32 sum of 2^(z log2 e - offset).
//   k_loss_rows   grid R, 1024 threads: node depths by pointer jumping in LDS,
//                 tree checks, one wave per row combines the slab partials in
//                 f64 into the row's logsumexp and lists the row's nodes
//                 (ballots, node order); the nodes gather their logits and the
//                 example's numerator is summed in a fixed order.
//   k_loss_total  one workgroup, only for R > 1: sums the R numerators.
//   k_loss_grad   (only with a gradient output) grid (ns, R*H): re-reads the
//                 slab, writes Omega/N * 2^(z log2 e - lse2) and subtracts the
//                 listed nodes' w/N at their tokens; rows no node scores are
//                 written as zeros without reading the logits.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "exit_law_dev.h"
#include "exit_loss.h"
#include "slab_dev.h"
#include "wave_ops.h"

namespace tev {
namespace {

constexpr float kLog2eF = 1.4426950408889634f;
constexpr double kLn2 = 0.69314718055994530942;

struct LossPtrs {
    unsigned *status;
    float *slab_m, *slab_s;
    double *lse2, *omega, *num;
    int32_t *ent_n, *ent_tok;
    float *ent_w;
};

LossPtrs loss_ptrs(char *ws, const LossWs &L) {
    return LossPtrs{(unsigned *)(ws + L.status), (float *)(ws + L.slab_m), (float *)(ws + L.slab_s),
                    (double *)(ws + L.lse2),     (double *)(ws + L.omega), (double *)(ws + L.num),
                    (int32_t *)(ws + L.ent_n),   (int32_t *)(ws + L.ent_tok), (float *)(ws + L.ent_w)};
}

// The same ownership for the f32 gradient: VW floats per group, stored as
// 16-byte vectors when VEC (then len is a multiple of VW).
template <typename T, bool VEC>
__device__ __forceinline__ void store_slab(float *g, int len, int tid, const float *val) {
    constexpr int VW = 16 / (int)sizeof(T);
    constexpr int SPAN = LOSS_THREADS * VW;
#pragma unroll
    for (int k = 0; k < LOSS_EPT / VW; k++) {
        const int idx = k * SPAN + tid * VW;
        if (VEC) {
            if (idx < len) {
#pragma unroll
                for (int j = 0; j < VW; j += 4)
                    *reinterpret_cast<float4 *>(g + idx + j) =
                        float4{val[k * VW + j], val[k * VW + j + 1], val[k * VW + j + 2], val[k * VW + j + 3]};
            }
        } else {
#pragma unroll
            for (int j = 0; j < VW; j++)
                if (idx + j < len) g[idx + j] = val[k * VW + j];
        }
    }
}

template <typename T, bool VEC>
__global__ __launch_bounds__(LOSS_THREADS) void k_loss_slabs(const T *__restrict__ z, int V, int ns,
                                                             float *__restrict__ slab_m,
                                                             float *__restrict__ slab_s) {
    __shared__ float s_max[LOSS_THREADS / 64], s_sum[LOSS_THREADS / 64];
    const int tid = threadIdx.x, s = blockIdx.x;
    const size_t m = blockIdx.y;
    const int start = s * LOSS_SLAB, len = min(LOSS_SLAB, V - start);
    float x[LOSS_EPT];
    load_slab<T, VEC, LOSS_THREADS, LOSS_EPT>(z + m * (size_t)V + start, len, tid, x);
    float mx = x[0];
#pragma unroll
    for (int j = 1; j < LOSS_EPT; j++) mx = fmaxf(mx, x[j]);
    mx = wave::max_f32(mx);
    if ((tid & 63) == 0) s_max[tid >> 6] = mx;
    __syncthreads();
    mx = fmaxf(fmaxf(s_max[0], s_max[1]), fmaxf(s_max[2], s_max[3]));
    // An integer offset: the row combine rescales slabs by exact powers of two.
    // -inf for an all -inf slab (sum 0); a NaN or +inf logit makes the sum NaN.
    const float Ms = floorf(mx * kLog2eF);
    float sum = Ms != Ms ? __builtin_nanf("") : 0.f;   // an all-NaN slab stays NaN
    if (Ms > -kInf) {
#pragma unroll
        for (int j = 0; j < LOSS_EPT; j++) sum += __builtin_amdgcn_exp2f(fmaf(x[j], kLog2eF, -Ms));
    }
    sum = wave::sum_f32(sum);
    if ((tid & 63) == 0) s_sum[tid >> 6] = sum;
    __syncthreads();
    if (tid == 0) {
        slab_m[m * ns + s] = Ms;
        slab_s[m * ns + s] = (s_sum[0] + s_sum[1]) + (s_sum[2] + s_sum[3]);
    }
}

__device__ __forceinline__ double block_sum_f64(double x, double *red) {
    constexpr int NWV = LOSS_ROW_THREADS / 64;
    x = wave::sum_f64(x);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = x;
    __syncthreads();
    double t = 0.0;
#pragma unroll
    for (int i = 0; i < NWV; i++) t += red[i];     // fixed order: reproducible
    return t;
}

template <typename T>
__global__ __launch_bounds__(LOSS_ROW_THREADS) void k_loss_rows(
    const T *__restrict__ z, const int32_t *__restrict__ parents, const int32_t *__restrict__ tokens,
    const float *__restrict__ weights, int B, int H, int V, int ns, LossPtrs W,
    float *__restrict__ row_lse, float *__restrict__ row_weight, float *__restrict__ loss) {
    constexpr int NWV = LOSS_ROW_THREADS / 64;
    __shared__ int s_anc[TEV_MAX_NODES], s_dist[TEV_MAX_NODES], s_tok[TEV_MAX_NODES];
    __shared__ float s_w[TEV_MAX_NODES];
    __shared__ double s_lse[LOSS_MAX_H], s_om[LOSS_MAX_H];
    __shared__ double s_red[NWV];
    __shared__ unsigned s_flags;
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, r = blockIdx.x;
    if (tid == 0) s_flags = 0u;
    int tok = 0;
    float w = 0.f;
    bool bad = false;
    if (tid < B) {
        const int p = parents[(size_t)r * B + tid];
        tok = tokens[(size_t)r * B + tid];
        w = weights[(size_t)r * B + tid];
        bad = tid == 0 ? p != -1 : (p < 0 || p >= tid || tok < 0 || tok >= V);
        s_anc[tid] = (tid == 0 || bad) ? 0 : p;
        s_dist[tid] = tid == 0 ? 0 : 1;
        s_tok[tid] = tok;
        s_w[tid] = w;
    }
    __syncthreads();
    if (bad) atomicOr(&s_flags, (unsigned)TEV_FLAG_TREE);
    // Pointer jumping: after round k every node points 2^k levels up (or at
    // the root) and s_dist counts the levels climbed; ceil(log2 B) rounds.
    for (int span = 1; span < B; span *= 2) {
        int a = 0, d = 0;
        if (tid < B) {
            const int an = s_anc[tid];
            a = s_anc[an];
            d = s_dist[tid] + s_dist[an];
        }
        __syncthreads();
        if (tid < B) {
            s_anc[tid] = a;
            s_dist[tid] = d;
        }
        __syncthreads();
    }
    const int depth = tid < B ? s_dist[tid] : 0;
    if (tid >= 1 && tid < B && depth > H) atomicOr(&s_flags, (unsigned)TEV_FLAG_TREE);
    // node v's term needs z at (its row, its token); the load is issued before
    // the rows are combined
    const bool scored = tid >= 1 && tid < B && !bad && w != 0.f && depth <= H;
    float zx = 0.f;
    if (scored) zx = to_f32<T>(z[((size_t)r * H + depth - 1) * V + tok]);

    for (int d = wv; d < H; d += NWV) {
        const size_t m = (size_t)r * H + d;
        float mrow = -kInf;
        for (int s = lane; s < ns; s += 64) mrow = fmaxf(mrow, W.slab_m[m * ns + s]);
        mrow = wave::max_f32(mrow);
        double acc = 0.0;
        for (int s = lane; s < ns; s += 64) {
            const float ms = W.slab_m[m * ns + s];
            const float ss = W.slab_s[m * ns + s];
            // a NaN sum survives the product with 0; an all -inf slab adds 0
            acc += (ms > -kInf) ? (double)ss * pow2_int(ms - mrow) : (double)ss;
        }
        acc = wave::sum_f64(acc);
        const double lse2 = mrow > -kInf ? (double)mrow + log2(acc) : -(double)kInf;
        // the row's nodes, in node order
        int cnt = 0;
        double om = 0.0;
        for (int c = 0; c < B; c += 64) {
            const int v = c + lane;
            const bool hit = v >= 1 && v < B && s_dist[v] == d + 1 && s_w[v] != 0.f;
            const uint64_t mask = __ballot(hit);
            if (hit) {
                const int pos = cnt + __popcll(mask & ((1ull << lane) - 1ull));
                W.ent_tok[m * B + pos] = s_tok[v];
                W.ent_w[m * B + pos] = s_w[v];
                om += (double)s_w[v];
            }
            cnt += __popcll(mask);
        }
        om = wave::sum_f64(om);
        if (lane == 0) {
            W.lse2[m] = lse2;
            W.omega[m] = om;
            W.ent_n[m] = cnt;
            s_lse[d] = lse2 * kLn2;
            s_om[d] = om;
            if (!isfinite(lse2)) atomicOr(&s_flags, (unsigned)TEV_FLAG_NONFINITE);
        }
    }
    __syncthreads();
    const unsigned fl = s_flags;
    const double term = scored ? (double)w * (s_lse[depth - 1] - (double)zx) : 0.0;
    const double num = block_sum_f64(term, s_red);
    const float qnan = __builtin_nanf("");
    for (int d = tid; d < H; d += LOSS_ROW_THREADS) {
        const size_t m = (size_t)r * H + d;
        row_lse[m] = fl ? qnan : (float)s_lse[d];
        row_weight[m] = fl ? qnan : (float)s_om[d];
    }
    if (tid == 0) {
        W.status[r] = fl;
        W.num[r] = fl ? (double)qnan : num;
        if (gridDim.x == 1) loss[0] = fl ? qnan : (B > 1 ? (float)(num / (double)(B - 1)) : 0.f);
    }
}

__global__ __launch_bounds__(LOSS_ROW_THREADS) void k_loss_total(const double *__restrict__ num,
                                                                 int R, int B, float *__restrict__ loss) {
    __shared__ double s_red[LOSS_ROW_THREADS / 64];
    double t = 0.0;
    for (int r = threadIdx.x; r < R; r += LOSS_ROW_THREADS) t += num[r];
    t = block_sum_f64(t, s_red);
    if (threadIdx.x == 0) loss[0] = B > 1 ? (float)(t / ((double)R * (B - 1))) : 0.f;
}

template <typename T, bool VEC>
__global__ __launch_bounds__(LOSS_THREADS) void k_loss_grad(const T *__restrict__ z, int B, int H, int V,
                                                            double invN, LossPtrs W,
                                                            float *__restrict__ grad) {
    constexpr int VW = 16 / (int)sizeof(T);
    const int tid = threadIdx.x, s = blockIdx.x;
    const size_t m = blockIdx.y;
    const int r = (int)(m / H);
    const int start = s * LOSS_SLAB, len = min(LOSS_SLAB, V - start);
    const unsigned fl = W.status[r];
    const double om = W.omega[m];
    float val[LOSS_EPT];
    if (fl != 0u || om == 0.0) {
        // a flagged example is NaN; a row that scores no node has gradient 0
        const float f = fl ? __builtin_nanf("") : 0.f;
#pragma unroll
        for (int j = 0; j < LOSS_EPT; j++) val[j] = f;
    } else {
        float x[LOSS_EPT];
        load_slab<T, VEC, LOSS_THREADS, LOSS_EPT>(z + m * (size_t)V + start, len, tid, x);
        const float c = (float)(om * invN);
        const float l2 = (float)W.lse2[m];
#pragma unroll
        for (int j = 0; j < LOSS_EPT; j++) val[j] = c * __builtin_amdgcn_exp2f(fmaf(x[j], kLog2eF, -l2));
        // the one-hot part: each listed node takes w/N off its token
        const int n = W.ent_n[m];
        for (int e = 0; e < n; e++) {
            const int idx = W.ent_tok[m * B + e] - start;
            if (idx >= 0 && idx < len && tid == (idx / VW) % LOSS_THREADS) {
                const int k = idx / (LOSS_THREADS * VW), j = idx % VW;
                const float dw = (float)((double)W.ent_w[m * B + e] * invN);
#pragma unroll
                for (int kk = 0; kk < LOSS_EPT / VW; kk++)
#pragma unroll
                    for (int jj = 0; jj < VW; jj++)
                        if (kk == k && jj == j) val[kk * VW + jj] -= dw;
            }
        }
    }
    store_slab<T, VEC>(grad + m * (size_t)V + start, len, tid, val);
}

template <typename T, bool VEC>
hipError_t launch_typed(const void *z, const int32_t *parents, const int32_t *tokens,
                        const float *weights, int R, int B, int H, int V, float *loss,
                        float *row_lse, float *row_weight, float *grad, char *ws, hipStream_t st) {
    const LossWs L = loss_ws_layout(R, B, H, V);
    const LossPtrs W = loss_ptrs(ws, L);
    const int ns = loss_slabs(V);
    const dim3 slabs((unsigned)ns, (unsigned)(R * H));
    const T *zt = static_cast<const T *>(z);
    k_loss_slabs<T, VEC><<<slabs, LOSS_THREADS, 0, st>>>(zt, V, ns, W.slab_m, W.slab_s);
    k_loss_rows<T><<<R, LOSS_ROW_THREADS, 0, st>>>(zt, parents, tokens, weights, B, H, V, ns, W,
                                                   row_lse, row_weight, loss);
    if (R > 1) k_loss_total<<<1, LOSS_ROW_THREADS, 0, st>>>(W.num, R, B, loss);
    if (grad) {
        const double invN = B > 1 ? 1.0 / ((double)R * (B - 1)) : 0.0;
        k_loss_grad<T, VEC><<<slabs, LOSS_THREADS, 0, st>>>(zt, B, H, V, invN, W, grad);
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_exit_loss(const void *draft_logits, int dtype, bool vec, const int32_t *parents,
                            const int32_t *tokens, const float *weights, int R, int B, int H, int V,
                            float *loss, float *row_lse, float *row_weight, float *grad, char *ws,
                            hipStream_t st) {
    if (dtype == TEV_BF16)
        return vec ? launch_typed<uint16_t, true>(draft_logits, parents, tokens, weights, R, B, H, V,
                                                  loss, row_lse, row_weight, grad, ws, st)
                   : launch_typed<uint16_t, false>(draft_logits, parents, tokens, weights, R, B, H, V,
                                                   loss, row_lse, row_weight, grad, ws, st);
    return vec ? launch_typed<float, true>(draft_logits, parents, tokens, weights, R, B, H, V, loss,
                                           row_lse, row_weight, grad, ws, st)
               : launch_typed<float, false>(draft_logits, parents, tokens, weights, R, B, H, V, loss,
                                            row_lse, row_weight, grad, ws, st);
}

}  // namespace tev
