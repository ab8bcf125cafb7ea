// exit_law.hip -- the exit law and TEV's two draws on gfx950.
//
// What is computed ("Where Draft Trees Lose Target Mass: Exit-Guided
// Speculative Decoding", Sec. 3 Eq. 1-2, Sec. 3.1 Eq. 4, Sec. 3.2 Eq. 6-7,
// App. B Algorithm 1):
//   p_v = softmax(s * logits[v]),  rho(v) = sum of p_v over non-child tokens,
//   P(0) = 1, P(u) = P(pa(u)) p_pa(u)(x_u),  w = P rho,  C = sum_{u>0} P(u),
//   V = inverse CDF of w at u1,  Y = inverse CDF of p_V^res at u2.
//
// k_vocab -- grid (ceil(nc / 4), R*B), 4 independent waves per workgroup,
// each wave on its own 4096-token chunk of one logit row, no workgroup
// barrier: the chunk maximum, then the chunk's sum of 2^(l*sL - M_c) split
// into a residual part (non-child tokens, masked through a per-wave LDS bitmap
// of the row's child tokens) and a child part.  Each logit is read exactly
// once: this pass is HBM-bound.
//
// k_reach -- one workgroup of 512 threads per request:
//   row pass (8 waves, rows dealt round-robin, four rows' chunk partials in
//   flight per wave): fixed-order fp64 combine of the row's chunk sums and the
//   running residual sums the sampler searches; rho by masking, never by
//   subtraction.
//   tree pass (wave 0, on the row results in LDS): child probabilities in
//   fp64, the reach P level by level (Algorithm 1's loop over depth, one
//   wave-level LDS sync per level), w, C and the exit CDF.
//
// k_sample -- one wave per (draw, request): exit draw over the node CDF,
// chunk search over the row's running residual sums, then an fp64 wave scan
// inside the one chunk that holds the bonus token.
//
// Numerics: sL = fl(s * log2 e); each element contributes
// 2^(fma(l, sL, -M_c)) with one rounding of the shifted exponent, M_c being a
// per-chunk f32 offset that cancels exactly in the fp64 combine.  Chunk and
// row combines, child probabilities, P, w, C and both CDFs are fp64.  All
// reductions run in a fixed order (no float atomics): results are
// bit-reproducible.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "tev_internal.h"
#include "wave_ops.h"

namespace tev {
namespace {

constexpr float kInf = __builtin_inff();
constexpr int NPL = TEV_MAX_NODES / 64;   // tree nodes per lane in the tree pass

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

template <typename T>
__device__ __forceinline__ float to_f32(T x);
template <>
__device__ __forceinline__ float to_f32<float>(float x) { return x; }
template <>
__device__ __forceinline__ float to_f32<uint16_t>(uint16_t x) {
    return __uint_as_float(((uint32_t)x) << 16);
}

// 16 bytes of logits -> floats.
__device__ __forceinline__ void load16(const float *p, float *x) {
    const float4 v = *reinterpret_cast<const float4 *>(p);
    x[0] = v.x; x[1] = v.y; x[2] = v.z; x[3] = v.w;
}
__device__ __forceinline__ void load16(const uint16_t *p, float *x) {
    const uint4 v = *reinterpret_cast<const uint4 *>(p);
    x[0] = bf16_lo(v.x); x[1] = bf16_hi(v.x);
    x[2] = bf16_lo(v.y); x[3] = bf16_hi(v.y);
    x[4] = bf16_lo(v.z); x[5] = bf16_hi(v.z);
    x[6] = bf16_lo(v.w); x[7] = bf16_hi(v.w);
}

struct ExitPtrs {
    unsigned *status, *flags;
    float *part_m, *row_m;
    double *part_r, *part_c, *rcum, *wcum;
};

// ----------------------------------------------------------------------------
// k_vocab.  Chunk c of row rv: lane t holds the elements k*(64*VW) + t*VW + j
// (coalesced 16-byte vectors); the row's child tokens inside the chunk are
// marked in a per-wave LDS bitmap whose word t belongs to lane t.
// ----------------------------------------------------------------------------
template <typename T, bool VEC>
__global__ __launch_bounds__(VOCAB_THREADS) void k_vocab(
    const T *__restrict__ logits, const int32_t *__restrict__ parents,
    const int32_t *__restrict__ tokens, int B, int V, int nc, float sL, ExitPtrs W) {
    constexpr int VW = 16 / (int)sizeof(T);
    constexpr int NV = EPT / VW;
    constexpr int SPAN = 64 * VW;
    constexpr unsigned VMASK = (1u << VW) - 1u;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int c = blockIdx.x * WAVES_PER_WG + wave;
    const int rv = blockIdx.y;
    const int r = rv / B, v = rv - r * B;
    __shared__ unsigned s_mask[WAVES_PER_WG][128];
    if (c >= nc) return;
    const int c0 = c * CHUNK;
    const int len = min(CHUNK, V - c0);
    const int32_t *par = parents + (size_t)r * B;
    const int32_t *tok = tokens + (size_t)r * B;

    const T *row = logits + (size_t)rv * (size_t)V + c0;
    float x[EPT];
#pragma unroll
    for (int k = 0; k < NV; k++) {
        const int idx = k * SPAN + lane * VW;
        if (VEC) {
            if (idx < len) {
                load16(row + idx, &x[k * VW]);
            } else {
#pragma unroll
                for (int j = 0; j < VW; j++) x[k * VW + j] = -kInf;
            }
        } else {
#pragma unroll
            for (int j = 0; j < VW; j++)
                x[k * VW + j] = (idx + j < len) ? to_f32<T>(row[idx + j]) : -kInf;
        }
    }
    s_mask[wave][2 * lane] = 0u;
    s_mask[wave][2 * lane + 1] = 0u;
    wave::lds_sync();
    bool dup = false;
    for (int u = 1 + lane; u < B; u += 64) {
        if (par[u] == v) {
            const int o = tok[u] - c0;
            if (o >= 0 && o < len) {
                const int k = o / SPAN, rem = o - k * SPAN;
                const int bitpos = k * VW + (rem % VW);            // 0..63 within the owner lane
                const unsigned bit = 1u << (bitpos & 31);
                const unsigned old = atomicOr(&s_mask[wave][2 * (rem / VW) + (bitpos >> 5)], bit);
                dup |= (old & bit) != 0u;
            }
        }
    }
    wave::lds_sync();
    const uint64_t mybits = (uint64_t)s_mask[wave][2 * lane] | ((uint64_t)s_mask[wave][2 * lane + 1] << 32);
    const bool wave_has_children = __any(mybits != 0ull);

    float m = x[0];
#pragma unroll
    for (int j = 1; j < EPT; j++) m = fmaxf(m, x[j]);
    m = wave::max_f32(m);
    const float Mc = m * sL;
    double accR = 0.0, accC = 0.0;
    if (m > -kInf) {
        if (!wave_has_children) {
            // common case: no child token of v in this chunk
#pragma unroll
            for (int k = 0; k < NV; k++) {
                float e[VW];
#pragma unroll
                for (int j = 0; j < VW; j++) e[j] = __builtin_amdgcn_exp2f(fmaf(x[k * VW + j], sL, -Mc));
#pragma unroll
                for (int w = VW / 2; w >= 1; w >>= 1)
#pragma unroll
                    for (int j = 0; j < w; j++) e[j] += e[j + w];
                accR += (double)e[0];
            }
        } else {
#pragma unroll
            for (int k = 0; k < NV; k++) {
                float e[VW];
#pragma unroll
                for (int j = 0; j < VW; j++) e[j] = __builtin_amdgcn_exp2f(fmaf(x[k * VW + j], sL, -Mc));
                const unsigned bits = (unsigned)(mybits >> (k * VW)) & VMASK;
                float cs = 0.f;
#pragma unroll
                for (int j = 0; j < VW; j++) {
                    const bool child = (bits >> j) & 1u;
                    cs += child ? e[j] : 0.f;
                    e[j] = child ? 0.f : e[j];
                }
                accC += (double)cs;
#pragma unroll
                for (int w = VW / 2; w >= 1; w >>= 1)
#pragma unroll
                    for (int j = 0; j < w; j++) e[j] += e[j + w];
                accR += (double)e[0];
            }
        }
    }
    const double Rc = wave::sum_f64(accR);
    const double Cc = wave::sum_f64(accC);
    const bool any_dup = __any(dup);
    if (lane == 0) {
        const size_t o = (size_t)rv * nc + c;
        unsigned f = 0u;
        if (!(m == m) || m == kInf || isnan(Rc) || isnan(Cc)) f |= TEV_FLAG_NONFINITE;
        if (any_dup) f |= TEV_FLAG_TREE;
        W.flags[o] = f;
        W.part_m[o] = (m > -kInf) ? Mc : -kInf;
        W.part_r[o] = Rc;
        W.part_c[o] = Cc;
    }
}

// ----------------------------------------------------------------------------
// k_reach.
// ----------------------------------------------------------------------------
constexpr int REACH_THREADS = 512;
constexpr int REACH_WAVES = REACH_THREADS / 64;
constexpr int ROW_BATCH = 4;        // rows whose partials a wave keeps in flight
constexpr int FAST_NC = 128;        // chunks per row held in registers (2 per lane)

template <typename T>
__global__ __launch_bounds__(REACH_THREADS) void k_reach(
    const T *__restrict__ logits, const int32_t *__restrict__ parents,
    const int32_t *__restrict__ tokens, int B, int V, int nc, float sL, ExitPtrs W,
    float *__restrict__ rho_out, float *__restrict__ reach_out, float *__restrict__ w_out,
    float *__restrict__ cov_out) {
    const int r = blockIdx.x;
    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63;
    __shared__ int s_par[TEV_MAX_NODES];
    __shared__ float s_M[TEV_MAX_NODES];
    __shared__ double s_Z[TEV_MAX_NODES];
    __shared__ double s_rho[TEV_MAX_NODES];
    __shared__ double s_P[TEV_MAX_NODES];
    __shared__ unsigned s_flags;
    const size_t rb0 = (size_t)r * B;

    if (tid == 0) s_flags = 0u;
    __syncthreads();
    // tree contract, one thread per node
    if (tid < B) {
        const int pa = parents[rb0 + tid];
        const int tk = tokens[rb0 + tid];
        const bool bad = (tid == 0) ? (pa != -1) : (pa < 0 || pa >= tid || tk < 0 || tk >= V);
        s_par[tid] = bad ? 0 : pa;
        if (bad) atomicOr(&s_flags, TEV_FLAG_TREE);
    }

    // ---- row pass ----
    for (int v0 = wave; v0 < B; v0 += REACH_WAVES * ROW_BATCH) {
        float pm[ROW_BATCH][2];
        unsigned pf[ROW_BATCH][2];
        double pr[ROW_BATCH][2], pcs[ROW_BATCH][2];
        const bool fast = nc <= FAST_NC;
        if (fast) {
#pragma unroll
            for (int q = 0; q < ROW_BATCH; q++) {
                const int v = v0 + q * REACH_WAVES;
#pragma unroll
                for (int h = 0; h < 2; h++) {
                    const int cc = lane + 64 * h;
                    const bool ok = v < B && cc < nc;
                    const size_t o = (rb0 + (ok ? v : 0)) * nc + (ok ? cc : 0);
                    pm[q][h] = ok ? W.part_m[o] : -kInf;
                    pf[q][h] = ok ? W.flags[o] : 0u;
                    pr[q][h] = ok ? W.part_r[o] : 0.0;
                    pcs[q][h] = ok ? W.part_c[o] : 0.0;
                }
            }
        }
#pragma unroll
        for (int q = 0; q < ROW_BATCH; q++) {
            const int v = v0 + q * REACH_WAVES;
            if (v >= B) break;
            const size_t base = (rb0 + v) * nc;
            float M;
            unsigned f;
            double carry = 0.0, csum = 0.0;
            if (fast) {
                M = wave::max_f32(fmaxf(pm[q][0], pm[q][1]));
                f = wave::or_u32(pf[q][0] | pf[q][1]);
#pragma unroll
                for (int h = 0; h < 2; h++) {
                    const int cc = lane + 64 * h;
                    const double sc = (pm[q][h] > -kInf) ? exp2((double)pm[q][h] - (double)M) : 0.0;
                    const double rs = pr[q][h] * sc;
                    csum += pcs[q][h] * sc;
                    const double incl = wave::incl_scan_f64(rs, lane);
                    if (cc < nc) W.rcum[base + cc] = carry + incl;
                    carry += wave::last_lane_d(incl);
                }
            } else {
                M = -kInf;
                f = 0u;
                for (int cc = lane; cc < nc; cc += 64) {
                    M = fmaxf(M, W.part_m[base + cc]);
                    f |= W.flags[base + cc];
                }
                M = wave::max_f32(M);
                f = wave::or_u32(f);
                for (int b0 = 0; b0 < nc; b0 += 64) {
                    const int cc = b0 + lane;
                    double rs = 0.0;
                    if (cc < nc) {
                        const float mc = W.part_m[base + cc];
                        const double sc = (mc > -kInf) ? exp2((double)mc - (double)M) : 0.0;
                        rs = W.part_r[base + cc] * sc;
                        csum += W.part_c[base + cc] * sc;
                    }
                    const double incl = wave::incl_scan_f64(rs, lane);
                    if (cc < nc) W.rcum[base + cc] = carry + incl;
                    carry += wave::last_lane_d(incl);
                }
            }
            csum = wave::sum_f64(csum);
            const double Z = carry + csum;
            if (!(M > -kInf) || !(Z > 0.0) || isnan(Z)) f |= TEV_FLAG_NONFINITE;
            if (lane == 0) {
                s_M[v] = M;
                s_Z[v] = Z;
                s_rho[v] = carry / Z;
                W.row_m[rb0 + v] = M;
                if (f) atomicOr(&s_flags, f);
            }
        }
    }
    __syncthreads();
    if (wave != 0) return;

    // ---- tree pass (wave 0): lane owns nodes NPL*lane .. NPL*lane + NPL - 1 ----
    const unsigned fl = s_flags;
    if (fl) {
        const float qnan = __builtin_nanf("");
#pragma unroll
        for (int k = 0; k < NPL; k++) {
            const int u = lane * NPL + k;
            if (u < B) {
                rho_out[rb0 + u] = qnan;
                reach_out[rb0 + u] = qnan;
                w_out[rb0 + u] = qnan;
                W.wcum[rb0 + u] = __builtin_nan("");
            }
        }
        if (lane == 0) {
            cov_out[r] = qnan;
            W.status[r] = fl;
        }
        return;
    }
    int pa[NPL], depth[NPL];
    double pc[NPL];
    int maxd = 0;
#pragma unroll
    for (int k = 0; k < NPL; k++) {
        const int u = lane * NPL + k;
        pa[k] = 0;
        depth[k] = 0;
        pc[k] = 0.0;
        if (u > 0 && u < B) {
            pa[k] = s_par[u];
            const int tk = tokens[rb0 + u];
            const float l = to_f32<T>(logits[(rb0 + pa[k]) * (size_t)V + tk]);
            pc[k] = exp2((double)l * (double)sL - (double)s_M[pa[k]]) / s_Z[pa[k]];
            for (int j = u; j > 0; j = s_par[j]) depth[k]++;
            maxd = max(maxd, depth[k]);
        }
    }
    maxd = wave::max_i32(maxd);
    // Reach, level by level (Algorithm 1's loop over depth): the nodes of
    // depth d read their parent's P, final since the previous level.
    if (lane == 0) s_P[0] = 1.0;
    for (int d = 1; d <= maxd; d++) {
        wave::lds_sync();
#pragma unroll
        for (int k = 0; k < NPL; k++)
            if (depth[k] == d) s_P[lane * NPL + k] = s_P[pa[k]] * pc[k];
    }
    wave::lds_sync();
    double P[NPL], w[NPL];
    double lane_c = 0.0, lane_w = 0.0;
#pragma unroll
    for (int k = 0; k < NPL; k++) {
        const int u = lane * NPL + k;
        P[k] = 0.0;
        w[k] = 0.0;
        if (u < B) {
            P[k] = s_P[u];
            w[k] = P[k] * s_rho[u];
            if (u > 0) lane_c += P[k];
        }
    }
    const double C = wave::sum_f64(lane_c);
    // Exit CDF: running sums in node order (lane-local, then across lanes).
#pragma unroll
    for (int k = 0; k < NPL; k++) lane_w += w[k];
    double run = wave::incl_scan_f64(lane_w, lane) - lane_w;
#pragma unroll
    for (int k = 0; k < NPL; k++) {
        const int u = lane * NPL + k;
        run += w[k];
        if (u < B) {
            W.wcum[rb0 + u] = run;
            rho_out[rb0 + u] = (float)s_rho[u];
            reach_out[rb0 + u] = (float)P[k];
            w_out[rb0 + u] = (float)w[k];
        }
    }
    if (lane == 0) {
        cov_out[r] = (float)C;
        W.status[r] = 0u;
    }
}

// ----------------------------------------------------------------------------
// In-chunk residual terms on a contiguous segment: lane t owns tokens
// [64t, 64t + 64) of the chunk, so a wave scan runs in token order.  Each term
// is computed exactly as in the chunk pass (same f32 operations and offset);
// child tokens are zero (bit j of the lane's mask word).
// ----------------------------------------------------------------------------
template <typename T, bool VEC>
__device__ __forceinline__ void segment_terms(const T *chunk, int len, float sL, float Mc,
                                              uint64_t bits, int lane, float *e) {
    constexpr int VW = 16 / (int)sizeof(T);
    const int base = lane * EPT;
    float x[EPT];
#pragma unroll
    for (int k = 0; k < EPT / VW; k++) {
        const int idx = base + k * VW;
        if (VEC) {
            if (idx < len) {
                load16(chunk + idx, &x[k * VW]);
            } else {
#pragma unroll
                for (int j = 0; j < VW; j++) x[k * VW + j] = -kInf;
            }
        } else {
#pragma unroll
            for (int j = 0; j < VW; j++) x[k * VW + j] = (idx + j < len) ? to_f32<T>(chunk[idx + j]) : -kInf;
        }
    }
#pragma unroll
    for (int j = 0; j < EPT; j++) {
        const float t = __builtin_amdgcn_exp2f(fmaf(x[j], sL, -Mc));
        e[j] = ((bits >> j) & 1ull) ? 0.f : t;
    }
}

// Child tokens of `node` inside [c0, c0 + len) -> bit (o % 64) of lane
// (o / 64)'s 64-bit mask, matching the contiguous ownership of segment_terms.
__device__ __forceinline__ uint64_t segment_child_bits(const int32_t *par, const int32_t *tok, int B,
                                                       int node, int c0, int len, unsigned *s_wmask,
                                                       int lane) {
    s_wmask[2 * lane] = 0u;
    s_wmask[2 * lane + 1] = 0u;
    wave::lds_sync();
    for (int u = 1 + lane; u < B; u += 64) {
        if (par[u] == node) {
            const int o = tok[u] - c0;
            if (o >= 0 && o < len) atomicOr(&s_wmask[o >> 5], 1u << (o & 31));
        }
    }
    wave::lds_sync();
    return (uint64_t)s_wmask[2 * lane] | ((uint64_t)s_wmask[2 * lane + 1] << 32);
}

// ----------------------------------------------------------------------------
// k_sample: grid (ceil(n_draws / 4), R), 256 threads, one wave per draw.
// ----------------------------------------------------------------------------
template <typename T, bool VEC>
__global__ __launch_bounds__(VOCAB_THREADS) void k_sample(
    const T *__restrict__ logits, const int32_t *__restrict__ parents,
    const int32_t *__restrict__ tokens, int B, int V, int nc, float sL,
    const unsigned *__restrict__ status, const float *__restrict__ part_m,
    const double *__restrict__ part_r, const float *__restrict__ row_m,
    const double *__restrict__ rcum, const double *__restrict__ wcum,
    const float *__restrict__ uniforms, int n_draws, int32_t *__restrict__ exit_node,
    int32_t *__restrict__ bonus_token) {
    const int wave_id = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int n = blockIdx.x * WAVES_PER_WG + wave_id;
    const int r = blockIdx.y;
    __shared__ unsigned s_mask[WAVES_PER_WG][128];
    if (n >= n_draws) return;
    const size_t kd = (size_t)r * n_draws + n;
    if (status[r] != 0u) {
        if (lane == 0) { exit_node[kd] = -1; bonus_token[kd] = -1; }
        return;
    }
    const double u1 = (double)uniforms[2 * kd];
    const double u2 = (double)uniforms[2 * kd + 1];

    // Exit node: the number of j with W_j <= u1 * S is the smallest j with u1 S < W_j.
    const double *Wc = wcum + (size_t)r * B;
    const double t1 = u1 * Wc[B - 1];
    int cnt = 0;
    for (int j = lane; j < B; j += 64) cnt += (Wc[j] <= t1) ? 1 : 0;
    int Vn = wave::sum_i32(cnt);
    if (Vn >= B) {   // rounding left no bin: last node with positive mass
        int best = -1;
        for (int j = lane; j < B; j += 64)
            if (j == 0 ? (Wc[0] > 0.0) : (Wc[j] > Wc[j - 1])) best = max(best, j);
        Vn = max(wave::max_i32(best), 0);
    }

    // Bonus token: the chunk whose running residual sum first exceeds u2 * T.
    const size_t rb = (size_t)r * B + Vn;
    const double *RC = rcum + rb * nc;
    const double t2 = u2 * RC[nc - 1];
    int cc = 0;
    for (int c = lane; c < nc; c += 64) cc += (RC[c] <= t2) ? 1 : 0;
    cc = wave::sum_i32(cc);
    if (cc >= nc) {
        int best = -1;
        for (int c = lane; c < nc; c += 64)
            if (part_r[rb * nc + c] > 0.0) best = max(best, c);
        cc = max(wave::max_i32(best), 0);
    }
    const double before = (cc > 0) ? RC[cc - 1] : 0.0;
    const float Mv = row_m[rb];
    const float Mc = part_m[rb * nc + cc];
    const double target = (t2 - before) * exp2((double)Mv - (double)Mc);

    const int c0 = cc * CHUNK;
    const int len = min(CHUNK, V - c0);
    const uint64_t bits = segment_child_bits(parents + (size_t)r * B, tokens + (size_t)r * B, B, Vn,
                                             c0, len, s_mask[wave_id], lane);
    float e[EPT];
    segment_terms<T, VEC>(logits + rb * (size_t)V + c0, len, sL, Mc, bits, lane, e);
    double seg = 0.0;
#pragma unroll
    for (int j = 0; j < EPT; j++) seg += (double)e[j];
    double run = wave::incl_scan_f64(seg, lane) - seg;
    int below = 0, last_pos = -1;
#pragma unroll
    for (int j = 0; j < EPT; j++) {
        run += (double)e[j];
        below += (run <= target) ? 1 : 0;
        if (e[j] > 0.f) last_pos = lane * EPT + j;
    }
    below = wave::sum_i32(below);
    if (below >= len) below = max(wave::max_i32(last_pos), 0);
    if (lane == 0) {
        exit_node[kd] = Vn;
        bonus_token[kd] = c0 + below;
    }
}

// ----------------------------------------------------------------------------
// k_residual_cdf: grid (ceil(nc / 4)), one wave per chunk; the sampler's
// residual CDF of one (request, node) row at every token, normalised.
// ----------------------------------------------------------------------------
template <typename T, bool VEC>
__global__ __launch_bounds__(VOCAB_THREADS) void k_residual_cdf(
    const T *__restrict__ logits, const int32_t *__restrict__ parents,
    const int32_t *__restrict__ tokens, int B, int V, int nc, float sL,
    const unsigned *__restrict__ status, const float *__restrict__ part_m,
    const float *__restrict__ row_m, const double *__restrict__ rcum, int r, int node,
    double *__restrict__ cdf) {
    const int wave_id = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int cc = blockIdx.x * WAVES_PER_WG + wave_id;
    __shared__ unsigned s_mask[WAVES_PER_WG][128];
    if (cc >= nc) return;
    const int c0 = cc * CHUNK;
    const int len = min(CHUNK, V - c0);
    if (status[r] != 0u) {
        for (int a = lane; a < len; a += 64) cdf[c0 + a] = __builtin_nan("");
        return;
    }
    const size_t rb = (size_t)r * B + node;
    const double *RC = rcum + rb * nc;
    const double total = RC[nc - 1];
    const double before = (cc > 0) ? RC[cc - 1] : 0.0;
    const float Mv = row_m[rb];
    const float Mc = part_m[rb * nc + cc];
    const double scale = exp2((double)Mc - (double)Mv);
    const uint64_t bits = segment_child_bits(parents + (size_t)r * B, tokens + (size_t)r * B, B, node,
                                             c0, len, s_mask[wave_id], lane);
    float e[EPT];
    segment_terms<T, VEC>(logits + rb * (size_t)V + c0, len, sL, Mc, bits, lane, e);
    double seg = 0.0;
#pragma unroll
    for (int j = 0; j < EPT; j++) seg += (double)e[j];
    double run = wave::incl_scan_f64(seg, lane) - seg;
#pragma unroll
    for (int j = 0; j < EPT; j++) {
        run += (double)e[j];
        const int a = lane * EPT + j;
        if (a < len) cdf[c0 + a] = (before + run * scale) / total;
    }
}

ExitPtrs exit_ptrs(char *ws, int R, int B, int V) {
    const ExitWs L = exit_ws_layout(R, B, V);
    ExitPtrs p;
    p.status = (unsigned *)(ws + L.status);
    p.flags = (unsigned *)(ws + L.flags);
    p.part_m = (float *)(ws + L.part_m);
    p.row_m = (float *)(ws + L.row_m);
    p.part_r = (double *)(ws + L.part_r);
    p.part_c = (double *)(ws + L.part_c);
    p.rcum = (double *)(ws + L.rcum);
    p.wcum = (double *)(ws + L.wcum);
    return p;
}

template <typename T, bool VEC>
hipError_t exit_law_impl(const T *logits, const int32_t *parents, const int32_t *tokens, int R,
                         int B, int V, float sL, float *rho, float *reach, float *w, float *cov,
                         char *ws, hipStream_t st) {
    const int nc = n_chunks(V);
    const ExitPtrs P = exit_ptrs(ws, R, B, V);
    k_vocab<T, VEC><<<dim3((nc + WAVES_PER_WG - 1) / WAVES_PER_WG, R * B), VOCAB_THREADS, 0, st>>>(
        logits, parents, tokens, B, V, nc, sL, P);
    k_reach<T><<<dim3(R), REACH_THREADS, 0, st>>>(logits, parents, tokens, B, V, nc, sL, P, rho,
                                                   reach, w, cov);
    return hipGetLastError();
}

template <typename T, bool VEC>
hipError_t sample_impl(const T *logits, const int32_t *parents, const int32_t *tokens, int R,
                       int B, int V, float sL, const char *ws, const float *uniforms,
                       int n_draws, int32_t *exit_node, int32_t *bonus, hipStream_t st) {
    const ExitWs L = exit_ws_layout(R, B, V);
    const int nc = n_chunks(V);
    k_sample<T, VEC><<<dim3((n_draws + WAVES_PER_WG - 1) / WAVES_PER_WG, R), VOCAB_THREADS, 0, st>>>(
        logits, parents, tokens, B, V, nc, sL, (const unsigned *)(ws + L.status),
        (const float *)(ws + L.part_m), (const double *)(ws + L.part_r),
        (const float *)(ws + L.row_m), (const double *)(ws + L.rcum),
        (const double *)(ws + L.wcum), uniforms, n_draws, exit_node, bonus);
    return hipGetLastError();
}

template <typename T, bool VEC>
hipError_t residual_cdf_impl(const T *logits, const int32_t *parents, const int32_t *tokens,
                             int R, int B, int V, float sL, const char *ws, int r, int node,
                             double *cdf, hipStream_t st) {
    const ExitWs L = exit_ws_layout(R, B, V);
    const int nc = n_chunks(V);
    k_residual_cdf<T, VEC><<<dim3((nc + WAVES_PER_WG - 1) / WAVES_PER_WG), VOCAB_THREADS, 0, st>>>(
        logits, parents, tokens, B, V, nc, sL, (const unsigned *)(ws + L.status),
        (const float *)(ws + L.part_m), (const float *)(ws + L.row_m),
        (const double *)(ws + L.rcum), r, node, cdf);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_exit_law(const void *logits, int dtype, bool vec, const int32_t *parents,
                           const int32_t *tokens, int R, int B, int V, float sL, float *rho,
                           float *reach, float *exit_mass, float *coverage, char *ws,
                           hipStream_t st) {
    if (dtype == TEV_BF16) {
        const uint16_t *p = (const uint16_t *)logits;
        return vec ? exit_law_impl<uint16_t, true>(p, parents, tokens, R, B, V, sL, rho, reach, exit_mass, coverage, ws, st)
                   : exit_law_impl<uint16_t, false>(p, parents, tokens, R, B, V, sL, rho, reach, exit_mass, coverage, ws, st);
    }
    const float *p = (const float *)logits;
    return vec ? exit_law_impl<float, true>(p, parents, tokens, R, B, V, sL, rho, reach, exit_mass, coverage, ws, st)
               : exit_law_impl<float, false>(p, parents, tokens, R, B, V, sL, rho, reach, exit_mass, coverage, ws, st);
}

hipError_t launch_sample(const void *logits, int dtype, bool vec, const int32_t *parents,
                         const int32_t *tokens, int R, int B, int V, float sL, const char *ws,
                         const float *uniforms, int n_draws, int32_t *exit_node,
                         int32_t *bonus_token, hipStream_t st) {
    if (dtype == TEV_BF16) {
        const uint16_t *p = (const uint16_t *)logits;
        return vec ? sample_impl<uint16_t, true>(p, parents, tokens, R, B, V, sL, ws, uniforms, n_draws, exit_node, bonus_token, st)
                   : sample_impl<uint16_t, false>(p, parents, tokens, R, B, V, sL, ws, uniforms, n_draws, exit_node, bonus_token, st);
    }
    const float *p = (const float *)logits;
    return vec ? sample_impl<float, true>(p, parents, tokens, R, B, V, sL, ws, uniforms, n_draws, exit_node, bonus_token, st)
               : sample_impl<float, false>(p, parents, tokens, R, B, V, sL, ws, uniforms, n_draws, exit_node, bonus_token, st);
}

hipError_t launch_residual_cdf(const void *logits, int dtype, bool vec, const int32_t *parents,
                               const int32_t *tokens, int R, int B, int V, float sL,
                               const char *ws, int r, int node, double *cdf, hipStream_t st) {
    if (dtype == TEV_BF16) {
        const uint16_t *p = (const uint16_t *)logits;
        return vec ? residual_cdf_impl<uint16_t, true>(p, parents, tokens, R, B, V, sL, ws, r, node, cdf, st)
                   : residual_cdf_impl<uint16_t, false>(p, parents, tokens, R, B, V, sL, ws, r, node, cdf, st);
    }
    const float *p = (const float *)logits;
    return vec ? residual_cdf_impl<float, true>(p, parents, tokens, R, B, V, sL, ws, r, node, cdf, st)
               : residual_cdf_impl<float, false>(p, parents, tokens, R, B, V, sL, ws, r, node, cdf, st);
}

}  // namespace tev
