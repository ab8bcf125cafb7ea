// exit_law.hip -- the exit law and TEV's two draws on gfx950.
//
// What is computed ("Where Draft Trees Lose Target Mass: Exit-Guided
// Speculative Decoding", Sec. 3 Eq. 1-2, Sec. 3.1 Eq. 4, Sec. 3.2 Eq. 6-7,
// App. B Algorithm 1):
//   p_v = softmax(s * logits[v]),  rho(v) = sum of p_v over non-child tokens,
//   P(0) = 1, P(u) = P(pa(u)) p_pa(u)(x_u),  w = P rho,  C = sum_{u>0} P(u),
//   V = inverse CDF of w at u1,  Y = inverse CDF of p_V^res at u2.
//
// Kernels:
//   k_vocab   one pass over the B*V logits, one workgroup per (row, chunk of
//             8192 tokens): the chunk maximum, then the chunk's sum of
//             2^(l*sL - M_c) split into a residual part (non-child tokens,
//             masked through an LDS bitmap of the row's child tokens) and a
//             child part.  HBM-bound: each logit is read once.
//   k_reach   one workgroup per request: fixed-order fp64 combine of the
//             chunk sums, child probabilities in fp64, rho, the reach P level
//             by level (a barrier per depth), w, C and the exit CDF.
//   k_sample  one workgroup per (draw, request): exit draw over the node CDF,
//             chunk search over the row's running residual sums, then an fp64
//             scan inside the one chunk that holds the bonus token.
//
// Numerics: sL = fl(s * log2 e); each element contributes
// 2^(fma(l, sL, -M_c)) with one rounding of the shifted exponent, M_c being a
// per-chunk f32 offset that cancels exactly in the fp64 combine.  Residual
// sums are formed by masking child tokens, never by subtracting them.  Chunk
// and row combines, child probabilities, P, w, C and both CDFs are fp64.  All
// reductions run in a fixed order (no float atomics): results are
// bit-reproducible.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "tev_internal.h"

namespace tev {
namespace {

constexpr float kInf = __builtin_inff();

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

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
    return x;
}
__device__ __forceinline__ double wave_sum(double x) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o);
    return x;
}
__device__ __forceinline__ int wave_sum_i(int x) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o);
    return x;
}
__device__ __forceinline__ int wave_max_i(int x) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) x = max(x, __shfl_xor(x, o));
    return x;
}

// Block reductions for 256 threads (4 waves); every thread gets the result.
__device__ __forceinline__ float block_max256(float x, float *s4) {
    x = wave_max(x);
    const int w = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) s4[w] = x;
    __syncthreads();
    const float r = fmaxf(fmaxf(s4[0], s4[1]), fmaxf(s4[2], s4[3]));
    __syncthreads();
    return r;
}
__device__ __forceinline__ double block_sum256(double x, double *s4) {
    x = wave_sum(x);
    const int w = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) s4[w] = x;
    __syncthreads();
    const double r = (s4[0] + s4[1]) + (s4[2] + s4[3]);
    __syncthreads();
    return r;
}
__device__ __forceinline__ int block_sum256_i(int x, int *s4) {
    x = wave_sum_i(x);
    const int w = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) s4[w] = x;
    __syncthreads();
    const int r = (s4[0] + s4[1]) + (s4[2] + s4[3]);
    __syncthreads();
    return r;
}
__device__ __forceinline__ int block_max256_i(int x, int *s4) {
    x = wave_max_i(x);
    const int w = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) s4[w] = x;
    __syncthreads();
    const int r = max(max(s4[0], s4[1]), max(s4[2], s4[3]));
    __syncthreads();
    return r;
}

// Marks, in an LDS bitmap of CHUNK bits, the child tokens of node v that fall
// in [c0, c0 + len).  Returns (through *dup) whether two children share a
// token.  Must be followed by a barrier before the bitmap is read.
__device__ __forceinline__ void build_child_mask(const int32_t *par, const int32_t *tok, int B, int v,
                                                 int c0, int len, unsigned *s_mask, int *s_dup) {
    for (int u = 1 + (int)threadIdx.x; u < B; u += VOCAB_THREADS) {
        if (par[u] == v) {
            const int o = tok[u] - c0;
            if (o >= 0 && o < len) {
                const unsigned bit = 1u << (o & 31);
                const unsigned old = atomicOr(&s_mask[o >> 5], bit);
                if (old & bit) *s_dup = 1;
            }
        }
    }
}

// ----------------------------------------------------------------------------
// k_vocab: grid (nc, R*B), 256 threads.  Thread t holds the elements
// k*(256*VW) + t*VW + j of its chunk (VW elements per 16-byte vector).
// ----------------------------------------------------------------------------
template <typename T, bool VEC>
__global__ __launch_bounds__(VOCAB_THREADS) void k_vocab(
    const T *__restrict__ logits, const int32_t *__restrict__ parents,
    const int32_t *__restrict__ tokens, int B, int V, int nc, float sL,
    unsigned *__restrict__ flags, float *__restrict__ part_m, double *__restrict__ part_r,
    double *__restrict__ part_c) {
    constexpr int VW = 16 / (int)sizeof(T);
    constexpr int NV = EPT / VW;
    constexpr unsigned VMASK = (1u << VW) - 1u;
    const int c = blockIdx.x;
    const int rv = blockIdx.y;
    const int r = rv / B, v = rv - r * B;
    const int tid = threadIdx.x;
    const int c0 = c * CHUNK;
    const int len = min(CHUNK, V - c0);

    __shared__ unsigned s_mask[CHUNK / 32];
    __shared__ float s_f[4];
    __shared__ double s_d[4];
    __shared__ int s_dup;

    // Issue the logit loads first; they are independent of the bitmap.
    const T *row = logits + (size_t)rv * (size_t)V + c0;
    float x[EPT];
#pragma unroll
    for (int k = 0; k < NV; k++) {
        const int idx = k * (VOCAB_THREADS * VW) + tid * VW;
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

    for (int i = tid; i < CHUNK / 32; i += VOCAB_THREADS) s_mask[i] = 0u;
    if (tid == 0) s_dup = 0;
    __syncthreads();
    build_child_mask(parents + (size_t)r * B, tokens + (size_t)r * B, B, v, c0, len, s_mask, &s_dup);

    float m = x[0];
#pragma unroll
    for (int j = 1; j < EPT; j++) m = fmaxf(m, x[j]);
    m = block_max256(m, s_f);   // the barrier inside also publishes s_mask

    const float Mc = m * sL;
    double accR = 0.0, accC = 0.0;
    if (m > -kInf) {
#pragma unroll
        for (int k = 0; k < NV; k++) {
            const int idx = k * (VOCAB_THREADS * VW) + tid * VW;
            float e[VW];
#pragma unroll
            for (int j = 0; j < VW; j++) e[j] = __builtin_amdgcn_exp2f(fmaf(x[k * VW + j], sL, -Mc));
            const unsigned bits = (s_mask[(idx >> 5) & (CHUNK / 32 - 1)] >> (idx & 31)) & VMASK;
            if (bits) {
                float cs = 0.f;
#pragma unroll
                for (int j = 0; j < VW; j++)
                    if ((bits >> j) & 1u) { cs += e[j]; e[j] = 0.f; }
                accC += (double)cs;
            }
            // pairwise sum of the vector's terms
#pragma unroll
            for (int w = VW / 2; w >= 1; w >>= 1)
#pragma unroll
                for (int j = 0; j < w; j++) e[j] += e[j + w];
            accR += (double)e[0];
        }
    }
    const double R = block_sum256(accR, s_d);
    const double C = block_sum256(accC, s_d);
    if (tid == 0) {
        const size_t o = (size_t)rv * nc + c;
        unsigned f = 0u;
        if (!(m == m) || m == kInf || isnan(R) || isnan(C)) f |= TEV_FLAG_NONFINITE;
        if (s_dup) f |= TEV_FLAG_TREE;
        flags[o] = f;
        part_m[o] = (m > -kInf) ? Mc : -kInf;
        part_r[o] = R;
        part_c[o] = C;
    }
}

// ----------------------------------------------------------------------------
// k_reach: grid (R), 256 threads, thread v owns node v.
// ----------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(256) void k_reach(
    const T *__restrict__ logits, const int32_t *__restrict__ parents,
    const int32_t *__restrict__ tokens, int B, int V, int nc, float sL,
    const unsigned *__restrict__ flags, const float *__restrict__ part_m,
    const double *__restrict__ part_r, const double *__restrict__ part_c,
    float *__restrict__ row_m, double *__restrict__ rcum, double *__restrict__ wcum,
    unsigned *__restrict__ status, float *__restrict__ rho_out, float *__restrict__ reach_out,
    float *__restrict__ w_out, float *__restrict__ cov_out) {
    const int r = blockIdx.x;
    const int v = threadIdx.x;
    const bool active = v < B;
    __shared__ int s_par[256];
    __shared__ float s_M[256];
    __shared__ double s_Z[256];
    __shared__ double s_P[256];
    __shared__ double s_scan[256];
    __shared__ unsigned s_flags;
    __shared__ int s_i4[4];

    if (v == 0) s_flags = 0u;
    __syncthreads();

    unsigned f = 0u;
    int pa = -1, tk = 0;
    double rho = 1.0;
    if (active) {
        pa = parents[(size_t)r * B + v];
        tk = tokens[(size_t)r * B + v];
        if (v == 0) {
            if (pa != -1) f |= TEV_FLAG_TREE;
        } else if (pa < 0 || pa >= v || tk < 0 || tk >= V) {
            f |= TEV_FLAG_TREE;
        }
        s_par[v] = (f & TEV_FLAG_TREE) ? 0 : pa;
        const size_t base = ((size_t)r * B + v) * nc;
        float M = -kInf;
        for (int c = 0; c < nc; c++) {
            f |= flags[base + c];
            M = fmaxf(M, part_m[base + c]);
        }
        if (!(M > -kInf)) f |= TEV_FLAG_NONFINITE;
        double Rs = 0.0, Cs = 0.0;
        for (int c = 0; c < nc; c++) {
            const float mc = part_m[base + c];
            const double sc = (mc > -kInf) ? exp2((double)mc - (double)M) : 0.0;
            Rs += part_r[base + c] * sc;
            Cs += part_c[base + c] * sc;
            rcum[base + c] = Rs;
        }
        const double Z = Rs + Cs;
        if (!(Z > 0.0) || isnan(Z)) f |= TEV_FLAG_NONFINITE;
        s_Z[v] = Z;
        s_M[v] = M;
        row_m[(size_t)r * B + v] = M;
        rho = Rs / Z;
        if (f) atomicOr(&s_flags, f);
    }
    __syncthreads();
    const unsigned fl = s_flags;
    if (fl) {
        const float qnan = __builtin_nanf("");
        if (active) {
            rho_out[(size_t)r * B + v] = qnan;
            reach_out[(size_t)r * B + v] = qnan;
            w_out[(size_t)r * B + v] = qnan;
            wcum[(size_t)r * B + v] = __builtin_nan("");
        }
        if (v == 0) {
            cov_out[r] = qnan;
            status[r] = fl;
        }
        return;
    }

    // Child probability p_pa(v)(x_v), fp64, against the parent's combined row.
    double pc = 0.0;
    int depth = 0;
    if (active && v > 0) {
        const float l = to_f32<T>(logits[((size_t)r * B + pa) * (size_t)V + tk]);
        pc = exp2((double)l * (double)sL - (double)s_M[pa]) / s_Z[pa];
        for (int j = v; j > 0; j = s_par[j]) depth++;
    }
    const int maxdepth = block_max256_i(active ? depth : 0, s_i4);

    // Reach, level by level: every node of depth d reads its parent's P,
    // final since the previous level's barrier (Algorithm 1, loop over depth).
    if (v == 0) s_P[0] = 1.0;
    for (int d = 1; d <= maxdepth; d++) {
        __syncthreads();
        if (active && depth == d) s_P[v] = s_P[pa] * pc;
    }
    __syncthreads();
    const double P = active ? s_P[v] : 0.0;
    const double w = P * rho;

    // Coverage: fixed-order tree sum of P over non-root nodes.
    s_scan[v] = (active && v > 0) ? P : 0.0;
    __syncthreads();
    for (int o = 128; o > 0; o >>= 1) {
        if (v < o) s_scan[v] += s_scan[v + o];
        __syncthreads();
    }
    const double C = s_scan[0];
    __syncthreads();

    // Exit CDF: inclusive Hillis-Steele scan of w in node-index order.
    s_scan[v] = active ? w : 0.0;
    __syncthreads();
    for (int o = 1; o < 256; o <<= 1) {
        const double add = (v >= o) ? s_scan[v - o] : 0.0;
        __syncthreads();
        s_scan[v] += add;
        __syncthreads();
    }
    if (active) {
        wcum[(size_t)r * B + v] = s_scan[v];
        rho_out[(size_t)r * B + v] = (float)rho;
        reach_out[(size_t)r * B + v] = (float)P;
        w_out[(size_t)r * B + v] = (float)w;
    }
    if (v == 0) {
        cov_out[r] = (float)C;
        status[r] = 0u;
    }
}

// ----------------------------------------------------------------------------
// In-chunk residual terms on a contiguous segment: thread t owns tokens
// [t*EPT, t*EPT + EPT) of the chunk, so a block scan runs in token order.
// Each term is computed exactly as in k_vocab (same f32 operations and
// offset), child tokens are zero.
// ----------------------------------------------------------------------------
template <typename T, bool VEC>
__device__ __forceinline__ void segment_terms(const T *chunk, int len, float sL, float Mc,
                                              const unsigned *s_mask, float *e) {
    constexpr int VW = 16 / (int)sizeof(T);
    const int base = threadIdx.x * EPT;
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
    const unsigned bits = s_mask[threadIdx.x];   // EPT == 32: one word per thread
#pragma unroll
    for (int j = 0; j < EPT; j++) {
        const float t = __builtin_amdgcn_exp2f(fmaf(x[j], sL, -Mc));
        e[j] = ((bits >> j) & 1u) ? 0.f : t;
    }
}

// Exclusive block scan (fp64) of one value per thread, 256 threads.
__device__ __forceinline__ double block_exclusive_scan256(double x, double *s_scan) {
    const int t = threadIdx.x;
    s_scan[t] = x;
    __syncthreads();
    for (int o = 1; o < 256; o <<= 1) {
        const double add = (t >= o) ? s_scan[t - o] : 0.0;
        __syncthreads();
        s_scan[t] += add;
        __syncthreads();
    }
    const double incl = s_scan[t];
    __syncthreads();
    return incl - x;
}

// ----------------------------------------------------------------------------
// k_sample: grid (n_draws, R), 256 threads.
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
    const int n = blockIdx.x;
    const int r = blockIdx.y;
    const int tid = threadIdx.x;
    const size_t kd = (size_t)r * n_draws + n;
    if (status[r] != 0u) {
        if (tid == 0) { exit_node[kd] = -1; bonus_token[kd] = -1; }
        return;
    }
    __shared__ int s_i4[4];
    __shared__ unsigned s_mask[CHUNK / 32];
    __shared__ double s_scan[256];
    __shared__ int s_dup;

    const double u1 = (double)uniforms[2 * kd];
    const double u2 = (double)uniforms[2 * kd + 1];

    // Exit node: number of j with W_j <= u1 * S is the smallest j with u1 S < W_j.
    const double *W = wcum + (size_t)r * B;
    const double t1 = u1 * W[B - 1];
    int cnt = 0;
    for (int j = tid; j < B; j += 256) cnt += (W[j] <= t1) ? 1 : 0;
    int Vn = block_sum256_i(cnt, s_i4);
    if (Vn >= B) {   // rounding left no bin: last node with positive mass
        int best = -1;
        for (int j = tid; j < B; j += 256)
            if (j == 0 ? (W[0] > 0.0) : (W[j] > W[j - 1])) best = max(best, j);
        Vn = max(block_max256_i(best, s_i4), 0);
    }

    // Bonus token: chunk whose running residual sum first exceeds u2 * T.
    const size_t rb = (size_t)r * B + Vn;
    const double *RC = rcum + rb * nc;
    const double t2 = u2 * RC[nc - 1];
    int cc = 0;
    for (int c = tid; c < nc; c += 256) cc += (RC[c] <= t2) ? 1 : 0;
    cc = block_sum256_i(cc, s_i4);
    if (cc >= nc) {
        int best = -1;
        for (int c = tid; c < nc; c += 256)
            if (part_r[rb * nc + c] > 0.0) best = max(best, c);
        cc = max(block_max256_i(best, s_i4), 0);
    }
    const double before = (cc > 0) ? RC[cc - 1] : 0.0;
    const float Mv = row_m[rb];
    const float Mc = part_m[rb * nc + cc];
    const double target = (t2 - before) * exp2((double)Mv - (double)Mc);

    const int c0 = cc * CHUNK;
    const int len = min(CHUNK, V - c0);
    for (int i = tid; i < CHUNK / 32; i += 256) s_mask[i] = 0u;
    if (tid == 0) s_dup = 0;
    __syncthreads();
    build_child_mask(parents + (size_t)r * B, tokens + (size_t)r * B, B, Vn, c0, len, s_mask, &s_dup);
    __syncthreads();

    float e[EPT];
    segment_terms<T, VEC>(logits + rb * (size_t)V + c0, len, sL, Mc, s_mask, e);
    double seg = 0.0;
#pragma unroll
    for (int j = 0; j < EPT; j++) seg += (double)e[j];
    double run = block_exclusive_scan256(seg, s_scan);
    int below = 0, last_pos = -1;
#pragma unroll
    for (int j = 0; j < EPT; j++) {
        run += (double)e[j];
        below += (run <= target) ? 1 : 0;
        if (e[j] > 0.f) last_pos = tid * EPT + j;
    }
    below = block_sum256_i(below, s_i4);
    if (below >= len) below = max(block_max256_i(last_pos, s_i4), 0);
    if (tid == 0) {
        exit_node[kd] = Vn;
        bonus_token[kd] = c0 + below;
    }
}

// ----------------------------------------------------------------------------
// k_residual_cdf: grid (nc), 256 threads; the sampler's residual CDF of one
// (request, node) row at every token, normalised by the row total.
// ----------------------------------------------------------------------------
template <typename T, bool VEC>
__global__ __launch_bounds__(VOCAB_THREADS) void k_residual_cdf(
    const T *__restrict__ logits, const int32_t *__restrict__ parents,
    const int32_t *__restrict__ tokens, int B, int V, int nc, float sL,
    const unsigned *__restrict__ status, const float *__restrict__ part_m,
    const float *__restrict__ row_m, const double *__restrict__ rcum, int r, int node,
    double *__restrict__ cdf) {
    const int cc = blockIdx.x;
    const int tid = threadIdx.x;
    __shared__ unsigned s_mask[CHUNK / 32];
    __shared__ double s_scan[256];
    __shared__ int s_dup;
    const int c0 = cc * CHUNK;
    const int len = min(CHUNK, V - c0);
    if (status[r] != 0u) {
        for (int a = tid; a < len; a += 256) cdf[c0 + a] = __builtin_nan("");
        return;
    }
    const size_t rb = (size_t)r * B + node;
    const double *RC = rcum + rb * nc;
    const double total = RC[nc - 1];
    const double before = (cc > 0) ? RC[cc - 1] : 0.0;
    const float Mv = row_m[rb];
    const float Mc = part_m[rb * nc + cc];
    const double scale = exp2((double)Mc - (double)Mv);
    for (int i = tid; i < CHUNK / 32; i += 256) s_mask[i] = 0u;
    if (tid == 0) s_dup = 0;
    __syncthreads();
    build_child_mask(parents + (size_t)r * B, tokens + (size_t)r * B, B, node, c0, len, s_mask, &s_dup);
    __syncthreads();
    float e[EPT];
    segment_terms<T, VEC>(logits + rb * (size_t)V + c0, len, sL, Mc, s_mask, e);
    double seg = 0.0;
#pragma unroll
    for (int j = 0; j < EPT; j++) seg += (double)e[j];
    double run = block_exclusive_scan256(seg, s_scan);
#pragma unroll
    for (int j = 0; j < EPT; j++) {
        run += (double)e[j];
        const int a = tid * EPT + j;
        if (a < len) cdf[c0 + a] = (before + run * scale) / total;
    }
}

template <typename T, bool VEC>
hipError_t exit_law_impl(const T *logits, const int32_t *parents, const int32_t *tokens, int R,
                         int B, int V, float sL, float *rho, float *reach, float *w, float *cov,
                         char *ws, hipStream_t st) {
    const ExitWs L = exit_ws_layout(R, B, V);
    const int nc = n_chunks(V);
    k_vocab<T, VEC><<<dim3(nc, R * B), VOCAB_THREADS, 0, st>>>(
        logits, parents, tokens, B, V, nc, sL, (unsigned *)(ws + L.flags), (float *)(ws + L.part_m),
        (double *)(ws + L.part_r), (double *)(ws + L.part_c));
    k_reach<T><<<dim3(R), 256, 0, st>>>(
        logits, parents, tokens, B, V, nc, sL, (const unsigned *)(ws + L.flags),
        (const float *)(ws + L.part_m), (const double *)(ws + L.part_r),
        (const double *)(ws + L.part_c), (float *)(ws + L.row_m), (double *)(ws + L.rcum),
        (double *)(ws + L.wcum), (unsigned *)(ws + L.status), rho, reach, w, cov);
    return hipGetLastError();
}

template <typename T, bool VEC>
hipError_t sample_impl(const T *logits, const int32_t *parents, const int32_t *tokens, int R,
                       int B, int V, float sL, const char *ws, const float *uniforms,
                       int n_draws, int32_t *exit_node, int32_t *bonus, hipStream_t st) {
    const ExitWs L = exit_ws_layout(R, B, V);
    const int nc = n_chunks(V);
    k_sample<T, VEC><<<dim3(n_draws, R), VOCAB_THREADS, 0, st>>>(
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
    (void)R;
    const ExitWs L = exit_ws_layout(R, B, V);
    const int nc = n_chunks(V);
    k_residual_cdf<T, VEC><<<dim3(nc), VOCAB_THREADS, 0, st>>>(
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
