// exit_law_dev.h -- device code of the exit law and TEV's two draws on gfx950,
// shared by the stand-alone launches and the fused verification round.
//
// What is computed ("Where Draft Trees Lose Target Mass: Exit-Guided
// Speculative Decoding", Sec. 3 Eq. 1-2, Sec. 3.1 Eq. 4, Sec. 3.2 Eq. 6-7,
// App. B Algorithm 1):
//   p_v = softmax(s * logits[v]),  rho(v) = sum of p_v over non-child tokens,
//   P(0) = 1, P(u) = P(pa(u)) p_pa(u)(x_u),  w = P rho,  C = sum_{u>0} P(u),
//   V = inverse CDF of w at u1,  Y = inverse CDF of p_V^res at u2.
//
// k_vocab -- grid (ceil(nc / (4 / SPLIT)), R*B), 4 waves per workgroup, one
// 4096-token chunk of one logit row per SPLIT waves (SPLIT = 2 for small
// problems, where halving the work per wave evens out the last round of waves
// over the SIMDs): the chunk maximum, then the chunk's sum of 2^(l*sL - M_c)
// split into a residual part (non-child tokens, masked through a per-wave LDS
// bitmap of the row's child tokens) and a child part.  Each logit is read
// exactly once: this pass is HBM-bound.
//
// k_reach -- one workgroup of 1024 threads per request:
//   row pass (16 waves, rows dealt round-robin, a batch of four rows' chunk
//   partials loaded together, the next batch issued before this one's
//   stores): fixed-order fp64 combine of the row's chunk sums and the running
//   residual sums the sampler searches; rho by masking, never by subtraction.
//   tree pass (wave 0, on the row results in LDS): child probabilities in
//   fp64 (their logits gathered while the row pass runs), the reach P by
//   pointer jumping along root paths, w, C and the exit CDF.
//
// k_sample -- one 256-thread workgroup per (draw, request), loads in three
// dependent rounds: exit draw over the node CDF, chunk search over the row's
// running residual sums, then an fp64 scan by the four waves together inside
// the one chunk that holds the bonus token.
//
// Numerics: sL = fl(s * log2 e); each element contributes
// 2^(fma(l, sL, -M_c)) with one rounding of the shifted exponent, M_c being
// an integer-valued per-chunk f32 offset (the floor of the chunk's largest
// l * sL), so that every term is below 2 and moving a chunk sum to another
// offset is an exact power of two.  Chunk and row combines, child
// probabilities, P, w, C and both CDFs are fp64.  All reductions run in a
// fixed order (no float atomics): results are bit-reproducible.
#pragma once

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "tev_internal.h"
#include "wave_ops.h"

namespace tev {
namespace {

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
    float2 *cterm;
};

// ----------------------------------------------------------------------------
// k_reach.
// ----------------------------------------------------------------------------
constexpr int ROW_BATCH = 4;        // rows per wave in one pass (one per 16-lane DPP row)
constexpr int SEG_CHUNKS = 4;       // consecutive chunks of a row per lane
constexpr int FAST_NC = 16 * SEG_CHUNKS;   // chunks per row held in registers (16 lanes x 4)

// Passes of rows a workgroup of nth threads needs for B rows.
__host__ __device__ constexpr int reach_batches(int B, int nth) {
    return (B + (nth / 64) * ROW_BATCH - 1) / ((nth / 64) * ROW_BATCH);
}

// Reductions and scans within each 16-lane DPP row (four independent rows
// per wave); every lane of a row receives the row's result.
__device__ __forceinline__ float row16_max_f32(float x) {
    x = fmaxf(x, wave::dpp_f<wave::kQuadXor1>(x));
    x = fmaxf(x, wave::dpp_f<wave::kQuadXor2>(x));
    x = fmaxf(x, wave::dpp_f<wave::kRowHalfMirror>(x));
    return fmaxf(x, wave::dpp_f<wave::kRowMirror>(x));
}
__device__ __forceinline__ unsigned row16_or_u32(unsigned x) {
    int y = (int)x;
    y |= wave::dpp_i<wave::kQuadXor1>(y);
    y |= wave::dpp_i<wave::kQuadXor2>(y);
    y |= wave::dpp_i<wave::kRowHalfMirror>(y);
    return (unsigned)(y | wave::dpp_i<wave::kRowMirror>(y));
}
__device__ __forceinline__ double row16_sum_f64(double x) {
    x += wave::dpp_d<wave::kQuadXor1>(x);
    x += wave::dpp_d<wave::kQuadXor2>(x);
    x += wave::dpp_d<wave::kRowHalfMirror>(x);
    return x + wave::dpp_d<wave::kRowMirror>(x);
}
// inclusive scan over the 16 lanes of each row, in lane order
__device__ __forceinline__ double row16_incl_scan_f64(double x) {
    x += wave::shr_d<1>(x);
    x += wave::shr_d<2>(x);
    x += wave::shr_d<4>(x);
    return x + wave::shr_d<8>(x);
}

// Arguments of the reach for one launch.
struct ReachArgs {
    const int32_t *parents, *tokens;
    int B, V, nc;
    float sL;
    ExitPtrs W;
    float *rho_out, *reach_out, *w_out, *cov_out;
};

// 2^e for an integer-valued e <= 0 (chunk offsets are integers): exact.
__device__ __forceinline__ double pow2_int(float e) {
    return __builtin_ldexp(1.0, (int)fmaxf(e, -2000.f));
}

// The reach of request r, by one workgroup of NTH threads; NB =
// reach_batches(B, NTH) batches of rows, a template parameter so that every
// load of the pipeline is unconditional.
template <int NB, int NTH>
__device__ __forceinline__ void reach_wg(const ReachArgs &A, const int r) {
    constexpr int REACH_WAVES = NTH / 64;
    const int32_t *__restrict__ parents = A.parents;
    const int32_t *__restrict__ tokens = A.tokens;
    const int B = A.B, V = A.V, nc = A.nc;
    const ExitPtrs &W = A.W;
    float *__restrict__ rho_out = A.rho_out;
    float *__restrict__ reach_out = A.reach_out;
    float *__restrict__ w_out = A.w_out;
    float *__restrict__ cov_out = A.cov_out;
    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63;
    __shared__ int s_anc[TEV_MAX_NODES];
    __shared__ float s_M[TEV_MAX_NODES];
    __shared__ double s_Z[TEV_MAX_NODES];
    __shared__ double s_rho[TEV_MAX_NODES];
    __shared__ double s_prod[TEV_MAX_NODES];
    __shared__ unsigned s_flags;
    const size_t rb0 = (size_t)r * B;
    const bool fast = nc <= FAST_NC;

    // Issue order: the tree arrays and every node's own term (recorded by
    // the vocabulary pass), then this wave's first batch of chunk partials; no
    // global store is issued before the last load.
    // Every load below is unconditional (out-of-range lanes read a clamped,
    // valid address and discard the value): conditional loads would make the
    // compiler wait for all outstanding loads where the branches join.
    const bool mine = tid < B;
    const int ti = min(tid, B - 1);
    const int pa = parents[rb0 + ti];
    const int tk = tokens[rb0 + ti];
    const float2 ct = W.cterm[rb0 + ti];
    // Row pass layout: each 16-lane DPP row of a wave takes one tree row per
    // pass, lane sl holding the row's chunks 4 sl .. 4 sl + 3 (nc <= 64), so a
    // wave combines four rows at once with in-row DPP steps only.
    const int sl = lane & 15;
    const int rrow = wave * ROW_BATCH + (lane >> 4);   // row of this lane within a pass
    float pm[2][SEG_CHUNKS];
    unsigned pf[2][SEG_CHUNKS];
    double pr[2][SEG_CHUNKS], pcs[2][SEG_CHUNKS];
    // Loads the partials of pass BT (row BT * ROW_BATCH * REACH_WAVES + rrow) into buffer BUF.
#define TEV_REACH_LOAD(BUF, BT)                                                                 \
    {                                                                                           \
        const int v = (BT) * ROW_BATCH * REACH_WAVES + rrow;                                    \
        _Pragma("unroll") for (int j = 0; j < SEG_CHUNKS; j++) {                                \
            const int c = SEG_CHUNKS * sl + j;                                                  \
            const bool ok = v < B && c < nc;   /* masked where used; unused when !fast */       \
            const size_t o = (rb0 + (ok ? v : 0)) * nc + (ok ? c : 0);                          \
            pm[BUF][j] = W.part_m[o];                                                           \
            pf[BUF][j] = W.flags[o];                                                            \
            pr[BUF][j] = W.part_r[o];                                                           \
            pcs[BUF][j] = W.part_c[o];                                                          \
        }                                                                                       \
    }
    TEV_REACH_LOAD(0, 0)
    // branch-free, so that no load is sunk into a branch that then waits on it
    const bool bad_node = (pa < 0) | (pa >= tid) | (tk < 0) | (tk >= V);
    const bool bad = mine & ((tid == 0) ? (pa != -1) : bad_node);
    const bool child = mine && tid > 0 && !bad;
    if (tid == 0) s_flags = 0u;
    __syncthreads();
    if (mine) s_anc[tid] = child ? pa : 0;
    if (bad) atomicOr(&s_flags, TEV_FLAG_TREE);

    // ---- row pass: per row the fp64 combine of its chunk partials ----
    // chunk offsets are integers, so rescaling a partial to the row offset M
    // is an exact power of two.
    auto finish_row = [&](int v, float M, unsigned f, double carry, double csum) {
        const double Z = carry + csum;
        if (!(M > -kInf) || !(Z > 0.0) || isnan(Z)) f |= TEV_FLAG_NONFINITE;
        s_M[v] = M;
        s_Z[v] = Z;
        s_rho[v] = carry / Z;
        W.row_m[rb0 + v] = M;
        if (f) atomicOr(&s_flags, f);
    };
    if (fast) {
        // Per row: the offset M (row maximum of the chunk offsets), the flags,
        // the running residual sums in chunk order (a serial prefix over the
        // lane's four chunks, then a scan over the row's lanes) and the
        // child-sum total; lane 15 of the row holds the residual total.
#define TEV_REACH_ROWS(BUF, BT)                                                                 \
    {                                                                                           \
        const int v = (BT) * ROW_BATCH * REACH_WAVES + rrow;                                    \
        float mloc = -kInf;                                                                     \
        unsigned floc = 0u;                                                                     \
        _Pragma("unroll") for (int j = 0; j < SEG_CHUNKS; j++) {                                \
            const bool ok = SEG_CHUNKS * sl + j < nc;                                           \
            mloc = fmaxf(mloc, ok ? pm[BUF][j] : -kInf);                                        \
            floc |= ok ? pf[BUF][j] : 0u;                                                       \
        }                                                                                       \
        const float M = row16_max_f32(mloc);                                                    \
        const unsigned f = row16_or_u32(floc);                                                  \
        double pre[SEG_CHUNKS], cs = 0.0, run = 0.0;                                            \
        _Pragma("unroll") for (int j = 0; j < SEG_CHUNKS; j++) {                                \
            const bool ok = SEG_CHUNKS * sl + j < nc;                                           \
            const float mc = ok ? pm[BUF][j] : -kInf;                                           \
            const double sc = (mc > -kInf) ? pow2_int(mc - M) : 0.0;                            \
            run += ok ? pr[BUF][j] * sc : 0.0;                                                  \
            pre[j] = run;                                                                       \
            cs += ok ? pcs[BUF][j] * sc : 0.0;                                                  \
        }                                                                                       \
        const double incl = row16_incl_scan_f64(run);                                           \
        const double excl = wave::shr_d<1>(incl);                                               \
        const double csum = row16_sum_f64(cs);                                                  \
        if (v < B) {                                                                            \
            _Pragma("unroll") for (int j = 0; j < SEG_CHUNKS; j++) {                            \
                const int c = SEG_CHUNKS * sl + j;                                              \
                if (c < nc) W.rcum[(rb0 + v) * nc + c] = excl + pre[j];                         \
            }                                                                                   \
            if (sl == 15) finish_row(v, M, f, incl, csum);                                      \
        }                                                                                       \
    }
        // pass bt + 1 is issued before pass bt's stores
#pragma unroll
        for (int bt = 0; bt < NB; bt++) {
            if (bt + 1 < NB) TEV_REACH_LOAD((bt + 1) & 1, bt + 1)
            TEV_REACH_ROWS(bt & 1, bt)
        }
#undef TEV_REACH_ROWS
    } else {
        for (int v = wave; v < B; v += REACH_WAVES) {
            const size_t base = (rb0 + v) * nc;
            float M = -kInf;
            unsigned f = 0u;
            for (int cc = lane; cc < nc; cc += 64) {
                M = fmaxf(M, W.part_m[base + cc]);
                f |= W.flags[base + cc];
            }
            M = wave::max_f32(M);
            f = wave::or_u32(f);
            double carry = 0.0, csum = 0.0;
            for (int b0 = 0; b0 < nc; b0 += 64) {
                const int cc = b0 + lane;
                double rs = 0.0;
                if (cc < nc) {
                    const float mc = W.part_m[base + cc];
                    const double sc = (mc > -kInf) ? pow2_int(mc - M) : 0.0;
                    rs = W.part_r[base + cc] * sc;
                    csum += W.part_c[base + cc] * sc;
                }
                const double incl = wave::incl_scan_f64(rs, lane);
                if (cc < nc) W.rcum[base + cc] = carry + incl;
                carry += wave::last_lane_d(incl);
            }
            csum = wave::sum_f64(csum);
            if (lane == 0) finish_row(v, M, f, carry, csum);
        }
    }
#undef TEV_REACH_LOAD
    __syncthreads();

    // Child probability of every node under its parent's distribution (fp64,
    // the node's term moved to the row offset by an exact power of two), kept
    // as the node's initial path product.
    const unsigned fl = s_flags;
    if (fl == 0u && mine) {
        double pc = 1.0;   // root: P(0) = 1
        if (tid > 0) pc = (double)ct.x * pow2_int(ct.y - s_M[pa]) / s_Z[pa];
        s_prod[tid] = pc;
    }
    __syncthreads();

    // ---- tree pass (wave 0): lane owns nodes NPL*lane .. NPL*lane + NPL - 1 ----
    // (the other waves return at once; a caller that runs more work in this
    // workgroup synchronises after it)
    auto tree_pass = [&]() {
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
    // Reach P(u) = product of child probabilities along u's root path (Eq. 4,
    // evaluated level by level in Algorithm 1).  Here by pointer jumping:
    // node u keeps (a, q) with P(u) = P(a) q; each round replaces (a, q) by
    // (a's a, q times a's q), so a path of depth d is done after
    // ceil(log2 d) rounds (a = 0 ends it, P(0) = 1).
    int a[NPL];
    double q[NPL];
#pragma unroll
    for (int k = 0; k < NPL; k++) {
        const int u = lane * NPL + k;
        a[k] = (u > 0 && u < B) ? s_anc[u] : 0;
        q[k] = (u < B) ? s_prod[u] : 0.0;
    }
    bool open = false;
#pragma unroll
    for (int k = 0; k < NPL; k++) open |= a[k] != 0;
    while (__any(open)) {
        int na[NPL];
        double nq[NPL];
#pragma unroll
        for (int k = 0; k < NPL; k++) {
            na[k] = 0;
            nq[k] = q[k];
            if (a[k] != 0) {
                na[k] = s_anc[a[k]];
                nq[k] = q[k] * s_prod[a[k]];
            }
        }
        wave::lds_sync();   // every read of this round precedes every write
        open = false;
#pragma unroll
        for (int k = 0; k < NPL; k++) {
            const int u = lane * NPL + k;
            if (a[k] != 0) {
                s_anc[u] = na[k];
                s_prod[u] = nq[k];
            }
            a[k] = na[k];
            q[k] = nq[k];
            open |= a[k] != 0;
        }
        wave::lds_sync();
    }
    double w[NPL];
    double lane_c = 0.0, lane_w = 0.0;
#pragma unroll
    for (int k = 0; k < NPL; k++) {
        const int u = lane * NPL + k;
        w[k] = 0.0;
        if (u < B) {
            w[k] = q[k] * s_rho[u];
            if (u > 0) lane_c += q[k];
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
            reach_out[rb0 + u] = (float)q[k];
            w_out[rb0 + u] = (float)w[k];
        }
    }
    if (lane == 0) {
        cov_out[r] = (float)C;
        W.status[r] = 0u;
    }
    };
    if (wave == 0) tree_pass();
}

// ----------------------------------------------------------------------------
// In-chunk residual terms on a contiguous segment: lane t owns tokens
// [64t, 64t + 64) of the chunk, so a wave scan runs in token order.  Each term
// is computed exactly as in the chunk pass (same f32 operations and offset);
// child tokens are zero (bit j of the lane's mask word).
// ----------------------------------------------------------------------------
// The in-chunk element (i, j) of lane `lane` for the vocabulary pass's
// interleaved ownership: elements k*(64*VW) + lane*VW + j, k < EPT/VW.  Every
// load is unconditional: out-of-range elements read a clamped, valid address
// and become -inf afterwards (a conditional load would make the compiler wait
// for each load before issuing the next).
template <typename T, bool VEC>
__device__ __forceinline__ void load_chunk(const T *chunk, int len, int lane, float *x) {
    constexpr int VW = 16 / (int)sizeof(T);
    constexpr int SPAN = 64 * VW;
#pragma unroll
    for (int k = 0; k < EPT / VW; k++) {
        const int idx = k * SPAN + lane * VW;
        if (VEC) {
            // len is a multiple of VW here (16-byte rows), so len - VW is a valid vector
            load16(chunk + min(idx, len - VW), &x[k * VW]);
#pragma unroll
            for (int j = 0; j < VW; j++) x[k * VW + j] = (idx < len) ? x[k * VW + j] : -kInf;
        } else {
#pragma unroll
            for (int j = 0; j < VW; j++) {
                const float t = to_f32<T>(chunk[min(idx + j, len - 1)]);
                x[k * VW + j] = (idx + j < len) ? t : -kInf;
            }
        }
    }
}

// A partial half (1 <= len < N * ... tokens) with the interleaved ownership of
// the vocabulary pass: N elements per lane, element k*(64*VW) + lane*VW + j;
// out-of-range elements become -inf.  Loads are unconditional, of clamped
// valid addresses (len >= VW when VEC: 16-byte rows).
template <typename T, bool VEC, int N>
__device__ __forceinline__ void load_chunk_part(const T *chunk, int len, int lane, float *x) {
    constexpr int VW = 16 / (int)sizeof(T);
    constexpr int SPAN = 64 * VW;
#pragma unroll
    for (int k = 0; k < N / VW; k++) {
        const int idx = k * SPAN + lane * VW;
        if (VEC) {
            load16(chunk + min(idx, len - VW), &x[k * VW]);
#pragma unroll
            for (int j = 0; j < VW; j++) x[k * VW + j] = (idx < len) ? x[k * VW + j] : -kInf;
        } else {
#pragma unroll
            for (int j = 0; j < VW; j++) {
                const float t = to_f32<T>(chunk[min(idx + j, len - 1)]);
                x[k * VW + j] = (idx + j < len) ? t : -kInf;
            }
        }
    }
}

// The sampler's contiguous ownership: lane t holds elements [64t, 64t + 64).
template <typename T, bool VEC>
__device__ __forceinline__ void segment_load(const T *chunk, int len, int lane, float *x) {
    constexpr int VW = 16 / (int)sizeof(T);
    const int base = lane * EPT;
#pragma unroll
    for (int k = 0; k < EPT / VW; k++) {
        const int idx = base + k * VW;
        if (VEC) {
            load16(chunk + min(idx, len - VW), &x[k * VW]);
#pragma unroll
            for (int j = 0; j < VW; j++) x[k * VW + j] = (idx < len) ? x[k * VW + j] : -kInf;
        } else {
#pragma unroll
            for (int j = 0; j < VW; j++) {
                const float t = to_f32<T>(chunk[min(idx + j, len - 1)]);
                x[k * VW + j] = (idx + j < len) ? t : -kInf;
            }
        }
    }
}

__device__ __forceinline__ void segment_terms(const float *x, float sL, float Mc, uint64_t bits,
                                              float *e) {
    const float off = (Mc > -kInf) ? Mc : 0.f;   // a chunk of -inf logits has only zero terms
#pragma unroll
    for (int j = 0; j < EPT; j++) {
        const float t = __builtin_amdgcn_exp2f(fmaf(x[j], sL, -off));
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

// The same mask from parents/tokens already in registers: lane t holds nodes
// 1 + t + 64k.
__device__ __forceinline__ uint64_t child_bits_regs(const int (&cpar)[NPL], const int (&ctok)[NPL],
                                                    int node, int c0, int len, unsigned *s_wmask,
                                                    int lane) {
    s_wmask[2 * lane] = 0u;
    s_wmask[2 * lane + 1] = 0u;
    wave::lds_sync();
#pragma unroll
    for (int k = 0; k < NPL; k++) {
        if (cpar[k] == node) {
            const int o = ctok[k] - c0;
            if (o >= 0 && o < len) atomicOr(&s_wmask[o >> 5], 1u << (o & 31));
        }
    }
    wave::lds_sync();
    return (uint64_t)s_wmask[2 * lane] | ((uint64_t)s_wmask[2 * lane + 1] << 32);
}

// ----------------------------------------------------------------------------
// The draws: one wave per (draw, request), 256-thread workgroups.
// ----------------------------------------------------------------------------
// Arguments of the draws for one launch.
template <typename T>
struct SampleArgs {
    const T *logits;
    const int32_t *parents, *tokens;
    int B, V, nc;
    float sL;
    const unsigned *status;
    const float *part_m;
    const double *part_r;
    const float *row_m;
    const double *rcum, *wcum;
    const float *uniforms;
    int n_draws;
    int32_t *exit_node, *bonus_token;
};

// Sum of one int per thread over an NTH-thread workgroup (every thread gets
// it); red is an NTH / 64-entry LDS scratch, reused only after a barrier.
template <int NTH>
__device__ __forceinline__ int block_sum_i32(int x, int *red) {
    const int w = wave::sum_i32(x);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = w;
    __syncthreads();
    int t = 0;
#pragma unroll
    for (int i = 0; i < NTH / 64; i++) t += red[i];
    __syncthreads();
    return t;
}

// Draw n of request r by one workgroup of NTH >= 256 threads.  Loads come in
// three dependent rounds, each issued as one group of unconditional loads:
// (1) everything that does not depend on the draw, (2) the exit node's running
// residual sums, (3) the one chunk that holds the bonus token, which the first
// four waves scan together (thread t owns tokens [16 t, 16 t + 16) of it; the
// other waves only join the barriers), so the draw is the same for any NTH.
constexpr int SAMPLE_THREADS = 256;
constexpr int SPT = CHUNK / SAMPLE_THREADS;   // 16 tokens per thread

template <typename T, bool VEC, int NTH = SAMPLE_THREADS>
__device__ __forceinline__ void sample_wg(const SampleArgs<T> &A, const int n, const int r) {
    static_assert(NTH >= SAMPLE_THREADS && NTH % 64 == 0, "at least four waves");
    const T *__restrict__ logits = A.logits;
    const int32_t *__restrict__ parents = A.parents;
    const int32_t *__restrict__ tokens = A.tokens;
    const int B = A.B, V = A.V, nc = A.nc;
    const float sL = A.sL;
    const double *__restrict__ part_r = A.part_r;
    const double *__restrict__ rcum = A.rcum;
    const double *__restrict__ wcum = A.wcum;
    const int n_draws = A.n_draws;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const bool act = tid < SAMPLE_THREADS;   // scans the chunk
    __shared__ int s_red[NTH / 64];
    __shared__ double s_wsum[NTH / 64];
    __shared__ unsigned s_bits[SAMPLE_THREADS];
    const size_t kd = (size_t)r * n_draws + n;

    // ---- load round 1 ----
    const unsigned st = A.status[r];
    const double u1 = (double)A.uniforms[2 * kd];
    const double u2 = (double)A.uniforms[2 * kd + 1];
    const double *Wc = wcum + (size_t)r * B;
    const double Wtot = Wc[B - 1];
    const double wj = Wc[min(tid, B - 1)];                      // node tid (B <= 256)
    const int ui = min(1 + tid, B - 1);
    const int cpar = parents[(size_t)r * B + ui];               // node 1 + tid
    const int ctok = tokens[(size_t)r * B + ui];
    if (st != 0u) {
        if (tid == 0) { A.exit_node[kd] = -1; A.bonus_token[kd] = -1; }
        return;
    }
    // Exit node: the number of j with W_j <= u1 * S is the smallest j with u1 S < W_j.
    const double t1 = u1 * Wtot;
    int Vn = block_sum_i32<NTH>((tid < B && wj <= t1) ? 1 : 0, s_red);
    if (Vn >= B) {   // rounding left no bin: last node with positive mass
        int best = -1;
        for (int j = lane; j < B; j += 64)
            if (j == 0 ? (Wc[0] > 0.0) : (Wc[j] > Wc[j - 1])) best = max(best, j);
        Vn = max(wave::max_i32(best), 0);
    }

    // ---- load round 2: the chunk whose running residual sum first exceeds u2 * T ----
    const size_t rb = (size_t)r * B + Vn;
    const double *RC = rcum + rb * nc;
    const double t2 = u2 * RC[nc - 1];
    int ccount = 0;
    for (int c0 = 0; c0 < nc; c0 += NTH) {
        const int c = c0 + tid;
        const double rc = RC[min(c, nc - 1)];
        ccount += (c < nc && rc <= t2) ? 1 : 0;
    }
    int cc = block_sum_i32<NTH>(ccount, s_red);
    if (cc >= nc) {
        int best = -1;
        for (int c = lane; c < nc; c += 64)
            if (part_r[rb * nc + c] > 0.0) best = max(best, c);
        cc = max(wave::max_i32(best), 0);
    }

    // ---- load round 3: the chunk ----
    const int c0 = cc * CHUNK;
    const int len = min(CHUNK, V - c0);
    const T *chunk = logits + rb * (size_t)V + c0;
    float x[SPT];
    {
        constexpr int VW = 16 / (int)sizeof(T);
#pragma unroll
        for (int k = 0; k < SPT / VW; k++) {
            const int idx = tid * SPT + k * VW;
            if (VEC) {
                load16(chunk + min(idx, len - VW), &x[k * VW]);
#pragma unroll
                for (int j = 0; j < VW; j++) x[k * VW + j] = (idx < len) ? x[k * VW + j] : -kInf;
            } else {
#pragma unroll
                for (int j = 0; j < VW; j++) {
                    const float t = to_f32<T>(chunk[min(idx + j, len - 1)]);
                    x[k * VW + j] = (idx + j < len) ? t : -kInf;
                }
            }
        }
    }
    const double rc_prev = RC[max(cc - 1, 0)];   // unconditional, issued with the chunk
    const float Mv = A.row_m[rb];
    const float Mc = A.part_m[rb * nc + cc];
    const double before = (cc > 0) ? rc_prev : 0.0;
    // offsets are integers with Mc <= Mv: the rescale is an exact power of two
    const double target = __builtin_ldexp(t2 - before, (int)fminf(Mv - Mc, 2000.f));

    // child tokens of Vn inside the chunk: bit j of word t marks token 16 t + j
    if (act) s_bits[tid] = 0u;
    __syncthreads();
    {
        const int o = ctok - c0;
        if ((1 + tid < B) & (cpar == Vn) & (o >= 0) & (o < len)) atomicOr(&s_bits[o / SPT], 1u << (o % SPT));
    }
    __syncthreads();
    const unsigned bits = act ? s_bits[tid] : 0u;
    const float off = (Mc > -kInf) ? Mc : 0.f;   // a chunk of -inf logits has only zero terms
    float e[SPT];
    double seg = 0.0;
#pragma unroll
    for (int j = 0; j < SPT; j++) {
        const float t = __builtin_amdgcn_exp2f(fmaf(x[j], sL, -off));
        e[j] = ((bits >> j) & 1u) ? 0.f : t;
        seg += (double)e[j];
    }
    // running sum in token order: in-wave scan, then the totals of earlier waves
    const double incl = wave::incl_scan_f64(seg, lane);
    if (lane == 63) s_wsum[wave] = incl;
    __syncthreads();
    double carry = 0.0;
    for (int w = 0; w < wave; w++) carry += s_wsum[w];
    double run = carry + incl - seg;
    int below = 0, last_pos = -1;
#pragma unroll
    for (int j = 0; j < SPT; j++) {
        run += (double)e[j];
        below += (act && run <= target) ? 1 : 0;
        if (e[j] > 0.f) last_pos = tid * SPT + j;
    }
    below = block_sum_i32<NTH>(below, s_red);
    if (below >= len) {
        const int lp = wave::max_i32(last_pos);
        if (lane == 0) s_red[wave] = lp;
        __syncthreads();
        int m = -1;
#pragma unroll
        for (int i = 0; i < NTH / 64; i++) m = max(m, s_red[i]);
        below = max(m, 0);
    }
    if (tid == 0) {
        A.exit_node[kd] = Vn;
        A.bonus_token[kd] = c0 + below;
    }
}

inline ExitPtrs exit_ptrs(char *ws, int R, int B, int V) {
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
    p.cterm = (float2 *)(ws + L.cterm);
    return p;
}

template <typename T>
inline SampleArgs<T> sample_args(const T *logits, const int32_t *parents, const int32_t *tokens,
                                 int R, int B, int V, float sL, const char *ws,
                                 const float *uniforms, int n_draws, int32_t *exit_node,
                                 int32_t *bonus) {
    const ExitWs L = exit_ws_layout(R, B, V);
    return SampleArgs<T>{logits, parents, tokens, B, V, n_chunks(V), sL,
                         (const unsigned *)(ws + L.status), (const float *)(ws + L.part_m),
                         (const double *)(ws + L.part_r), (const float *)(ws + L.row_m),
                         (const double *)(ws + L.rcum), (const double *)(ws + L.wcum), uniforms,
                         n_draws, exit_node, bonus};
}

}  // namespace
}  // namespace tev
