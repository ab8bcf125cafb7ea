// tree_attn_dev.h -- device code of the bf16 tree-attention kernels, shared by
// the stand-alone attention launches and the fused verification round.
//
// What is computed ("CAST: Cost-Aware Speculative Trees from One-Pass Block
// Drafters", App. B Lemma 1; App. C "Packed verification"): query (r, i, h)
// attends to the P cached prefix rows and to the rows of its own root path
// (itself included) of kv head g = h / G, G = Hq / Hkv; cache row P + j holds
// tree node j.
#pragma once

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "tev_internal.h"
#include "wave_ops.h"

namespace tev {
namespace {


typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
// Plain clang vectors for 16- and 8-byte moves: unlike HIP's uint4 struct they
// stay in registers (struct copies become memcpy that the compiler keeps in
// memory).
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));


__device__ __forceinline__ float wave_sum_f(float x) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o);
    return x;
}

// Loads the request's parents into LDS and checks the tree contract
// (parents[0] = -1, 0 <= parents[i] < i).  Returns true if valid.
__device__ __forceinline__ bool load_parents(const int32_t *par, int B, int *s_par, int *s_bad) {
    if (threadIdx.x == 0) *s_bad = 0;
    for (int i = threadIdx.x; i < B; i += blockDim.x) s_par[i] = par[i];
    __syncthreads();
    for (int i = threadIdx.x; i < B; i += blockDim.x) {
        const int p = s_par[i];
        const bool ok = (i == 0) ? (p == -1) : (p >= 0 && p < i);
        if (!ok) *s_bad = 1;
    }
    __syncthreads();
    return *s_bad == 0;
}

// ----------------------------------------------------------------------------
// bf16 MFMA kernel.
// ----------------------------------------------------------------------------
constexpr int KB = 32;   // keys per block
constexpr float kLazy = 8.0f;    // slack of the softmax reference max (log2 units)

constexpr int NW = 8;            // waves per workgroup: 4 row waves x 2 key groups
constexpr int NT = NW * 64;
constexpr int RWV = 4;           // row waves per key group
constexpr int SB = 2 * KB;       // keys per stage: one block for each key group
constexpr int PD = 2;            // stages in flight per workgroup (register prefetch depth)

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

// Transposing LDS read (gfx950 ds_read_b64_tr_b16).  Within each 16-lane
// group, lane 4j + q fetches 8 bytes (four 16-bit values); lane i receives
// value (i & 3) of the fetch of lane 4j + (i >> 2) in slot j, j = 0..3.
__device__ __forceinline__ i16x4 lds_read_tr16(const uint16_t *p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(p));
}

// p = hi + lo with hi = bf16(p) and lo = bf16(p - hi): the product with bf16
// V then carries about 16 significant bits of p.
__device__ __forceinline__ void split_bf16x8(const float *p, bf16x8 &hi, bf16x8 &lo) {
#pragma unroll
    for (int e = 0; e < 8; e++) {
        const __bf16 h = (__bf16)p[e];
        hi[e] = h;
        lo[e] = (__bf16)(p[e] - (float)h);
    }
}

// Arguments of one attention launch.
struct AttnArgs {
    const uint16_t *q, *k, *v;
    const int32_t *parents;
    int B, Hq, Hkv, P;
    float c_log2;
    int row_blocks, splits, keys_per_split, n_wg;
    float *out;
    uint16_t *part_o;
    float *part_ml;
    unsigned *status;
};

// Task of workgroup b in a grid whose first ceil(n/8)*8 workgroups serve n
// tasks.  Hardware dispatches workgroup b to XCD b % 8, so task
// (b % 8) * ceil(n/8) + b / 8 puts consecutive tasks -- the row blocks that
// stream the same K/V -- on the same XCD and its L2.  Returns >= n for idle
// workgroups.
__device__ __forceinline__ int xcd_task(int b, int n) {
    const int per_xcd = (n + 7) / 8;
    return (b % 8) * per_xcd + b / 8;
}

// One workgroup of the bf16 attention, task = (row block, prefix split,
// request * kv head), row block fastest.
//
// Waves: wave w serves query rows [(w & 3) * 16 NQT, +16 NQT) of the block
// (NQT tiles of 16) over key group w >> 2, i.e. the 32-key block kg of every
// 64-key stage; two waves per SIMD hide each other's latencies, and the two
// groups' results are merged through LDS at the end.
template <int D, int NQT>
__device__ __forceinline__ void attn_mfma_wg(const AttnArgs &A, const int task) {
    const uint16_t *__restrict__ q = A.q;
    const uint16_t *__restrict__ k = A.k;
    const uint16_t *__restrict__ v = A.v;
    const int32_t *__restrict__ parents = A.parents;
    const int B = A.B, Hq = A.Hq, Hkv = A.Hkv, P = A.P;
    const float c_log2 = A.c_log2;
    const int row_blocks = A.row_blocks, splits = A.splits, keys_per_split = A.keys_per_split;
    const int n_wg = A.n_wg;
    float *__restrict__ out = A.out;
    uint16_t *__restrict__ part_o = A.part_o;
    float *__restrict__ part_ml = A.part_ml;
    unsigned *__restrict__ status = A.status;
    constexpr int DS = D / 32;          // k-steps of the score product
    constexpr int DT = D / 16;          // 16-row tiles of O^T
    constexpr int RS = D + 8;           // K and V row stride in LDS (bf16 elements)
    constexpr int WR = RWV * NQT * 16;  // query rows per workgroup
    constexpr int ITEMS = SB * D / 8;   // 16-byte chunks of a stage's K (and of its V)
    constexpr int NI = ITEMS / NT;
    static_assert(ITEMS % NT == 0, "stage chunks must divide over the threads");
    constexpr int STG = SB * RS;        // bf16 elements of one stage buffer of K (or V)
    constexpr int STAGE_BYTES = 2 * 2 * STG * 2;
    constexpr int XCH_BYTES = RWV * NQT * DT * 64 * 16;   // second group's accumulators
    constexpr int SMEM = STAGE_BYTES > XCH_BYTES ? STAGE_BYTES : XCH_BYTES;

    const int rb = task % row_blocks;
    const int sp = (task / row_blocks) % splits;
    const int rg = task / (row_blocks * splits);

    const int G = Hq / Hkv;
    const int rows_total = G * B;
    const int r = rg / Hkv, g = rg - r * Hkv;
    const int tid = threadIdx.x;
    __builtin_assume(tid < NT);
    const int lane = tid & 63, wave = tid >> 6;
    const int l16 = lane & 15, grp = lane >> 4;
    const int kg = wave >> 2, rw = wave & 3;

    // Stage buffers: K [2][SB][RS] then V [2][SB][RS], both row-major; after
    // the loop the same bytes carry the second key group's accumulators.
    __shared__ __attribute__((aligned(16))) unsigned char s_mem[SMEM];
    uint16_t *const s_k = reinterpret_cast<uint16_t *>(s_mem);
    uint16_t *const s_v = s_k + 2 * STG;
    __shared__ unsigned s_anc[TEV_MAX_NODES * 8];
    __shared__ int s_par[TEV_MAX_NODES];
    __shared__ float s_xml[RWV][NQT][64][2];
    __shared__ int s_bad;

    const bool last = (sp == splits - 1);
    const int kbeg = sp * keys_per_split;
    const int kend = last ? P + B : kbeg + keys_per_split;
    const int nkv = P + B;
    const uint16_t *kbase = k + ((size_t)r * Hkv + g) * (size_t)nkv * D;
    const uint16_t *vbase = v + ((size_t)r * Hkv + g) * (size_t)nkv * D;
    const int nstages = (kend - kbeg + SB - 1) / SB;

    // PD register stages, one named array pair per stage; chunk n of a thread
    // is (key, 8 columns) of both K and V, columns fastest (coalesced rows).
    u32x4 kreg0[NI], kreg1[NI];
    u32x4 vreg0[NI], vreg1[NI];
    auto gload = [=](u32x4 (&kr)[NI], u32x4 (&vr)[NI], int kb) __attribute__((always_inline)) {
#pragma unroll
        for (int n = 0; n < NI; n++) {
            const int item = tid + n * NT;
            const int key = item / (D / 8), d0 = (item % (D / 8)) * 8;
            const size_t off = (size_t)min(kb + key, nkv - 1) * D + d0;
            kr[n] = *reinterpret_cast<const u32x4 *>(kbase + off);
            vr[n] = *reinterpret_cast<const u32x4 *>(vbase + off);
        }
    };
    auto lstore = [=](const u32x4 (&kr)[NI], const u32x4 (&vr)[NI], uint16_t *sk, uint16_t *sv)
                      __attribute__((always_inline)) {
#pragma unroll
        for (int n = 0; n < NI; n++) {
            const int item = tid + n * NT;
            const int key = item / (D / 8), d0 = (item % (D / 8)) * 8;
            *reinterpret_cast<u32x4 *>(&sk[key * RS + d0]) = kr[n];
            *reinterpret_cast<u32x4 *>(&sv[key * RS + d0]) = vr[n];
        }
    };

    // Issue order: Q^T operands and the request's parents first, then the K/V
    // prefetch, so that waiting for the small loads never waits for the stream.
    bf16x8 qop[NQT][DS];
    int qnode[NQT], qrow[NQT];
#pragma unroll
    for (int t = 0; t < NQT; t++) {
        const int row = rb * WR + rw * NQT * 16 + t * 16 + l16;
        qrow[t] = row;
        const int rr = min(row, rows_total - 1);
        const int i = rr / G, hh = rr - i * G;
        qnode[t] = i;
        const uint16_t *qp = q + (((size_t)r * B + i) * Hq + g * G + hh) * D;
#pragma unroll
        for (int ds = 0; ds < DS; ds++)
            qop[t][ds] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4 *>(qp + ds * 32 + grp * 8));
    }
    static_assert(NT >= TEV_MAX_NODES, "one thread per tree node");
    // Unconditional load of a clamped index, stored to LDS below by every
    // workgroup (a load used only by the last split would be sunk into its
    // branch, and the compiler would wait for all outstanding loads there).
    const int par_raw = parents[(size_t)r * B + min(tid, B - 1)];
    const int my_par = tid < B ? par_raw : -1;

    // Every stage load is unconditional (a workgroup has at least one stage;
    // loads past the last stage re-read its keys): conditional loads would
    // make the compiler wait for all outstanding loads where branches join.
    static_assert(PD == 2, "the pipeline below is written out for two register stages");
    gload(kreg0, vreg0, kbeg);
    gload(kreg1, vreg1, kbeg + min(1, nstages - 1) * SB);

    // Tree contract (parents[0] = -1, 0 <= parents[i] < i) and the ancestor
    // bitmap of every node (bit j of node i: j lies on i's root path).
    bool tree_ok = true;
    if (tid < TEV_MAX_NODES) s_par[tid] = my_par;   // read by the last split only
    if (last) {
        if (tid == 0) s_bad = 0;
        __syncthreads();
        if (tid < B && !((tid == 0) ? (my_par == -1) : (my_par >= 0 && my_par < tid))) s_bad = 1;
        __syncthreads();
        tree_ok = s_bad == 0;
        if (tree_ok && tid < B) {
            unsigned a[8] = {0u, 0u, 0u, 0u, 0u, 0u, 0u, 0u};
            for (int j = tid; j >= 0; j = s_par[j]) {
#pragma unroll
                for (int w = 0; w < 8; w++) a[w] |= ((j >> 5) == w) ? (1u << (j & 31)) : 0u;
            }
#pragma unroll
            for (int w = 0; w < 8; w++) s_anc[tid * 8 + w] = a[w];
        }
        if (rb == 0 && g == 0 && tid == 0) status[r] = tree_ok ? 0u : TEV_FLAG_TREE;
    }

    f32x4 acc[NQT][DT];          // O^T, un-normalised
    float m_run[NQT], l_run[NQT];
#pragma unroll
    for (int t = 0; t < NQT; t++) {
        m_run[t] = -kInf;
        l_run[t] = 0.f;
#pragma unroll
        for (int dt = 0; dt < DT; dt++) acc[t][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    // This lane's fetch rows for the V^T operands: key 4 grp + (l16 >> 2) of
    // each half-block, columns 4 (l16 & 3) of every 16-column tile.
    const int vrow = 4 * grp + (l16 >> 2), vcol = 4 * (l16 & 3);

    // One 32-key block of this wave's key group: kb is its first key, buf the
    // LDS stage buffer that holds it.
    auto compute = [=](int kb, int buf, f32x4 (&acc)[NQT][DT], float (&m_run)[NQT], float (&l_run)[NQT])
                       __attribute__((always_inline)) {
        const bool masked = (kb + KB > P) || (kb + KB > kend);
        const uint16_t *sk = s_k + buf * STG + kg * KB * RS;
        const uint16_t *sv = s_v + buf * STG + kg * KB * RS;

        // S^T tiles of every query tile: K operands loaded one key tile at a time.
        f32x4 S[NQT][2];
#pragma unroll
        for (int t = 0; t < NQT; t++) S[t][0] = S[t][1] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kt = 0; kt < 2; kt++) {
            bf16x8 kop[DS];
#pragma unroll
            for (int ds = 0; ds < DS; ds++)
                kop[ds] = *reinterpret_cast<const bf16x8 *>(&sk[(kt * 16 + l16) * RS + ds * 32 + grp * 8]);
#pragma unroll
            for (int ds = 0; ds < DS; ds++)
#pragma unroll
                for (int t = 0; t < NQT; t++)
                    S[t][kt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kop[ds], qop[t][ds], S[t][kt], 0, 0, 0);
        }

        // Online softmax per query column; P^T operands as bf16 hi + lo.
        bf16x8 phi[NQT], plo[NQT];
#pragma unroll
        for (int t = 0; t < NQT; t++) {
            // sv[e]: key kb + grp*4 + e (e < 4) or kb + 16 + grp*4 + (e - 4)
            float s8[8] = {S[t][0][0], S[t][0][1], S[t][0][2], S[t][0][3],
                           S[t][1][0], S[t][1][1], S[t][1][2], S[t][1][3]};
            if (masked) {
                const unsigned *anc = &s_anc[qnode[t] * 8];
#pragma unroll
                for (int e = 0; e < 8; e++) {
                    const int key = kb + (e < 4 ? grp * 4 + e : 16 + grp * 4 + (e - 4));
                    const int j = key - P;                       // tree node of this key, if >= 0
                    const unsigned word = anc[(j >> 5) & 7];
                    const bool on_path = tree_ok & (j >= 0) & (((word >> (j & 31)) & 1u) != 0u);
                    const bool vis = (key < kend) & ((key < P) | on_path);
                    s8[e] = vis ? s8[e] : -kInf;
                }
            }
            float bm = s8[0];
#pragma unroll
            for (int e = 1; e < 8; e++) bm = fmaxf(bm, s8[e]);
            bm = fmaxf(bm, __shfl_xor(bm, 16));
            bm = fmaxf(bm, __shfl_xor(bm, 32));
            // The reference max moves only when the block's max exceeds it by
            // more than kLazy (log2 units): probabilities stay <= 2^kLazy and
            // the accumulators are rescaled only when it moves.
            const float bmc = bm * c_log2;
            const bool grow = bmc > m_run[t] + kLazy;
            const float m_new = grow ? bmc : m_run[t];
            const float m_use = (m_new == -kInf) ? 0.f : m_new;
            const float alpha = grow ? __builtin_amdgcn_exp2f(m_run[t] - m_use) : 1.0f;
            float pv[8];
            float ps = 0.f;
#pragma unroll
            for (int e = 0; e < 8; e++) {
                pv[e] = __builtin_amdgcn_exp2f(fmaf(s8[e], c_log2, -m_use));
                ps += pv[e];
            }
            l_run[t] = l_run[t] * alpha + ps;
            m_run[t] = m_new;
            if (__any(grow)) {
#pragma unroll
                for (int dt = 0; dt < DT; dt++) acc[t][dt] *= alpha;
            }
            split_bf16x8(pv, phi[t], plo[t]);
        }

        // O^T += V^T P^T: V^T operands by transposing reads, one d-tile at a time.
#pragma unroll
        for (int dt = 0; dt < DT; dt++) {
            const i16x4 lo4 = lds_read_tr16(sv + vrow * RS + dt * 16 + vcol);
            const i16x4 hi4 = lds_read_tr16(sv + (16 + vrow) * RS + dt * 16 + vcol);
            const bf16x8 vop = __builtin_bit_cast(bf16x8, (i16x8)__builtin_shufflevector(lo4, hi4, 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
            for (int t = 0; t < NQT; t++) {
                acc[t][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vop, phi[t], acc[t][dt], 0, 0, 0);
                acc[t][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vop, plo[t], acc[t][dt], 0, 0, 0);
            }
        }
    };

    // Stage 0 into LDS buffer 0 (the tree bitmap above is also published here).
    lstore(kreg0, vreg0, s_k, s_v);
    __syncthreads();

    // Stage s sits in register slot s % PD until it is written to LDS buffer
    // s & 1 at the end of iteration s - 1; its slot is then refilled with
    // stage s + PD at the start of iteration s.  SL is the slot of stage
    // s = s0 + SL, NX the slot of stage s + 1.
#define TEV_ATTN_STAGE(SL, NX)                                                                  \
    {                                                                                           \
        const int s = s0 + (SL);                                                                \
        if (s < nstages) {                                                                      \
            gload(kreg##SL, vreg##SL, kbeg + min(s + PD, nstages - 1) * SB);                    \
            const int kb = kbeg + s * SB + kg * KB;                                             \
            if (kb < kend) compute(kb, s & 1, acc, m_run, l_run);                               \
            if (s + 1 < nstages) {                                                              \
                const int nb = (s + 1) & 1;                                                     \
                __syncthreads(); /* all waves are done reading buffer nb */                     \
                lstore(kreg##NX, vreg##NX, s_k + nb * STG, s_v + nb * STG);                     \
                __syncthreads();                                                                \
            }                                                                                   \
        }                                                                                       \
    }
    for (int s0 = 0; s0 < nstages; s0 += PD) {
        TEV_ATTN_STAGE(0, 1)
        TEV_ATTN_STAGE(1, 0)
    }
#undef TEV_ATTN_STAGE

    // The second key group hands (m, l, acc) to the first through LDS.
    __syncthreads();   // every wave is done with the stage buffers
    f32x4 *xo = reinterpret_cast<f32x4 *>(s_mem);
    if (kg == 1) {
#pragma unroll
        for (int t = 0; t < NQT; t++) {
#pragma unroll
            for (int dt = 0; dt < DT; dt++) xo[((rw * NQT + t) * DT + dt) * 64 + lane] = acc[t][dt];
            s_xml[rw][t][lane][0] = m_run[t];
            s_xml[rw][t][lane][1] = l_run[t];
        }
    }
    __syncthreads();
    if (kg == 1) return;   // no barrier below this point
#pragma unroll
    for (int t = 0; t < NQT; t++) {
        const float m1 = s_xml[rw][t][lane][0], l1 = s_xml[rw][t][lane][1];
        const float M = fmaxf(m_run[t], m1);
        const float Mu = (M == -kInf) ? 0.f : M;
        const float a0 = __builtin_amdgcn_exp2f(m_run[t] - Mu), a1 = __builtin_amdgcn_exp2f(m1 - Mu);
#pragma unroll
        for (int dt = 0; dt < DT; dt++) acc[t][dt] = acc[t][dt] * a0 + xo[((rw * NQT + t) * DT + dt) * 64 + lane] * a1;
        l_run[t] = l_run[t] * a0 + l1 * a1;
        m_run[t] = M;
    }

    // Finalise: the four lanes of a query column hold disjoint key subsets.
    const size_t rows_all = (size_t)(n_wg / (row_blocks * splits)) * rows_total;
#pragma unroll
    for (int t = 0; t < NQT; t++) {
        float lt = l_run[t];
        lt += __shfl_xor(lt, 16);
        lt += __shfl_xor(lt, 32);
        const int row = qrow[t];
        if (row >= rows_total) continue;
        const int i = row / G, hh = row - i * G;
        if (splits == 1) {
            float *o = out + (((size_t)r * B + i) * Hq + g * G + hh) * D;
            const float inv = 1.0f / lt;
#pragma unroll
            for (int dt = 0; dt < DT; dt++) {
                f32x4 val = acc[t][dt] * inv;
                if (!tree_ok) val = f32x4{__builtin_nanf(""), __builtin_nanf(""), __builtin_nanf(""), __builtin_nanf("")};
                *reinterpret_cast<f32x4 *>(o + dt * 16 + grp * 4) = val;
            }
        } else {
            // The split's normalised output o / l in fp16, in units of 2^u
            // chosen from the row's largest |o / l| (scaled values below 2^15,
            // the largest above 2^14): half the bytes of fp32 partials, about
            // 2^-12 relative to the row's largest value.
            const float inv = 1.0f / lt;
            float mx = 0.f;
#pragma unroll
            for (int dt = 0; dt < DT; dt++)
#pragma unroll
                for (int j = 0; j < 4; j++) mx = fmaxf(mx, fabsf(acc[t][dt][j]));
            mx = fmaxf(mx, __shfl_xor(mx, 16));
            mx = fmaxf(mx, __shfl_xor(mx, 32));
            mx *= inv;
            int ex = 0;
            (void)frexpf(mx, &ex);                          // mx = f 2^ex, f in [0.5, 1)
            const int u = (mx > 0.f) ? min(max(ex - 15, -126), 127) : 0;
            const float sc = inv * __builtin_ldexpf(1.0f, -u);
            const size_t prow = (size_t)sp * rows_all + (size_t)rg * rows_total + row;
            uint16_t *o16 = part_o + prow * D;
#pragma unroll
            for (int dt = 0; dt < DT; dt++) {
                const f32x4 val = acc[t][dt] * sc;
                f16x4 h;
#pragma unroll
                for (int j = 0; j < 4; j++) h[j] = (_Float16)val[j];
                *reinterpret_cast<f16x4 *>(o16 + dt * 16 + grp * 4) = h;
            }
            if (grp == 0)
                *reinterpret_cast<f32x4 *>(part_ml + prow * 4) = f32x4{m_run[t], lt, (float)u, 0.f};
        }
    }
}

constexpr int MAX_SPLITS = 32;

// Merge split partials: one wave per query row (block b of 256 threads takes
// rows 4b .. 4b + 3); lane s reads split s's (m, l, u), every lane its D/64
// output columns of all splits.  All loads are unconditional (clamped split
// index), so they are all in flight before the first use.
template <int D>
__device__ __forceinline__ void attn_combine_wg(const uint16_t *__restrict__ part_o,
                                                const float *__restrict__ part_ml, int splits,
                                                int Hkv, int G, int B, int Hq, size_t rows_all,
                                                const unsigned *__restrict__ status,
                                                float *__restrict__ out, const int block) {
    constexpr int DPL = D / 64;
    static_assert(DPL == 1 || DPL == 2, "head_dim 64 or 128");
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const size_t row = (size_t)block * 4 + wave;
    if (row >= rows_all) return;
    const int rows_total = G * B;
    const int rg = (int)(row / rows_total);
    const int rr = (int)(row - (size_t)rg * rows_total);
    const int r = rg / Hkv, g = rg - r * Hkv;
    const int i = rr / G, hh = rr - i * G;
    const f32x4 ml = *reinterpret_cast<const f32x4 *>(part_ml + ((size_t)min(lane, splits - 1) * rows_all + row) * 4);
    uint32_t o[MAX_SPLITS];   // DPL fp16 values of split s (one or two halves)
#pragma unroll
    for (int s = 0; s < MAX_SPLITS; s++) {
        const uint16_t *p = part_o + ((size_t)min(s, splits - 1) * rows_all + row) * D + lane * DPL;
        o[s] = DPL == 2 ? *reinterpret_cast<const uint32_t *>(p) : (uint32_t)*p;
    }
    const bool mine = lane < splits;
    const float ms = mine ? ml[0] : -kInf, ls = mine ? ml[1] : 0.f;
    const float M = wave::max_f32(ms);
    const float wgt = (ms > -kInf) ? __builtin_amdgcn_exp2f(ms - M) : 0.f;
    const float L = wave::sum_f32(ls * wgt);
    const float f = (wgt * ls) * __builtin_ldexpf(1.0f, mine ? (int)ml[2] : 0);   // weight of split s's unit
    float acc[DPL];
#pragma unroll
    for (int j = 0; j < DPL; j++) acc[j] = 0.f;
#pragma unroll
    for (int s = 0; s < MAX_SPLITS; s++) {
        if (s < splits) {
            const float fs = wave::readlane_f(f, s);
#pragma unroll
            for (int j = 0; j < DPL; j++) {
                const _Float16 h = __builtin_bit_cast(_Float16, (uint16_t)(o[s] >> (16 * j)));
                acc[j] = fmaf(fs, (float)h, acc[j]);
            }
        }
    }
    const bool bad = status[r] != 0u;
    float *dst = out + (((size_t)r * B + i) * Hq + g * G + hh) * D + lane * DPL;
#pragma unroll
    for (int j = 0; j < DPL; j++) dst[j] = bad ? __builtin_nanf("") : acc[j] / L;
}

}  // namespace
}  // namespace tev
