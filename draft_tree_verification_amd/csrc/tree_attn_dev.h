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
constexpr int KS = 64;           // keys per stage
constexpr int KT = KS / 16;      // 16-key score tiles per stage
constexpr int KSTEP = KS / 32;   // 32-key steps of the PV product per stage
constexpr float kLazy = 8.0f;    // slack of the softmax reference max (log2 units)

constexpr int NW = 8;            // waves per workgroup, each owning 16 NQT query rows
constexpr int NT = NW * 64;
constexpr int PD = 2;            // stages in flight per workgroup (register prefetch depth)
constexpr int VS_MIN = -100;     // initial (smallest) exponent of the V scale

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

// Transposing LDS read (gfx950 ds_read_b64_tr_b16).  Within each 16-lane
// group, lane 4j + q fetches 8 bytes (four 16-bit values); lane i receives
// value (i & 3) of the fetch of lane 4j + (i >> 2) in slot j, j = 0..3.
__device__ __forceinline__ i16x4 lds_read_tr16(const uint16_t *p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(p));
}

// Two bf16 values (one 32-bit word) -> two fp16 values scaled by 2^-vs, as
// integer operations on the bit fields: the 8-bit exponent is rebiased to 5
// bits by subtracting bias = (127 - 15 + vs) << 7 with unsigned saturation and
// the 7-bit mantissa is widened to 10 bits.  Exact for every magnitude whose
// scaled value lies in [2^-14, 2^16); smaller ones become zero or a value
// below 2^-14 (the caller keeps the largest scaled magnitude in [2^14, 2^15),
// so this is an absolute error below 2^-28 of it).  Inputs must be finite.
__device__ __forceinline__ uint32_t bf16x2_to_f16x2(uint32_t w, u16x2 bias) {
    u16x2 d = __builtin_elementwise_sub_sat(__builtin_bit_cast(u16x2, w & 0x7fff7fffu), bias);
    d = d << (u16x2){3, 3};
    return __builtin_bit_cast(uint32_t, d) | (w & 0x80008000u);
}

// Largest |bf16| bit pattern (sign cleared) of the two halves of w and m.
__device__ __forceinline__ u16x2 absmax_bits(u16x2 m, uint32_t w) {
    return __builtin_elementwise_max(m, __builtin_bit_cast(u16x2, w & 0x7fff7fffu));
}

// max over the four 16-lane groups of a wave (lanes l, l ^ 16, l ^ 32, l ^ 48)
// with the gfx950 row-swap permutes (no LDS traffic).
__device__ __forceinline__ float max_over_groups(float x) {
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = __builtin_elementwise_maximum(__uint_as_float(a[0]), __uint_as_float(a[1]));
    const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __builtin_elementwise_maximum(__uint_as_float(b[0]), __uint_as_float(b[1]));
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

// Workgroup barrier that orders LDS traffic only (release and acquire of the
// local address space), so that global loads issued before it stay in flight.
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// 3-input maximum (v_maximum3_f32: no canonicalisation of MFMA results).
__device__ __forceinline__ float vmax3(float a, float b, float c) {
    return __builtin_elementwise_maximum(__builtin_elementwise_maximum(a, b), c);
}

// One workgroup of the bf16 attention, task = (row block, prefix split,
// request * kv head), row block fastest.
//
// Wave w serves query rows [w * 16 NQT, (w + 1) * 16 NQT) of the block over
// every 64-key stage of the split.  Per stage and wave:
//   S^T (64 keys x 16 queries per tile) = K Q^T        bf16 MFMA 16x16x32
//   online softmax per query column (lazy reference max), P^T in fp16,
//   O^T (D x 16) += V^T P^T                            fp16 MFMA 16x16x32
//   l (16 x 16, all rows equal) += 1 P^T               same MFMA, A = ones
// so the softmax denominator sums exactly the fp16 probabilities the numerator
// uses.  K and V stages are double buffered in LDS; two more stages are in
// flight in registers.
//
// V enters fp16 scaled by a per-workgroup power of two 2^-vs: every wave
// publishes the largest |V| bit pattern of its share of a stage one iteration
// before the stage is written, and vs grows (never shrinks) whenever that value
// would reach 2^15; the accumulators follow with an exact rescale.  One barrier
// per stage, which waits for LDS traffic only: the global loads of the next
// stages stay in flight across it.
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
    constexpr int RSK = D + 16;         // K row stride in LDS (32 bytes past a bank period)
    constexpr int RSV = D + 16;         // V row stride (the same: conflict-free transposing reads)
    constexpr int WR = NW * NQT * 16;   // query rows per workgroup
    constexpr int CPR = D / 8;          // 16-byte chunks per key row
    constexpr int ITEMS = KS * CPR;     // chunks of a stage's K (and of its V)
    constexpr int NI = ITEMS / NT;
    static_assert(ITEMS % NT == 0, "stage chunks must divide over the threads");
    constexpr int STK = KS * RSK;       // elements of one K stage buffer
    constexpr int STV = KS * RSV;       // elements of one V stage buffer

    const int rb = task % row_blocks;
    const int sp = (task / row_blocks) % splits;
    const int rg = task / (row_blocks * splits);

    const int G = Hq / Hkv;
    const int rows_total = G * B;
    const int r = rg / Hkv, g = rg - r * Hkv;
    const int tid = threadIdx.x;
    __builtin_assume(tid < NT);
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int l16 = lane & 15, grp = lane >> 4;

    __shared__ __attribute__((aligned(16))) uint16_t s_k[2 * STK];
    __shared__ __attribute__((aligned(16))) uint16_t s_v[2 * STV];
    __shared__ unsigned s_anc[TEV_MAX_NODES * 8];
    __shared__ int s_par[TEV_MAX_NODES];
    __shared__ __attribute__((aligned(16))) unsigned s_vmax[2][NW];
    __shared__ int s_bad;

    const bool last = (sp == splits - 1);
    const int kbeg = sp * keys_per_split;
    const int kend = last ? P + B : kbeg + keys_per_split;
    const int nkv = P + B;
    const uint16_t *kbase = k + ((size_t)r * Hkv + g) * (size_t)nkv * D;
    const uint16_t *vbase = v + ((size_t)r * Hkv + g) * (size_t)nkv * D;
    const int nstages = (kend - kbeg + KS - 1) / KS;

    // PD register stages, one named array pair per stage; chunk n of a thread
    // is (key, 8 columns) of both K and V, columns fastest (coalesced rows).
    // Buffer loads against the head's K / V extent: rows past P + B read as
    // zero (masked out below), so the per-thread offsets never change and no
    // load is conditional.  Loads past the last stage re-read it.
    const __amdgpu_buffer_rsrc_t krsrc = __builtin_amdgcn_make_buffer_rsrc(
        (void *)kbase, (short)0, nkv * D * 2, 0x00020000);
    const __amdgpu_buffer_rsrc_t vrsrc = __builtin_amdgcn_make_buffer_rsrc(
        (void *)vbase, (short)0, nkv * D * 2, 0x00020000);
    u32x4 kreg0[NI], kreg1[NI];
    u32x4 vreg0[NI], vreg1[NI];
    auto gload = [=](u32x4 (&kr)[NI], u32x4 (&vr)[NI], int s) __attribute__((always_inline)) {
        const int soff = (kbeg + min(s, nstages - 1) * KS) * D * 2;
#pragma unroll
        for (int n = 0; n < NI; n++) {
            const int voff = (tid + n * NT) * 16;   // (key, 8 columns) chunk, bytes
            kr[n] = __builtin_amdgcn_raw_buffer_load_b128(krsrc, voff, soff, 0);
            vr[n] = __builtin_amdgcn_raw_buffer_load_b128(vrsrc, voff, soff, 0);
        }
    };
    // This wave's largest |V| bit pattern of a register stage, into slot set ss.
    auto publish_vmax = [=](const u32x4 (&vr)[NI], int ss) __attribute__((always_inline)) {
        u16x2 m = {0, 0};
#pragma unroll
        for (int n = 0; n < NI; n++)
#pragma unroll
            for (int j = 0; j < 4; j++) m = absmax_bits(m, vr[n][j]);
        const int mx = wave::max_i32((int)max((unsigned)m[0], (unsigned)m[1]));
        if (lane == 0) s_vmax[ss][wave] = (unsigned)mx;
    };
    // After a barrier: the workgroup's largest |V| exponent of a stage.
    auto stage_vexp = [=](int ss) __attribute__((always_inline)) {
        unsigned mx = 0u;
#pragma unroll
        for (int w4 = 0; w4 < NW; w4 += 4) {
            const u32x4 a = *reinterpret_cast<const u32x4 *>(&s_vmax[ss][w4]);
            mx = max(mx, max(max(a[0], a[1]), max(a[2], a[3])));
        }
        return (int)(mx >> 7) - 127;   // unbiased exponent of the largest |V| (-127: zero)
    };
    auto lstore = [=](const u32x4 (&kr)[NI], const u32x4 (&vr)[NI], uint16_t *sk, uint16_t *sv, int vsc)
                      __attribute__((always_inline)) {
        const unsigned short bb = (unsigned short)((112 + vsc) << 7);
        const u16x2 bias = {bb, bb};
#pragma unroll
        for (int n = 0; n < NI; n++) {
            const int item = tid + n * NT;
            const int key = item / CPR, d0 = (item % CPR) * 8;
            *reinterpret_cast<u32x4 *>(&sk[key * RSK + d0]) = kr[n];
            u32x4 hv;
#pragma unroll
            for (int j = 0; j < 4; j++) hv[j] = bf16x2_to_f16x2(vr[n][j], bias);
            *reinterpret_cast<u32x4 *>(&sv[key * RSV + d0]) = hv;
        }
    };

    // Issue order: Q^T operands and the request's parents first, then the K/V
    // prefetch, so that waiting for the small loads never waits for the stream.
    const int wrow0 = rb * WR + (wave & 3) * NQT * 16 + (wave >> 2) * 4 * NQT * 16;
    bf16x8 qop[NQT][DS];
    int qnode[NQT], qrow[NQT];
#pragma unroll
    for (int t = 0; t < NQT; t++) {
        const int row = wrow0 + t * 16 + l16;
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
    static_assert(NW % 4 == 0 && KS % 32 == 0, "four-wave groups, 32-key steps");
    // Unconditional load of a clamped index, stored to LDS below by every
    // workgroup (a load used only by the last split would be sunk into its
    // branch, and the compiler would wait for all outstanding loads there).
    const int par_raw = parents[(size_t)r * B + min(tid, B - 1)];
    const int my_par = tid < B ? par_raw : -1;

    static_assert(PD == 2, "the pipeline below is written out for two register stages");
    gload(kreg0, vreg0, 0);
    gload(kreg1, vreg1, 1);

    // Tree contract (parents[0] = -1, 0 <= parents[i] < i) and the ancestor
    // bitmap of every node (bit j of node i: j lies on i's root path).
    bool tree_ok = true;
    if (tid < TEV_MAX_NODES) s_par[tid] = my_par;   // read by the last split only
    if (last) {
        if (tid == 0) s_bad = 0;
        lds_barrier();
        if (tid < B && !((tid == 0) ? (my_par == -1) : (my_par >= 0 && my_par < tid))) s_bad = 1;
        lds_barrier();
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

    f32x4 acc[NQT][DT];          // O^T in units of 2^vs_acc, un-normalised
    f32x4 accl[NQT];             // softmax denominators (every entry the column's sum)
    float m_run[NQT];
#pragma unroll
    for (int t = 0; t < NQT; t++) {
        m_run[t] = -kInf;
        accl[t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int dt = 0; dt < DT; dt++) acc[t][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    // vs: the scale of the latest stage written to LDS; vs_acc: the units of
    // this wave's accumulators.
    int vs = VS_MIN, vs_acc = VS_MIN;
    // Stage t is written to LDS with the current vs, grown to cover its largest |V|.
    auto store_stage = [&](const u32x4 (&kr)[NI], const u32x4 (&vr)[NI], int t) __attribute__((always_inline)) {
        vs = max(vs, min(max(stage_vexp(t & 1) - 14, VS_MIN), 120));
        lstore(kr, vr, s_k + (t & 1) * STK, s_v + (t & 1) * STV, vs);
    };
    // This lane's fetch rows for the V^T operands: key 4 grp + (l16 >> 2) of
    // each 16-key half, columns 4 (l16 & 3) of every 16-column tile.
    const int vrow = 4 * grp + (l16 >> 2), vcol = 4 * (l16 & 3);
    f16x8 ones;
#pragma unroll
    for (int e = 0; e < 8; e++) ones[e] = (_Float16)1.0f;

    // QK of the stage in K buffer kbuf.
    auto qk = [&](f32x4 (&S)[NQT][KT], int kbuf) __attribute__((always_inline)) {
        const uint16_t *sk = s_k + kbuf * STK;
#pragma unroll
        for (int t = 0; t < NQT; t++)
#pragma unroll
            for (int kt = 0; kt < KT; kt++) S[t][kt] = f32x4{0.f, 0.f, 0.f, 0.f};
        // d-step outermost: the NQT x KT accumulators form independent chains,
        // so consecutive MFMAs never wait for each other's results.
#pragma unroll
        for (int ds = 0; ds < DS; ds++) {
            bf16x8 kop[KT];
#pragma unroll
            for (int kt = 0; kt < KT; kt++)
                kop[kt] = *reinterpret_cast<const bf16x8 *>(&sk[(kt * 16 + l16) * RSK + ds * 32 + grp * 8]);
#pragma unroll
            for (int kt = 0; kt < KT; kt++)
#pragma unroll
                for (int t = 0; t < NQT; t++)
                    S[t][kt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kop[kt], qop[t][ds], S[t][kt], 0, 0, 0);
        }
    };

    // Softmax and PV of stage t (first key kb, scores S) against its V buffer,
    // whose values are in units of 2^vst.
    auto spv = [&](f32x4 (&S)[NQT][KT], int t_stage, int vst) __attribute__((always_inline)) {
        const int kb = kbeg + t_stage * KS;
        const bool tree_keys = kb + KS > P;                  // stage holds tree rows
        const bool past_end = kb + KS > kend;                // stage runs past the split
        const uint16_t *sv = s_v + (t_stage & 1) * STV;
        // accumulators into the units of this stage's V
        if (vst > vs_acc) {
            const float f = __builtin_ldexpf(1.0f, vs_acc - vst);
#pragma unroll
            for (int t = 0; t < NQT; t++)
#pragma unroll
                for (int dt = 0; dt < DT; dt++) acc[t][dt] *= f;
            vs_acc = vst;
        }
        // S[t][kt][i] is key kb + 16 kt + 4 grp + i; one branch for every tile
        // (the key arithmetic stays inside it).  A prefix stage that runs
        // past its split only needs the range test.
        if (!tree_keys && past_end) {
#pragma unroll
            for (int kt = 0; kt < KT; kt++)
#pragma unroll
                for (int i = 0; i < 4; i++) {
                    const bool in_range = kb + 16 * kt + 4 * grp + i < kend;
#pragma unroll
                    for (int t = 0; t < NQT; t++) S[t][kt][i] = in_range ? S[t][kt][i] : -kInf;
                }
        } else if (tree_keys) {
#pragma unroll
            for (int kt = 0; kt < KT; kt++)
#pragma unroll
                for (int i = 0; i < 4; i++) {
                    const int key = kb + 16 * kt + 4 * grp + i;
                    const int j = key - P;                       // tree node of this key, if >= 0
                    const bool in_range = key < kend;
#pragma unroll
                    for (int t = 0; t < NQT; t++) {
                        const unsigned word = s_anc[qnode[t] * 8 + ((j >> 5) & 7)];
                        const bool on_path = tree_ok & (j >= 0) & (((word >> (j & 31)) & 1u) != 0u);
                        const bool vis = in_range & ((key < P) | on_path);
                        S[t][kt][i] = vis ? S[t][kt][i] : -kInf;
                    }
                }
        }
        f16x8 pop[NQT][KSTEP];
#pragma unroll
        for (int t = 0; t < NQT; t++) {
            float bm = vmax3(S[t][0][0], S[t][0][1], S[t][0][2]);
            bm = vmax3(bm, S[t][0][3], S[t][1][0]);
            bm = vmax3(bm, S[t][1][1], S[t][1][2]);
            bm = __builtin_elementwise_maximum(bm, S[t][1][3]);
#pragma unroll
            for (int kt = 2; kt < KT; kt++) {
                bm = vmax3(bm, S[t][kt][0], S[t][kt][1]);
                bm = vmax3(bm, S[t][kt][2], S[t][kt][3]);
            }
            bm = max_over_groups(bm);
            // The reference max moves only when the stage's max exceeds it by
            // more than kLazy (log2 units): probabilities stay <= 2^kLazy and
            // the accumulators are rescaled only when it moves.
            const float bmc = bm * c_log2;
            const bool grow = bmc > m_run[t] + kLazy;
            const float m_new = grow ? bmc : m_run[t];
            const float m_use = (m_new == -kInf) ? 0.f : m_new;
            if (__any(grow)) {
                const float alpha = grow ? __builtin_amdgcn_exp2f(m_run[t] - m_use) : 1.0f;
#pragma unroll
                for (int dt = 0; dt < DT; dt++) acc[t][dt] *= alpha;
                accl[t] *= alpha;
            }
            m_run[t] = m_new;
#pragma unroll
            for (int ks = 0; ks < KSTEP; ks++) {
                // k-step ks: keys kb + 32 ks + {4 grp + i, 16 + 4 grp + i}
                float pv[8];
#pragma unroll
                for (int i = 0; i < 4; i++) {
                    pv[i] = __builtin_amdgcn_exp2f(fmaf(S[t][2 * ks][i], c_log2, -m_use));
                    pv[4 + i] = __builtin_amdgcn_exp2f(fmaf(S[t][2 * ks + 1][i], c_log2, -m_use));
                }
#pragma unroll
                for (int e = 0; e < 4; e++) {
                    const auto h = __builtin_amdgcn_cvt_pkrtz(pv[2 * e], pv[2 * e + 1]);
                    pop[t][ks][2 * e] = (_Float16)h[0];
                    pop[t][ks][2 * e + 1] = (_Float16)h[1];
                }
            }
        }
        // O^T += V^T P^T and l += 1 P^T: V^T operands by transposing reads.
#pragma unroll
        for (int ks = 0; ks < KSTEP; ks++) {
            const uint16_t *svk = sv + 32 * ks * RSV;
#pragma unroll
            for (int dt = 0; dt < DT; dt++) {
                const i16x4 lo4 = lds_read_tr16(svk + vrow * RSV + dt * 16 + vcol);
                const i16x4 hi4 = lds_read_tr16(svk + (16 + vrow) * RSV + dt * 16 + vcol);
                const f16x8 vop = __builtin_bit_cast(f16x8, (i16x8)__builtin_shufflevector(lo4, hi4, 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
                for (int t = 0; t < NQT; t++)
                    acc[t][dt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vop, pop[t][ks], acc[t][dt], 0, 0, 0);
            }
#pragma unroll
            for (int t = 0; t < NQT; t++)
                accl[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ones, pop[t][ks], accl[t], 0, 0, 0);
        }
    };

    // Prologue: stage 0 into LDS (the tree bitmap above is also published by
    // the barriers here), stage 2 into register slot 0, stage 1's |V| published.
    publish_vmax(vreg0, 0);
    lds_barrier();
    store_stage(kreg0, vreg0, 0);
    gload(kreg0, vreg0, 2);
    publish_vmax(vreg1, 1);
    lds_barrier();

    // Iteration s: write stage s + 1 (register slot (s+1) % 2, its |V| was
    // published before the last barrier), refill that slot with stage s + 3,
    // compute stage s, publish stage s + 2's |V| (slot s % 2), one barrier.
    // Unrolled twice (SL = s % 2, NX = the other slot) with no condition
    // around a load or store -- stages past the last are clamped re-reads,
    // written to a buffer nobody reads -- so that the compiler never has to
    // wait for the prefetched stages where control flow joins.
    f32x4 S[NQT][KT];
#define TEV_ATTN_STAGE(SL, NX)                                                                  \
    {                                                                                           \
        const int s = s0 + (SL);                                                                \
        const int vs_s = vs;   /* the scale stage s was written with */                        \
        store_stage(kreg##NX, vreg##NX, s + 1);                                                 \
        gload(kreg##NX, vreg##NX, s + 3);                                                       \
        qk(S, s & 1);                                                                           \
        spv(S, s, vs_s);                                                                        \
        publish_vmax(vreg##SL, s & 1);                                                          \
        lds_barrier();                                                                          \
    }
    for (int s0 = 0;; s0 += PD) {
        TEV_ATTN_STAGE(0, 1)
        if (s0 + 1 >= nstages) break;
        TEV_ATTN_STAGE(1, 0)
        if (s0 + 2 >= nstages) break;
    }
#undef TEV_ATTN_STAGE

    // Finalise: every lane of a query column holds the full sums.  With
    // splits, tile t of each wave is staged through LDS (the stage buffers are
    // free after the last barrier; wave w owns rows [16 w, 16 w + 16) of
    // buffer t) and written back as whole rows below.
    const size_t rows_all = (size_t)(n_wg / (row_blocks * splits)) * rows_total;
    constexpr int RST = D + 8;          // staging row stride (elements)
    static_assert(NQT <= 2 && NW * 16 * RST <= 2 * STK && NW * 16 * RST <= 2 * STV,
                  "a wave's staged tiles fit the K and V stage buffers");
#pragma unroll
    for (int t = 0; t < NQT; t++) {
        const float lt = accl[t][0];
        const int row = qrow[t];
        if (row >= rows_total) continue;
        const int i = row / G, hh = row - i * G;
        const float inv = __builtin_ldexpf(1.0f, vs_acc) / lt;   // O = acc 2^vs_acc / l
        if (splits == 1) {
            float *o = out + (((size_t)r * B + i) * Hq + g * G + hh) * D;
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
            float mx = 0.f;
#pragma unroll
            for (int dt = 0; dt < DT; dt++)
#pragma unroll
                for (int j = 0; j < 4; j++) mx = fmaxf(mx, fabsf(acc[t][dt][j]));
            mx = max_over_groups(mx) * inv;
            int ex = 0;
            (void)frexpf(mx, &ex);                          // mx = f 2^ex, f in [0.5, 1)
            const int u = (mx > 0.f) ? min(max(ex - 15, -126), 127) : 0;
            const float sc = inv * __builtin_ldexpf(1.0f, -u);
            const size_t prow = (size_t)sp * rows_all + (size_t)rg * rows_total + row;
            uint16_t *tile = (t == 0 ? s_k : s_v) + wave * 16 * RST;
#pragma unroll
            for (int dt = 0; dt < DT; dt++) {
                const f32x4 val = acc[t][dt] * sc;
                f16x4 h;
#pragma unroll
                for (int j = 0; j < 4; j++) h[j] = (_Float16)val[j];
                *reinterpret_cast<f16x4 *>(tile + l16 * RST + dt * 16 + grp * 4) = h;
            }
            if (grp == 0)
                *reinterpret_cast<f32x4 *>(part_ml + prow * 4) = f32x4{m_run[t], lt, (float)u, 0.f};
        }
    }
    if (splits > 1) {
        // Each store instruction writes four whole 2D-byte rows; the partials
        // are read once, by the combine, so they are written as streaming
        // (non-temporal) stores.  The staging writes above came from this
        // wave, so in-order LDS access is the only ordering needed.
        __builtin_amdgcn_wave_barrier();
#pragma unroll
        for (int t = 0; t < NQT; t++) {
            const uint16_t *tile = (t == 0 ? s_k : s_v) + wave * 16 * RST;
#pragma unroll
            for (int it = 0; it < D / 32; it++) {
                const int idx = it * 64 + lane;
                const int rr = idx / (D / 8), ch = idx % (D / 8);
                const int row = wrow0 + t * 16 + rr;
                const u32x4 w = *reinterpret_cast<const u32x4 *>(tile + rr * RST + ch * 8);
                if (row < rows_total) {
                    const size_t prow = (size_t)sp * rows_all + (size_t)rg * rows_total + row;
                    __builtin_nontemporal_store(w, reinterpret_cast<u32x4 *>(part_o + prow * D + ch * 8));
                }
            }
        }
    }
}

constexpr int MAX_SPLITS = 32;

// Merge split partials: one wave per query row (block b of 256 threads takes
// rows 4b .. 4b + 3); lane s reads split s's (m, l, u), every lane its D/64
// output columns of NS >= splits splits.  All loads are unconditional
// (clamped split index), so they are all in flight before the first use.
template <int D, int NS>
__device__ __forceinline__ void attn_combine_ns(const uint16_t *__restrict__ part_o,
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
    uint32_t o[NS];   // DPL fp16 values of split s (one or two halves)
#pragma unroll
    for (int s = 0; s < NS; s++) {
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
    for (int s = 0; s < NS; s++) {
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

// Loads as many splits as the launch can have: 8, 16, or MAX_SPLITS (splits is
// uniform, so one branch is taken; the loads of each stay unconditional).
template <int D>
__device__ __forceinline__ void attn_combine_wg(const uint16_t *__restrict__ part_o,
                                                const float *__restrict__ part_ml, int splits,
                                                int Hkv, int G, int B, int Hq, size_t rows_all,
                                                const unsigned *__restrict__ status,
                                                float *__restrict__ out, const int block) {
    if (splits <= 8)
        attn_combine_ns<D, 8>(part_o, part_ml, splits, Hkv, G, B, Hq, rows_all, status, out, block);
    else if (splits <= 16)
        attn_combine_ns<D, 16>(part_o, part_ml, splits, Hkv, G, B, Hq, rows_all, status, out, block);
    else
        attn_combine_ns<D, MAX_SPLITS>(part_o, part_ml, splits, Hkv, G, B, Hq, rows_all, status, out, block);
}

}  // namespace
}  // namespace tev
