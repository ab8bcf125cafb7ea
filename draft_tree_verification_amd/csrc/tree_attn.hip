// tree_attn.hip -- one layer of ancestor-masked tree attention on gfx950.
//
// What is computed ("CAST: Cost-Aware Speculative Trees from One-Pass Block
// Drafters", App. B Lemma 1; App. C "Packed verification"): query (r, i, h)
// attends to the P cached prefix rows and to the rows of its own root path
// (itself included) of kv head g = h / G, G = Hq / Hkv; cache row P + j holds
// tree node j.
//
// k_attn_mfma (bf16): one workgroup serves up to NW*NQT*16 query rows of one
// (request, kv head) -- the G*B rows (node i, head g*G + hh) share that head's
// K/V, so the GQA group times the tree makes the products dense -- over one
// split of the prefix; the last split also takes the B tree rows under the
// ancestor mask.  Per 32-key block, K (row-major) and V (transposed, key pairs
// packed in 32-bit words) are staged in LDS, double buffered, while the next
// block's global loads are in flight.  Scores are formed transposed,
//   S^T (32 keys x 16 queries) = K (32 x D) . Q^T (D x 16),
// with v_mfma_f32_16x16x32_bf16, so each lane holds one query column; the
// online-softmax probabilities of that column are exactly the B operand of
//   O^T (D x 16) += V^T (D x 32 keys) . P^T (32 keys x 16),
// with the 32 keys of a block taken in the order the score tiles leave them
// in registers (the V^T operand is read from LDS in the same order).  Tree
// rows are masked by a per-node ancestor bitmap in LDS (one bit per node).
// Partial results of split prefixes are merged by k_attn_combine.
//
// k_attn_alu (fp32): one wave per query row, lanes over head_dim, online
// softmax in fp32 -- a plain vector-ALU kernel for fp32 inputs.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <type_traits>
#include <utility>

#include "tev_internal.h"
#include "wave_ops.h"

namespace tev {
namespace {

constexpr float kInf = __builtin_inff();

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
// Plain clang vectors for 16- and 8-byte moves: unlike HIP's u32x4 struct they
// stay in registers (struct copies become memcpy that the compiler keeps in
// memory).
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

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
// fp32 vector-ALU kernel: grid (ceil(B*Hq/4), R), 256 threads, wave = one row.
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
    // prefix rows, then the root path of node i (walked upward)
    int j = i;
    for (int key = 0;; key++) {
        int row;
        if (key < P) {
            row = key;
        } else {
            if (j < 0) break;
            row = P + j;
            j = s_par[j];
        }
        float dot = 0.f;
#pragma unroll
        for (int p = 0; p < PER; p++) dot = fmaf(qv[p], kb[(size_t)row * D + lane + 64 * p], dot);
        const float s = wave_sum_f(dot) * scale;
        const float mn = fmaxf(m, s);
        const float alpha = expf(m - mn);
        const float pr = expf(s - mn);
        l = l * alpha + pr;
#pragma unroll
        for (int p = 0; p < PER; p++) acc[p] = acc[p] * alpha + pr * vb[(size_t)row * D + lane + 64 * p];
        m = mn;
    }
#pragma unroll
    for (int p = 0; p < PER; p++) o[lane + 64 * p] = acc[p] / l;
}

// ----------------------------------------------------------------------------
// bf16 MFMA kernel.
// ----------------------------------------------------------------------------
constexpr int KB = 32;   // keys per block
constexpr int kVsMin = -100;     // smallest V exponent shift (all-zero blocks)
constexpr float kLazy = 8.0f;    // slack of the softmax reference max (log2 units)

__device__ __forceinline__ uint32_t half_of(const u32x4 &x, int e) {
    const uint32_t w = x[e >> 1];
    return (e & 1) ? (w >> 16) : (w & 0xffffu);
}

__device__ __forceinline__ f16x8 pack_f16x8(const float *p) {
    f16x8 r;
#pragma unroll
    for (int e = 0; e < 8; e++) r[e] = (_Float16)p[e];
    return r;
}

// bf16 bit pattern -> fp16 bit pattern of the value times 2^-vs (exact while
// the scaled magnitude stays within fp16's normal range).
__device__ __forceinline__ uint32_t bf16_to_f16_scaled(uint32_t b, float scale) {
    const float f = __uint_as_float(b << 16) * scale;
    const _Float16 h = (_Float16)f;
    return (uint32_t)__builtin_bit_cast(uint16_t, h);
}

// Largest |value| of the 8 bf16 in x, as a 15-bit magnitude pattern (the
// ordering of non-negative IEEE patterns is the ordering of the values).
__device__ __forceinline__ uint32_t max_mag8(const u32x4 &x) {
    uint32_t m = 0;
#pragma unroll
    for (int i = 0; i < 4; i++) m = max(m, max(x[i] & 0x7fffu, (x[i] >> 16) & 0x7fffu));
    return m;
}

constexpr int PD = 4;   // K/V blocks in flight per workgroup (register prefetch depth)

// Grid: a 1-D list of n_wg workgroup tasks (row block, prefix split, request *
// kv head), row block fastest.  Hardware dispatches workgroup i to XCD i % 8,
// so task L = (i % 8) * ceil(n_wg / 8) + i / 8 puts consecutive tasks -- the
// row blocks that stream the same K/V -- on the same XCD and its L2.
template <int D, int NQT, int NW>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(1, 1))) void k_attn_mfma(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ k,
    const uint16_t *__restrict__ v, const int32_t *__restrict__ parents, int B, int Hq, int Hkv,
    int P, float c_log2, int row_blocks, int splits, int keys_per_split, int n_wg,
    float *__restrict__ out, float *__restrict__ part_o, float *__restrict__ part_ml,
    unsigned *__restrict__ status) {
    constexpr int NT = NW * 64;
    constexpr int DS = D / 32;          // k-steps of the score product
    constexpr int DT = D / 16;          // 16-row tiles of O^T
    constexpr int KROW = D + 8;         // K row stride in LDS (bf16 elements)
    constexpr int VROW = KB + 4;        // V^T row stride in LDS (fp16 elements)
    constexpr int WR = NW * NQT * 16;   // query rows per workgroup
    constexpr int K_ITEMS = KB * D / 8;         // 16-byte chunks of a K block
    constexpr int V_ITEMS = (KB / 2) * (D / 8); // (key pair, 8-column) items of a V block
    constexpr int NKI = (K_ITEMS + NT - 1) / NT;
    constexpr int NVI = (V_ITEMS + NT - 1) / NT;

    const int per_xcd = (n_wg + 7) / 8;
    const int task = (int)(blockIdx.x % 8) * per_xcd + (int)(blockIdx.x / 8);
    if (task >= n_wg) return;
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
    constexpr bool K_FULL = (K_ITEMS % NT) == 0;   // every thread owns NKI K chunks
    constexpr bool V_FULL = (V_ITEMS % NT) == 0;

    __shared__ __attribute__((aligned(16))) uint16_t s_k[2][KB * KROW];
    __shared__ __attribute__((aligned(16))) uint16_t s_vt[2][D * VROW];
    __shared__ unsigned s_anc[TEV_MAX_NODES * 8];
    __shared__ int s_par[TEV_MAX_NODES];
    __shared__ uint32_t s_wmax[2][NW];
    __shared__ int s_bad;

    const bool last = (sp == splits - 1);
    const int kbeg = sp * keys_per_split;
    const int kend = last ? P + B : kbeg + keys_per_split;
    const int nkv = P + B;
    const uint16_t *kbase = k + ((size_t)r * Hkv + g) * (size_t)nkv * D;
    const uint16_t *vbase = v + ((size_t)r * Hkv + g) * (size_t)nkv * D;
    const int nblocks = (kend - kbeg + KB - 1) / KB;

    // PD register stages, one named array pair per stage
    u32x4 kreg0[NKI], kreg1[NKI], kreg2[NKI], kreg3[NKI];
    u32x4 vreg0[NVI][2], vreg1[NVI][2], vreg2[NVI][2], vreg3[NVI][2];
    auto gload = [=](u32x4 (&kr)[NKI], u32x4 (&vr)[NVI][2], int kb) __attribute__((always_inline)) {
#pragma unroll
        for (int n = 0; n < NKI; n++) {
            const int item = tid + n * NT;
            if (K_FULL || item < K_ITEMS) {
                const int key = item / (D / 8), d0 = (item % (D / 8)) * 8;
                const int kk = min(kb + key, nkv - 1);
                kr[n] = *reinterpret_cast<const u32x4 *>(kbase + (size_t)kk * D + d0);
            }
        }
#pragma unroll
        for (int n = 0; n < NVI; n++) {
            const int item = tid + n * NT;
            if (V_FULL || item < V_ITEMS) {
                const int kp = item % (KB / 2), d0 = (item / (KB / 2)) * 8;
                const int k0 = min(kb + 2 * kp, nkv - 1), k1 = min(kb + 2 * kp + 1, nkv - 1);
                vr[n][0] = *reinterpret_cast<const u32x4 *>(vbase + (size_t)k0 * D + d0);
                vr[n][1] = *reinterpret_cast<const u32x4 *>(vbase + (size_t)k1 * D + d0);
            } else {
                vr[n][0] = u32x4{0u, 0u, 0u, 0u};
                vr[n][1] = u32x4{0u, 0u, 0u, 0u};
            }
        }
    };
    // Largest |V| of the block held in register slot sl, per wave, into s_wmax[buf].
    auto publish_vmax = [=](const u32x4 (&vr)[NVI][2], uint32_t *wmax) __attribute__((always_inline)) {
        uint32_t m = 0;
#pragma unroll
        for (int n = 0; n < NVI; n++) m = max(m, max(max_mag8(vr[n][0]), max_mag8(vr[n][1])));
        m = (uint32_t)wave::max_i32((int)m);
        if (lane == 0) wmax[wave] = m;
    };
    // K as is; V transposed and converted to fp16 times 2^-vs.  vs is the
    // smallest exponent seen so far that keeps every scaled |V| below 2^15: it
    // only ever grows, so the accumulators change units only when a block with
    // larger values arrives.
    auto lstore = [=](const u32x4 (&kr)[NKI], const u32x4 (&vr)[NVI][2], uint16_t *sk, uint16_t *svt,
                      const uint32_t *wmax, int &vs_run) __attribute__((always_inline)) {
#pragma unroll
        for (int n = 0; n < NKI; n++) {
            const int item = tid + n * NT;
            if (K_FULL || item < K_ITEMS) {
                const int key = item / (D / 8), d0 = (item % (D / 8)) * 8;
                *reinterpret_cast<u32x4 *>(&sk[key * KROW + d0]) = kr[n];
            }
        }
        uint32_t mb = 0;
#pragma unroll
        for (int w = 0; w < NW; w++) mb = max(mb, wmax[w]);
        const int ebits = (int)(mb >> 7);                       // bf16 biased exponent
        const int vs_need = mb == 0 ? kVsMin : min(max(ebits - 141, kVsMin), 15);
        vs_run = max(vs_run, vs_need);
        const float vscale = __builtin_ldexpf(1.0f, -vs_run);
#pragma unroll
        for (int n = 0; n < NVI; n++) {
            const int item = tid + n * NT;
            if (V_FULL || item < V_ITEMS) {
                const int kp = item % (KB / 2), d0 = (item / (KB / 2)) * 8;
#pragma unroll
                for (int e = 0; e < 8; e++) {
                    const uint32_t w = bf16_to_f16_scaled(half_of(vr[n][0], e), vscale) |
                                       (bf16_to_f16_scaled(half_of(vr[n][1], e), vscale) << 16);
                    *reinterpret_cast<uint32_t *>(&svt[(d0 + e) * VROW + 2 * kp]) = w;
                }
            }
        }
    };

    // Issue order: Q^T operands and the request's parents first, then the K/V
    // prefetch, so that waiting for the small loads never waits for the stream.
    bf16x8 qop[NQT][DS];
    int qnode[NQT], qrow[NQT];
#pragma unroll
    for (int t = 0; t < NQT; t++) {
        const int row = rb * WR + wave * NQT * 16 + t * 16 + l16;
        qrow[t] = row;
        const int rr = min(row, rows_total - 1);
        const int i = rr / G, hh = rr - i * G;
        qnode[t] = i;
        const uint16_t *qp = q + (((size_t)r * B + i) * Hq + g * G + hh) * D;
#pragma unroll
        for (int ds = 0; ds < DS; ds++)
            qop[t][ds] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4 *>(qp + ds * 32 + grp * 8));
    }
    constexpr int NPAR = (TEV_MAX_NODES + NT - 1) / NT;
    int my_par[NPAR];
#pragma unroll
    for (int n = 0; n < NPAR; n++) {
        const int i = tid + n * NT;
        my_par[n] = (last && i < B) ? parents[(size_t)r * B + i] : -1;
    }

    if (0 < nblocks) gload(kreg0, vreg0, kbeg);
    if (1 < nblocks) gload(kreg1, vreg1, kbeg + KB);
    if (2 < nblocks) gload(kreg2, vreg2, kbeg + 2 * KB);
    if (3 < nblocks) gload(kreg3, vreg3, kbeg + 3 * KB);

    // Tree contract (parents[0] = -1, 0 <= parents[i] < i) and the ancestor
    // bitmap of every node (bit j of node i: j lies on i's root path).
    bool tree_ok = true;
    if (last) {
        if (tid == 0) s_bad = 0;
#pragma unroll
        for (int n = 0; n < NPAR; n++) {
            const int i = tid + n * NT;
            if (i < B) s_par[i] = my_par[n];
        }
        __syncthreads();
#pragma unroll
        for (int n = 0; n < NPAR; n++) {
            const int i = tid + n * NT, p = my_par[n];
            if (i < B && !((i == 0) ? (p == -1) : (p >= 0 && p < i))) s_bad = 1;
        }
        __syncthreads();
        tree_ok = s_bad == 0;
        if (tree_ok) {
#pragma unroll
            for (int n = 0; n < NPAR; n++) {
                const int i = tid + n * NT;
                if (i >= B) continue;
                unsigned a[8] = {0u, 0u, 0u, 0u, 0u, 0u, 0u, 0u};
                for (int j = i; j >= 0; j = s_par[j]) {
#pragma unroll
                    for (int w = 0; w < 8; w++) a[w] |= ((j >> 5) == w) ? (1u << (j & 31)) : 0u;
                }
#pragma unroll
                for (int w = 0; w < 8; w++) s_anc[i * 8 + w] = a[w];
            }
        }
        if (rb == 0 && g == 0 && tid == 0) status[r] = tree_ok ? 0u : TEV_FLAG_TREE;
    }

    f32x4 acc[NQT][DT];          // O^T in units of 2^-vs_cur
    float m_run[NQT], l_run[NQT];
#pragma unroll
    for (int t = 0; t < NQT; t++) {
        m_run[t] = -kInf;
        l_run[t] = 0.f;
#pragma unroll
        for (int dt = 0; dt < DT; dt++) acc[t][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    int vs_cur = kVsMin;   // unit of acc: 2^-vs_cur
    int vs_run = kVsMin;   // unit of the V block last written to LDS

    auto compute = [=](int kb, int buf, f32x4 (&acc)[NQT][DT], float (&m_run)[NQT], float (&l_run)[NQT],
                       int &vs_cur, const int vs_blk) __attribute__((always_inline)) {
        const float vfix = __builtin_ldexpf(1.0f, vs_cur - vs_blk);   // re-express acc in 2^-vs_blk
        const bool vchange = vs_blk != vs_cur;
        vs_cur = vs_blk;
        const bool masked = (kb + KB > P) || (kb + KB > kend);

        // S^T tiles of every query tile: K operands loaded one key tile at a time.
        f32x4 S[NQT][2];
#pragma unroll
        for (int t = 0; t < NQT; t++) S[t][0] = S[t][1] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kt = 0; kt < 2; kt++) {
            bf16x8 kop[DS];
#pragma unroll
            for (int ds = 0; ds < DS; ds++)
                kop[ds] = *reinterpret_cast<const bf16x8 *>(&s_k[buf][(kt * 16 + l16) * KROW + ds * 32 + grp * 8]);
#pragma unroll
            for (int ds = 0; ds < DS; ds++)
#pragma unroll
                for (int t = 0; t < NQT; t++)
                    S[t][kt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kop[ds], qop[t][ds], S[t][kt], 0, 0, 0);
        }

        // Online softmax per query column; P^T operands in fp16.
        f16x8 pop[NQT];
#pragma unroll
        for (int t = 0; t < NQT; t++) {
            // sv[e]: key kb + grp*4 + e (e < 4) or kb + 16 + grp*4 + (e - 4)
            float sv[8] = {S[t][0][0], S[t][0][1], S[t][0][2], S[t][0][3],
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
                    sv[e] = vis ? sv[e] : -kInf;
                }
            }
            float bm = sv[0];
#pragma unroll
            for (int e = 1; e < 8; e++) bm = fmaxf(bm, sv[e]);
            bm = fmaxf(bm, __shfl_xor(bm, 16));
            bm = fmaxf(bm, __shfl_xor(bm, 32));
            // The reference max moves only when the block's max exceeds it by
            // more than kLazy (log2 units): probabilities stay <= 2^kLazy, exact
            // in fp16, and the accumulators are rescaled only when it moves.
            const float bmc = bm * c_log2;
            const bool grow = bmc > m_run[t] + kLazy;
            const float m_new = grow ? bmc : m_run[t];
            const float m_use = (m_new == -kInf) ? 0.f : m_new;
            const float alpha = grow ? __builtin_amdgcn_exp2f(m_run[t] - m_use) : 1.0f;
            float pv[8];
            float ps = 0.f;
#pragma unroll
            for (int e = 0; e < 8; e++) {
                pv[e] = __builtin_amdgcn_exp2f(fmaf(sv[e], c_log2, -m_use));
                ps += pv[e];
            }
            l_run[t] = l_run[t] * alpha + ps;
            m_run[t] = m_new;
            if (vchange || __any(grow)) {
                const float f = alpha * vfix;
#pragma unroll
                for (int dt = 0; dt < DT; dt++) acc[t][dt] *= f;
            }
            pop[t] = pack_f16x8(pv);
        }

        // O^T += V^T P^T: V operands loaded one d-tile at a time.
#pragma unroll
        for (int dt = 0; dt < DT; dt++) {
            const uint16_t *vr = &s_vt[buf][(dt * 16 + l16) * VROW];
            const u32x2 lo = *reinterpret_cast<const u32x2 *>(vr + grp * 4);
            const u32x2 hi = *reinterpret_cast<const u32x2 *>(vr + 16 + grp * 4);
            const f16x8 vop = __builtin_bit_cast(f16x8, u32x4{lo.x, lo.y, hi.x, hi.y});
#pragma unroll
            for (int t = 0; t < NQT; t++)
                acc[t][dt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vop, pop[t], acc[t][dt], 0, 0, 0);
        }
    };

    // Block 0 into LDS buffer 0 (the tree bitmap above is also published here).
    if (nblocks > 0) publish_vmax(vreg0, s_wmax[0]);
    __syncthreads();
    if (nblocks > 0) lstore(kreg0, vreg0, s_k[0], s_vt[0], s_wmax[0], vs_run);
    __syncthreads();

    // Block b sits in register slot b % PD until it is written to LDS buffer
    // b & 1 at the end of iteration b - 1; its slot is then refilled with block
    // b + PD at the start of iteration b.
    // One pipeline stage: block b = b0 + SL lives in stage SL's registers; NX is
    // the stage that holds block b + 1.
#define TEV_ATTN_STAGE(SL, NX)                                                                  \
    {                                                                                           \
        const int b = b0 + (SL);                                                                \
        if (b < nblocks) {                                                                      \
            if (b + PD < nblocks) gload(kreg##SL, vreg##SL, kbeg + (b + PD) * KB);              \
            compute(kbeg + b * KB, b & 1, acc, m_run, l_run, vs_cur, vs_run);                   \
            if (b + 1 < nblocks) {                                                              \
                const int nb = (b + 1) & 1;                                                     \
                publish_vmax(vreg##NX, s_wmax[nb]);                                             \
                __syncthreads(); /* all waves are done reading buffer nb */                     \
                lstore(kreg##NX, vreg##NX, s_k[nb], s_vt[nb], s_wmax[nb], vs_run);              \
                __syncthreads();                                                                \
            }                                                                                   \
        }                                                                                       \
    }
    static_assert(PD == 4, "the pipeline below is written out for four register stages");
    for (int b0 = 0; b0 < nblocks; b0 += PD) {
        TEV_ATTN_STAGE(0, 1)
        TEV_ATTN_STAGE(1, 2)
        TEV_ATTN_STAGE(2, 3)
        TEV_ATTN_STAGE(3, 0)
    }
#undef TEV_ATTN_STAGE
    const float vunscale = __builtin_ldexpf(1.0f, vs_cur);

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
            const float inv = vunscale / lt;
#pragma unroll
            for (int dt = 0; dt < DT; dt++) {
                f32x4 val = acc[t][dt] * inv;
                if (!tree_ok) val = f32x4{__builtin_nanf(""), __builtin_nanf(""), __builtin_nanf(""), __builtin_nanf("")};
                *reinterpret_cast<f32x4 *>(o + dt * 16 + grp * 4) = val;
            }
        } else {
            const size_t prow = (size_t)sp * rows_all + (size_t)rg * rows_total + row;
            float *o = part_o + prow * D;
#pragma unroll
            for (int dt = 0; dt < DT; dt++) *reinterpret_cast<f32x4 *>(o + dt * 16 + grp * 4) = acc[t][dt] * vunscale;
            if (grp == 0) {
                part_ml[prow * 2] = m_run[t];
                part_ml[prow * 2 + 1] = lt;
            }
        }
    }
}

constexpr int MAX_SPLITS = 32;

// Merge split partials: one wave per query row (grid ceil(rows_all / 4), 256
// threads); lane s reads split s's (m, l), every lane its D/64 output
// columns of all splits, all loads issued before the first use.
template <int D>
__global__ __launch_bounds__(256) void k_attn_combine(const float *__restrict__ part_o,
                                                      const float *__restrict__ part_ml,
                                                      int splits, int Hkv, int G, int B, int Hq,
                                                      size_t rows_all,
                                                      const unsigned *__restrict__ status,
                                                      float *__restrict__ out) {
    constexpr int DPL = D / 64;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const size_t row = (size_t)blockIdx.x * 4 + wave;
    if (row >= rows_all) return;
    const int rows_total = G * B;
    const int rg = (int)(row / rows_total);
    const int rr = (int)(row - (size_t)rg * rows_total);
    const int r = rg / Hkv, g = rg - r * Hkv;
    const int i = rr / G, hh = rr - i * G;
    float ms = -kInf, ls = 0.f;
    if (lane < splits) {
        ms = part_ml[((size_t)lane * rows_all + row) * 2];
        ls = part_ml[((size_t)lane * rows_all + row) * 2 + 1];
    }
    float o[MAX_SPLITS][DPL];
#pragma unroll
    for (int s = 0; s < MAX_SPLITS; s++)
#pragma unroll
        for (int j = 0; j < DPL; j++)
            o[s][j] = (s < splits) ? part_o[((size_t)s * rows_all + row) * D + lane * DPL + j] : 0.f;
    const float M = wave::max_f32(ms);
    const float wgt = (ms > -kInf) ? __builtin_amdgcn_exp2f(ms - M) : 0.f;
    const float L = wave::sum_f32(ls * wgt);
    float acc[DPL];
#pragma unroll
    for (int j = 0; j < DPL; j++) acc[j] = 0.f;
#pragma unroll
    for (int s = 0; s < MAX_SPLITS; s++) {
        if (s < splits) {
            const float ws = wave::readlane_f(wgt, s);
#pragma unroll
            for (int j = 0; j < DPL; j++) acc[j] = fmaf(ws, o[s][j], acc[j]);
        }
    }
    const bool bad = status[r] != 0u;
    float *dst = out + (((size_t)r * B + i) * Hq + g * G + hh) * D + lane * DPL;
#pragma unroll
    for (int j = 0; j < DPL; j++) dst[j] = bad ? __builtin_nanf("") : acc[j] / L;
}

template <int D, int NQT, int NW>
hipError_t mfma_impl(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                     const int32_t *parents, int R, int B, int Hq, int Hkv, int P, float scale,
                     float *out, char *ws, const AttnPlan &pl, hipStream_t st) {
    const AttnWs L = attn_ws_layout(R, B, Hq, Hkv, D, P);
    const float c_log2 = (float)((double)scale * 1.4426950408889634);
    float *part_o = (float *)(ws + L.part_o);
    float *part_ml = (float *)(ws + L.part_ml);
    unsigned *status = (unsigned *)(ws + L.status);
    const int n_wg = pl.row_blocks * pl.splits * R * Hkv;
    const int grid = 8 * ((n_wg + 7) / 8);
    k_attn_mfma<D, NQT, NW><<<dim3(grid), NW * 64, 0, st>>>(
        q, k, v, parents, B, Hq, Hkv, P, c_log2, pl.row_blocks, pl.splits, pl.keys_per_split, n_wg,
        out, part_o, part_ml, status);
    if (pl.splits > 1) {
        const int G = Hq / Hkv;
        const size_t rows_all = (size_t)R * Hkv * G * B;
        k_attn_combine<D><<<dim3((unsigned)((rows_all + 3) / 4)), 256, 0, st>>>(
            part_o, part_ml, pl.splits, Hkv, G, B, Hq, rows_all, status, out);
    }
    return hipGetLastError();
}

}  // namespace

AttnPlan attn_plan(int R, int B, int Hq, int Hkv, int D, int P) {
    (void)D;
    AttnPlan p{};
    p.nqt = 2;
    p.nw = 4;
    p.rows_per_wg = p.nw * p.nqt * 16;
    const int G = Hq / Hkv;
    p.row_blocks = (G * B + p.rows_per_wg - 1) / p.rows_per_wg;
    const long base = (long)R * Hkv * p.row_blocks;
    // Enough workgroups to cover 256 CUs twice, each split keeping >= 256
    // prefix keys so that per-split fixed costs stay small.
    long want = (512 + base - 1) / base;
    long maxs = P / 256;
    if (maxs < 1) maxs = 1;
    if (maxs > MAX_SPLITS) maxs = MAX_SPLITS;
    int S = (int)(want < maxs ? want : maxs);
    if (S < 1) S = 1;
    int kps = 0;
    if (S > 1) {
        kps = (P + S - 1) / S;
        kps = (kps + KB - 1) / KB * KB;
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
    if (D == 64) return mfma_impl<64, 2, 4>(qb, kb, vb, parents, R, B, Hq, Hkv, P, scale, out, ws, pl, st);
    return mfma_impl<128, 2, 4>(qb, kb, vb, parents, R, B, Hq, Hkv, P, scale, out, ws, pl, st);
}

}  // namespace tev
