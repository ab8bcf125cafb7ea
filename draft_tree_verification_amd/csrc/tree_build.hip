// tree_build.hip -- best-first draft tree over the top-K retained universe on
// gfx950.
//
// What is computed ("CAST: Cost-Aware Speculative Trees from One-Pass Block
// Drafters", App. C "Candidate construction" and Thm. 1; "Multi-Future
// Drafting", App. B, where the merged heap with one mode is DDTree's builder):
// for request r with draft logits z [L][V] (row j = draft position j + 1, q_j
// its softmax over the whole vocabulary), each position keeps its K most
// likely tokens (larger logit first, then smaller token id; rank = position in
// that list), and the tree is the B - 1 prefixes of that universe with the
// largest plug-in score prod_j q_j(y_j), emitted best first.  The key of a
// prefix is s = (sum_j z_{j,y_j}) - (sum_j lse_j): the logit sum is
// accumulated along the path in f64 (exact for bf16 logits), the logsumexp
// sum is one constant per depth.  Equal keys go to the shorter prefix, then to
// the lexicographically smaller rank sequence.
//
// Launches:
//   k_tb_slabs  grid (ns, R*L), 256 threads: one 8192-logit slab in registers;
//               slab maximum and f64 sum of exp(z - maximum); the slab's K
//               best keys, best first.  The K-th largest per-thread maximum
//               bounds the slab's K-th key from below, so only keys at or
//               above it (at most 32 K) go to LDS, where each is ranked by
//               counting.  key = (order-preserving bits of z) << 32 | ~token,
//               unique per token, so "larger logit, then smaller token" is one
//               unsigned comparison.
//   k_tb_rows   grid R*L, 256 threads: the row's slab lists in LDS; the largest
//               K-th entry over the lists bounds the row's K-th key from below;
//               each key at or above it is ranked by a binary search in every
//               list.  Writes the row's top K and its logsumexp (f64).
//   k_tb_heap   grid R, one wave: the best-first search.  The frontier sits in
//               registers (4 slots per lane; it never holds more than B
//               entries); each pop is one wave maximum over the keys (ties
//               settled by depth and rank sequence), emits a node and pushes
//               its next sibling and its first child.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "exit_law_dev.h"
#include "slab_dev.h"
#include "tree_build.h"
#include "wave_ops.h"

namespace tev {
namespace {

// order-preserving maps of float / double bits to unsigned integers
__device__ __forceinline__ uint32_t ord32(float x) {
    const uint32_t u = __float_as_uint(x);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float unord32(uint32_t o) {
    return __uint_as_float((o & 0x80000000u) ? (o & 0x7fffffffu) : ~o);
}
__device__ __forceinline__ uint64_t ord64(double x) {
    const uint64_t u = (uint64_t)__double_as_longlong(x);
    return (u >> 63) ? ~u : (u | (1ull << 63));
}
__device__ __forceinline__ uint64_t make_key(float x, int token) {
    return ((uint64_t)ord32(x) << 32) | (uint64_t)(~(uint32_t)token);
}
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t x) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        const uint64_t y = __shfl_xor(x, o);
        x = y > x ? y : x;
    }
    return x;
}

template <typename T, bool VEC>
__global__ __launch_bounds__(TB_THREADS) void k_tb_slabs(const T *__restrict__ z, int V, int ns, int K,
                                                         unsigned *__restrict__ flag,
                                                         float *__restrict__ slab_m,
                                                         double *__restrict__ slab_s,
                                                         uint64_t *__restrict__ cand) {
    constexpr int VW = 16 / (int)sizeof(T);
    constexpr int SPAN = TB_THREADS * VW;
    constexpr int NWV = TB_THREADS / 64;
    extern __shared__ uint64_t s_cand[];             // at most TB_EPT * K keys
    __shared__ uint64_t s_tmax[TB_THREADS];
    __shared__ float s_max[NWV];
    __shared__ double s_sum[NWV];
    __shared__ int s_cnt[NWV];
    __shared__ uint64_t s_tau;
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, s = blockIdx.x;
    const size_t m = blockIdx.y;
    const int start = s * TB_SLAB, len = min(TB_SLAB, V - start);
    float x[TB_EPT];
    load_slab<T, VEC, TB_THREADS, TB_EPT>(z + m * (size_t)V + start, len, tid, x);
    bool bad = false;
    float mx = -kInf;
    uint64_t tmax = 0;
#pragma unroll
    for (int k = 0; k < TB_EPT / VW; k++)
#pragma unroll
        for (int j = 0; j < VW; j++) {
            const float v = x[k * VW + j];
            const int idx = k * SPAN + tid * VW + j;
            bad |= (v != v) | (v == kInf);
            mx = fmaxf(mx, v);
            const uint64_t key = idx < len ? make_key(v, start + idx) : 0ull;
            tmax = key > tmax ? key : tmax;
        }
    mx = wave::max_f32(mx);
    if (lane == 0) s_max[wv] = mx;
    s_tmax[tid] = tmax;
    if (tid == 0) s_tau = 1ull;
    const int any_bad = __syncthreads_or(bad);
    mx = fmaxf(fmaxf(s_max[0], s_max[1]), fmaxf(s_max[2], s_max[3]));
    double acc = 0.0;
    if (mx > -kInf) {
#pragma unroll
        for (int j = 0; j < TB_EPT; j++) acc += exp((double)x[j] - (double)mx);
    }
    acc = wave::sum_f64(acc);
    if (lane == 0) s_sum[wv] = acc;
    // the thread whose maximum ranks K-th sets the bound (keys are unique)
    int rank = 0;
    for (int j = 0; j < TB_THREADS; j++) rank += s_tmax[j] > tmax;
    if (rank == K - 1 && tmax != 0ull) s_tau = tmax;
    __syncthreads();
    const uint64_t tau = s_tau;
    int cnt = 0;
#pragma unroll
    for (int k = 0; k < TB_EPT / VW; k++)
#pragma unroll
        for (int j = 0; j < VW; j++) {
            const int idx = k * SPAN + tid * VW + j;
            cnt += (idx < len && make_key(x[k * VW + j], start + idx) >= tau) ? 1 : 0;
        }
    int incl = cnt;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int t = __shfl_up(incl, o);
        if (lane >= o) incl += t;
    }
    if (lane == 63) s_cnt[wv] = incl;
    __syncthreads();
    int pos = incl - cnt;
    for (int w = 0; w < wv; w++) pos += s_cnt[w];
    const int n = s_cnt[0] + s_cnt[1] + s_cnt[2] + s_cnt[3];
#pragma unroll
    for (int k = 0; k < TB_EPT / VW; k++)
#pragma unroll
        for (int j = 0; j < VW; j++) {
            const int idx = k * SPAN + tid * VW + j;
            const uint64_t key = idx < len ? make_key(x[k * VW + j], start + idx) : 0ull;
            if (idx < len && key >= tau) s_cand[pos++] = key;
        }
    __syncthreads();
    uint64_t *out = cand + (m * ns + s) * (size_t)K;
    for (int i = tid; i < n; i += TB_THREADS) {
        const uint64_t c = s_cand[i];
        int r = 0;
        for (int j = 0; j < n; j++) r += s_cand[j] > c;
        if (r < K) out[r] = c;
    }
    for (int i = n + tid; i < K; i += TB_THREADS) out[i] = 0ull;   // a short slab: no more keys
    if (tid == 0) {
        slab_m[m * ns + s] = mx;
        slab_s[m * ns + s] = (s_sum[0] + s_sum[1]) + (s_sum[2] + s_sum[3]);
        flag[m * ns + s] = any_bad ? (unsigned)TEV_FLAG_NONFINITE : 0u;
    }
}

__global__ __launch_bounds__(TB_THREADS) void k_tb_rows(const unsigned *__restrict__ flag,
                                                        const float *__restrict__ slab_m,
                                                        const double *__restrict__ slab_s,
                                                        const uint64_t *__restrict__ cand, int ns, int K,
                                                        uint64_t *__restrict__ top, double *__restrict__ lse,
                                                        unsigned *__restrict__ row_flag) {
    extern __shared__ uint64_t s_list[];              // ns lists of K keys, each best first
    __shared__ uint64_t s_bound;
    const int tid = threadIdx.x, lane = tid & 63;
    const size_t m = blockIdx.x;
    const int nk = ns * K;
    for (int i = tid; i < nk; i += TB_THREADS) s_list[i] = cand[m * (size_t)nk + i];
    if (tid < 64) {
        // the row's logsumexp from the slab partials (ns <= 64: one per lane)
        float ms = -kInf;
        double ss = 0.0;
        unsigned fl = 0u;
        if (lane < ns) {
            ms = slab_m[m * ns + lane];
            ss = slab_s[m * ns + lane];
            fl = flag[m * ns + lane];
        }
        const float M = wave::max_f32(ms);
        double acc = (ms > -kInf) ? ss * exp((double)ms - (double)M) : 0.0;
        acc = wave::sum_f64(acc);
        const double l = M > -kInf ? (double)M + log(acc) : -(double)kInf;
        const bool any = __ballot(fl != 0u) != 0ull;
        if (lane == 0) {
            lse[m] = l;
            // NaN or +inf logits, or a row that is all -inf: q is undefined
            row_flag[m] = (any || !(l > -(double)kInf && l < (double)kInf)) ? (unsigned)TEV_FLAG_NONFINITE : 0u;
        }
    }
    __syncthreads();
    if (tid < 64) {
        uint64_t b = 1ull;
        for (int s = lane; s < ns; s += 64) {
            const uint64_t e = s_list[s * K + K - 1];
            b = e > b ? e : b;
        }
        b = wave_max_u64(b);
        if (lane == 0) s_bound = b;
    }
    __syncthreads();
    const uint64_t bound = s_bound;
    uint64_t *o = top + m * (size_t)K;
    for (int i = tid; i < nk; i += TB_THREADS) {
        const uint64_t c = s_list[i];
        if (c < bound) continue;
        // rank = number of keys above c: a binary search in every sorted list
        int r = 0;
        for (int s = 0; s < ns; s++) {
            const uint64_t *l = s_list + s * K;
            int lo = 0, hi = K;                         // first index whose key is <= c
            while (lo < hi) {
                const int mid = (lo + hi) >> 1;
                if (l[mid] > c) lo = mid + 1; else hi = mid;
            }
            r += lo;
        }
        if (r < K) o[r] = c;
    }
}

// The rank of depth d (1-based) packed big-endian: depths 1..8 in hi, 9..16 in lo.
__device__ __forceinline__ int rank_at(uint64_t hi, uint64_t lo, int d) {
    return d <= 8 ? (int)((hi >> (8 * (8 - d))) & 255u) : (int)((lo >> (8 * (16 - d))) & 255u);
}
__device__ __forceinline__ void set_rank(uint64_t &hi, uint64_t &lo, int d, int r) {
    if (d <= 8) {
        const int sh = 8 * (8 - d);
        hi = (hi & ~(255ull << sh)) | ((uint64_t)r << sh);
    } else {
        const int sh = 8 * (16 - d);
        lo = (lo & ~(255ull << sh)) | ((uint64_t)r << sh);
    }
}

struct Entry {
    double s, sz;
    uint64_t hi, lo;
    int depth, parent;      // depth 0: empty slot
};

// a before b in pop order: larger key, then shorter, then smaller rank sequence
__device__ __forceinline__ bool before(const Entry &a, const Entry &b) {
    if (a.depth == 0) return false;
    if (b.depth == 0) return true;
    if (a.s != b.s) return a.s > b.s;
    if (a.depth != b.depth) return a.depth < b.depth;
    if (a.hi != b.hi) return a.hi < b.hi;
    return a.lo < b.lo;
}

__device__ __forceinline__ Entry readlane_entry(const Entry &e, int l) {
    Entry o;
    o.s = wave::readlane_d(e.s, l);
    o.sz = wave::readlane_d(e.sz, l);
    o.hi = ((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(e.hi >> 32), l) << 32) |
           (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)e.hi, l);
    o.lo = ((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(e.lo >> 32), l) << 32) |
           (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)e.lo, l);
    o.depth = __builtin_amdgcn_readlane(e.depth, l);
    o.parent = __builtin_amdgcn_readlane(e.parent, l);
    return o;
}

constexpr int SLOTS = 4;    // frontier slots per lane: 256 entries >= B

__global__ __launch_bounds__(64) void k_tb_heap(const uint64_t *__restrict__ top, const double *__restrict__ lse,
                                                const unsigned *__restrict__ row_flag,
                                                const int32_t *__restrict__ root_tokens, int L, int K, int B,
                                                unsigned *__restrict__ status, int32_t *__restrict__ parents,
                                                int32_t *__restrict__ tokens, double *__restrict__ scores) {
    __shared__ double s_tz[TB_MAX_L * TB_MAX_K];
    __shared__ int s_tt[TB_MAX_L * TB_MAX_K];
    __shared__ double s_C[TB_MAX_L + 1];
    __shared__ double s_nsz[TEV_MAX_NODES];
    const int lane = threadIdx.x, r = blockIdx.x;
    unsigned fl = 0u;
    for (int i = lane; i < L * K; i += 64) {
        const uint64_t key = top[(size_t)r * L * K + i];
        s_tz[i] = (double)unord32((uint32_t)(key >> 32));
        s_tt[i] = (int)~(uint32_t)key;
    }
    for (int j = lane; j < L; j += 64) fl |= row_flag[(size_t)r * L + j];
    fl = (unsigned)wave::sum_i32((int)fl) != 0u ? (unsigned)TEV_FLAG_NONFINITE : 0u;
    if (lane == 0) {
        double c = 0.0;                                 // C[d] = lse_0 + ... + lse_{d-1}, in order
        s_C[0] = 0.0;
        for (int j = 0; j < L; j++) {
            c += lse[(size_t)r * L + j];
            s_C[j + 1] = c;
        }
        s_nsz[0] = 0.0;
        status[r] = fl;
        parents[(size_t)r * B] = -1;
        tokens[(size_t)r * B] = fl ? -1 : (root_tokens ? root_tokens[r] : 0);
        scores[(size_t)r * B] = fl ? __builtin_nan("") : 0.0;
    }
    __syncthreads();
    if (fl) {
        for (int n = 1 + lane; n < B; n += 64) {
            parents[(size_t)r * B + n] = -1;
            tokens[(size_t)r * B + n] = -1;
            scores[(size_t)r * B + n] = __builtin_nan("");
        }
        return;
    }
    Entry f[SLOTS];
#pragma unroll
    for (int q = 0; q < SLOTS; q++) f[q] = Entry{0.0, 0.0, 0ull, 0ull, 0, 0};
    if (B > 1 && lane == 0) {                            // the rank-0 token of position 1
        f[0].sz = s_tz[0];
        f[0].s = f[0].sz - s_C[1];
        f[0].depth = 1;
    }
    for (int n = 1; n < B; n++) {
        // the lane's best slot
        int bq = 0;
        Entry mine = f[0];
#pragma unroll
        for (int q = 1; q < SLOTS; q++)
            if (before(f[q], mine)) {
                mine = f[q];
                bq = q;
            }
        const uint64_t o = mine.depth ? ord64(mine.s) : 0ull;
        const uint64_t best = wave_max_u64(o);
        uint64_t ball = __ballot(o == best && mine.depth != 0);
        if (ball == 0ull) {                              // the universe is exhausted
            for (int i = n + lane; i < B; i += 64) {
                parents[(size_t)r * B + i] = -1;
                tokens[(size_t)r * B + i] = -1;
                scores[(size_t)r * B + i] = __builtin_nan("");
            }
            break;
        }
        int wl = __ffsll((long long)ball) - 1;
        Entry w = readlane_entry(mine, wl);
        ball &= ball - 1;
        while (ball) {                                   // equal keys: depth, then rank sequence
            const int l = __ffsll((long long)ball) - 1;
            ball &= ball - 1;
            const Entry e = readlane_entry(mine, l);
            if (before(e, w)) {
                w = e;
                wl = l;
            }
        }
        // emit node n
        const int d = w.depth;
        const int rk = rank_at(w.hi, w.lo, d);
        if (lane == 0) {
            parents[(size_t)r * B + n] = w.parent;
            tokens[(size_t)r * B + n] = s_tt[(d - 1) * K + rk];
            scores[(size_t)r * B + n] = w.s;
            s_nsz[n] = w.sz;
        }
        // the winner's slot takes the next sibling (or empties)
        Entry sib{0.0, 0.0, 0ull, 0ull, 0, 0};
        if (rk + 1 < K) {
            sib.sz = s_nsz[w.parent] + s_tz[(d - 1) * K + rk + 1];
            sib.s = sib.sz - s_C[d];
            sib.hi = w.hi;
            sib.lo = w.lo;
            set_rank(sib.hi, sib.lo, d, rk + 1);
            sib.depth = d;
            sib.parent = w.parent;
        }
        if (lane == wl) {
#pragma unroll
            for (int q = 0; q < SLOTS; q++)
                if (q == bq) f[q] = sib;
        }
        // the first child goes to the first free slot of the first lane with one
        if (d < L) {
            Entry ch;
            ch.sz = w.sz + s_tz[d * K];
            ch.s = ch.sz - s_C[d + 1];
            ch.hi = w.hi;
            ch.lo = w.lo;                                // rank 0 at depth d + 1: byte already 0
            ch.depth = d + 1;
            ch.parent = n;
            int fq = -1;
#pragma unroll
            for (int q = SLOTS - 1; q >= 0; q--)
                if (f[q].depth == 0) fq = q;
            const uint64_t fb = __ballot(fq >= 0);
            if (lane == __ffsll((long long)fb) - 1) {
#pragma unroll
                for (int q = 0; q < SLOTS; q++)
                    if (q == fq) f[q] = ch;
            }
        }
    }
}

template <typename T, bool VEC>
hipError_t launch_typed(const void *z, const int32_t *root_tokens, int R, int L, int V, int K, int B,
                        int32_t *parents, int32_t *tokens, double *scores, char *ws, hipStream_t st) {
    const TreeWs W = tree_ws_layout(R, L, V, K);
    const int ns = tb_slabs(V);
    unsigned *flag = (unsigned *)(ws + W.flag);
    float *slab_m = (float *)(ws + W.slab_m);
    double *slab_s = (double *)(ws + W.slab_s);
    uint64_t *cand = (uint64_t *)(ws + W.cand);
    uint64_t *top = (uint64_t *)(ws + W.top);
    double *lse = (double *)(ws + W.lse);
    unsigned *row_flag = (unsigned *)(ws + W.row_flag);
    k_tb_slabs<T, VEC><<<dim3((unsigned)ns, (unsigned)(R * L)), TB_THREADS, (size_t)TB_EPT * K * 8, st>>>(
        static_cast<const T *>(z), V, ns, K, flag, slab_m, slab_s, cand);
    k_tb_rows<<<R * L, TB_THREADS, (size_t)ns * K * 8, st>>>(flag, slab_m, slab_s, cand, ns, K, top, lse,
                                                             row_flag);
    k_tb_heap<<<R, 64, 0, st>>>(top, lse, row_flag, root_tokens, L, K, B, (unsigned *)(ws + W.status),
                                parents, tokens, scores);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_build_tree(const void *draft_logits, int dtype, bool vec, const int32_t *root_tokens,
                             int R, int L, int V, int K, int B, int32_t *parents, int32_t *tokens,
                             double *scores, char *ws, hipStream_t st) {
    if (dtype == TEV_BF16)
        return vec ? launch_typed<uint16_t, true>(draft_logits, root_tokens, R, L, V, K, B, parents, tokens,
                                                  scores, ws, st)
                   : launch_typed<uint16_t, false>(draft_logits, root_tokens, R, L, V, K, B, parents, tokens,
                                                   scores, ws, st);
    return vec ? launch_typed<float, true>(draft_logits, root_tokens, R, L, V, K, B, parents, tokens, scores,
                                           ws, st)
               : launch_typed<float, false>(draft_logits, root_tokens, R, L, V, K, B, parents, tokens, scores,
                                            ws, st);
}

}  // namespace tev
