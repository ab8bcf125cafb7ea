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
//               best keys, best first (block_top_k).  key = (order-preserving
//               bits of z) << 32 | ~token,
//               unique per token, so "larger logit, then smaller token" is one
//               unsigned comparison.
//   k_tb_rows   grid R*L, 256 threads: the union of the row's slab lists, 32
//               keys per thread, through the same selection; writes the row's
//               top K and its logsumexp (f64).
//   k_tb_heap   grid R, one wave: the best-first search.  The frontier has
//               one slot per node holding that node's next child; a slot's
//               key word sits in registers (ceil(B / 64) per lane) and the
//               rest of it in an LDS record.  Each pop is one DPP wave
//               maximum over the key words, exact stages among the slots
//               that tie there, one read of the winner's record, and the
//               winner's slot moved to the next sibling and the new node's
//               slot opened with its rank-0 child.  With several draft modes
//               the grid is R * M and each mode's pops go to a stream.
//   k_tb_merge  grid R, 1024 threads (several modes only): the merged heap
//               from the modes' streams -- each entry's place in the merged
//               order, canonical prefix ids, the nodes at each prefix's
//               first place.
#include <hip/hip_runtime.h>

#include <algorithm>
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
    return u ^ ((uint64_t)((int64_t)u >> 63) | (1ull << 63));   // negative: all bits flipped; else the sign bit set
}
__device__ __forceinline__ uint64_t make_key(float x, int token) {
    return ((uint64_t)ord32(x) << 32) | (uint64_t)(~(uint32_t)token);
}

// Wave-wide bitwise AND and OR, and an inclusive prefix sum over the lanes
// (in-row steps by DPP, then the totals of the rows before).
__device__ __forceinline__ uint32_t wave_and_u32(uint32_t x) {
    x &= (uint32_t)wave::dpp_i<wave::kQuadXor1>((int)x);
    x &= (uint32_t)wave::dpp_i<wave::kQuadXor2>((int)x);
    x &= (uint32_t)wave::dpp_i<wave::kRowHalfMirror>((int)x);
    x &= (uint32_t)wave::dpp_i<wave::kRowMirror>((int)x);
    return ((uint32_t)__builtin_amdgcn_readlane((int)x, 0) & (uint32_t)__builtin_amdgcn_readlane((int)x, 16)) &
           ((uint32_t)__builtin_amdgcn_readlane((int)x, 32) & (uint32_t)__builtin_amdgcn_readlane((int)x, 48));
}
__device__ __forceinline__ uint32_t wave_or_u32(uint32_t x) {
    x |= (uint32_t)wave::dpp_i<wave::kQuadXor1>((int)x);
    x |= (uint32_t)wave::dpp_i<wave::kQuadXor2>((int)x);
    x |= (uint32_t)wave::dpp_i<wave::kRowHalfMirror>((int)x);
    x |= (uint32_t)wave::dpp_i<wave::kRowMirror>((int)x);
    return ((uint32_t)__builtin_amdgcn_readlane((int)x, 0) | (uint32_t)__builtin_amdgcn_readlane((int)x, 16)) |
           ((uint32_t)__builtin_amdgcn_readlane((int)x, 32) | (uint32_t)__builtin_amdgcn_readlane((int)x, 48));
}
__device__ __forceinline__ int wave_incl_scan_i32(int x, int lane) {
    x += __builtin_amdgcn_mov_dpp(x, wave::kRowShr + 1, 0xF, 0xF, true);
    x += __builtin_amdgcn_mov_dpp(x, wave::kRowShr + 2, 0xF, 0xF, true);
    x += __builtin_amdgcn_mov_dpp(x, wave::kRowShr + 4, 0xF, 0xF, true);
    x += __builtin_amdgcn_mov_dpp(x, wave::kRowShr + 8, 0xF, 0xF, true);
    const int r0 = __builtin_amdgcn_readlane(x, 15), r1 = __builtin_amdgcn_readlane(x, 31),
              r2 = __builtin_amdgcn_readlane(x, 47);
    const int row = lane >> 4;
    return x + (row == 0 ? 0 : row == 1 ? r0 : row == 2 ? r0 + r1 : (r0 + r1) + r2);
}

// Radix select of the K-th largest of the 32-bit values v[i] that are in the
// set (in[i]), by the whole wave, most significant bit first, over the bits on
// which those values differ (bits they all share are the answer's).  rem: K
// on entry, the rank of the answer among the set's values equal to it on
// return (1 = the first of them).
template <int VPL>
__device__ __forceinline__ uint32_t wave_radix_select(const uint32_t (&v)[VPL], const bool (&in)[VPL], int &rem) {
    uint32_t a = ~0u, o = 0u;
#pragma unroll
    for (int i = 0; i < VPL; i++) {
        a &= in[i] ? v[i] : ~0u;
        o |= in[i] ? v[i] : 0u;
    }
    const uint32_t all1 = wave_and_u32(a), any1 = wave_or_u32(o);
    uint32_t vary = all1 ^ any1, prefix = all1, mask = ~vary;
    while (vary) {
        const uint32_t bit = 1u << (31 - __clz((int)vary));
        vary &= ~bit;
        const uint32_t m = mask | bit, cand = prefix | bit;
        int cnt = 0;
#pragma unroll
        for (int i = 0; i < VPL; i++) cnt += __popcll(__ballot(in[i] && (v[i] & m) == cand));
        if (cnt >= rem)
            prefix = cand;
        else
            rem -= cnt;
        mask = m;
    }
    return prefix;
}

// The K-th largest high half th of the 64 VPL values v (with multiplicity;
// K <= 64 VPL), by the whole wave; rem returns the answer's rank among the
// values whose high half is th.
template <int VPL>
__device__ __forceinline__ uint32_t wave_kth_high(const uint64_t (&v)[VPL], int K, int &rem) {
    uint32_t h[VPL];
    bool in[VPL];
#pragma unroll
    for (int i = 0; i < VPL; i++) {
        h[i] = (uint32_t)(v[i] >> 32);
        in[i] = true;
    }
    rem = K;
    return wave_radix_select<VPL>(h, in, rem);
}
// The K-th largest of the values v, given th and rem from wave_kth_high: the
// low halves of the values whose high half is th.
template <int VPL>
__device__ __forceinline__ uint64_t wave_kth_exact(const uint64_t (&v)[VPL], uint32_t th, int rem) {
    uint32_t l[VPL];
    bool in[VPL];
#pragma unroll
    for (int i = 0; i < VPL; i++) {
        l[i] = (uint32_t)v[i];
        in[i] = (uint32_t)(v[i] >> 32) == th;
    }
    return ((uint64_t)th << 32) | wave_radix_select<VPL>(l, in, rem);
}

// The K best of the keys the workgroup holds, N per thread (0 = no key),
// written best first to out[0..K) (0 past the last key).  K threads hold a key
// whose high half is at least th, the K-th largest high half of the
// per-thread maxima, so the K-th key is at least th << 32; the caller's floor
// (0: none) bounds it from below too.  The keys at or above the larger bound
// are compacted into LDS, where each is ranked by counting the larger ones;
// should they be more than N K (maxima tied on their high halves), the bound
// becomes the K-th largest maximum itself, which at most K threads reach.
// Keys are unique, so the ranks are distinct.
template <int N>
__device__ __forceinline__ void block_top_k(const uint64_t (&key)[N], int K, uint64_t *s_c, uint64_t *s_tmax,
                                            int *s_cnt, uint64_t *out, uint64_t floor_key = 0ull) {
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    static_assert(TB_THREADS == 256, "four maxima per lane of one wave");
    uint64_t tmax = 0ull;
#pragma unroll
    for (int j = 0; j < N; j++) tmax = key[j] > tmax ? key[j] : tmax;
    s_tmax[tid] = tmax;
    __syncthreads();
    // every wave selects the same bound from the 256 maxima
    uint64_t tv[4];
#pragma unroll
    for (int i = 0; i < 4; i++) tv[i] = s_tmax[4 * lane + i];
    int rem;
    const uint32_t th = wave_kth_high<4>(tv, K, rem);
    uint64_t tau = (uint64_t)th << 32;
    int cnt, incl, n, pass = 0;
    for (;; pass++) {
        tau = tau > floor_key ? tau : floor_key;
        tau = tau > 1ull ? tau : 1ull;                // 0 is no key
        cnt = 0;
#pragma unroll
        for (int j = 0; j < N; j++) cnt += key[j] >= tau ? 1 : 0;
        incl = wave_incl_scan_i32(cnt, lane);
        if (lane == 63) s_cnt[wv + 4 * pass] = incl;
        __syncthreads();
        n = 0;
#pragma unroll
        for (int w = 0; w < TB_THREADS / 64; w++) n += s_cnt[w + 4 * pass];
        if (pass == 1 || n <= N * K) break;           // uniform
        tau = wave_kth_exact<4>(tv, th, rem);
    }
    int pos = incl - cnt;
    for (int w = 0; w < wv; w++) pos += s_cnt[w + 4 * pass];
    // every key is stored, the others to the wave's lane slot past the
    // N K + 16 compacted ones, so no store waits on a branch
    const int spare = N * K + 16 + tid;
#pragma unroll
    for (int j = 0; j < N; j++) {
        const bool c = key[j] >= tau;
        s_c[c ? pos : spare] = key[j];
        pos += c ? 1 : 0;
    }
    const int n16 = (n + 15) & ~15;                   // zero padding: never above a key
    for (int i = n + tid; i < n16; i += TB_THREADS) s_c[i] = 0ull;
    __syncthreads();
    // rank by counting; with few keys, G adjacent lanes share a key's count
    const int G = n <= TB_THREADS / 4 ? 4 : n <= TB_THREADS / 2 ? 2 : 1;   // uniform
    const int seg = ((n16 / G) + 15) & ~15;
    for (int i0 = 0; i0 < n; i0 += TB_THREADS / G) {
        const int i = i0 + tid / G, g = tid % G;
        const uint64_t c = i < n ? s_c[i] : 0ull;
        int r = 0;
        const int j1 = min(n16, (g + 1) * seg);
        for (int j = g * seg; j < j1; j += 16) {
            ulonglong2 t[8];
#pragma unroll
            for (int u = 0; u < 8; u++) t[u] = *reinterpret_cast<const ulonglong2 *>(s_c + j + 2 * u);
#pragma unroll
            for (int u = 0; u < 8; u++) r += (t[u].x > c ? 1 : 0) + (t[u].y > c ? 1 : 0);
        }
        if (G >= 2) r += wave::dpp_i<wave::kQuadXor1>(r);
        if (G == 4) r += wave::dpp_i<wave::kQuadXor2>(r);
        if (i < n && g == 0 && r < K) out[r] = c;
    }
    for (int i = n + tid; i < K; i += TB_THREADS) out[i] = 0ull;
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
    extern __shared__ __align__(16) uint64_t s_c[];   // TB_EPT * K keys, 16 of padding, a spare slot per thread
    __shared__ uint64_t s_tmax[TB_THREADS];
    __shared__ float s_max[NWV];
    __shared__ double s_sum[NWV];
    __shared__ int s_cnt[2 * NWV];                   // per wave, two passes
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, s = blockIdx.x;
    const size_t m = blockIdx.y;
    const int start = s * TB_SLAB, len = min(TB_SLAB, V - start);
    float x[TB_EPT];
    load_slab<T, VEC, TB_THREADS, TB_EPT>(z + m * (size_t)V + start, len, tid, x);
    bool bad = false;
    float mx = -kInf;
#pragma unroll
    for (int j = 0; j < TB_EPT; j++) {
        bad |= (x[j] != x[j]) | (x[j] == kInf);
        mx = fmaxf(mx, x[j]);
    }
    mx = wave::max_f32(mx);
    if (lane == 0) s_max[wv] = mx;
    const int any_bad = __syncthreads_or(bad);
    mx = fmaxf(fmaxf(s_max[0], s_max[1]), fmaxf(s_max[2], s_max[3]));
    double acc = 0.0;
    if (mx > -kInf) {
#pragma unroll
        for (int j = 0; j < TB_EPT; j++) acc += exp((double)x[j] - (double)mx);
    }
    acc = wave::sum_f64(acc);
    if (lane == 0) s_sum[wv] = acc;
    uint64_t key[TB_EPT];
#pragma unroll
    for (int k = 0; k < TB_EPT / VW; k++)
#pragma unroll
        for (int j = 0; j < VW; j++) {
            const int idx = k * SPAN + tid * VW + j;
            key[k * VW + j] = idx < len ? make_key(x[k * VW + j], start + idx) : 0ull;
        }
    block_top_k<TB_EPT>(key, K, s_c, s_tmax, s_cnt, cand + (m * ns + s) * (size_t)K);
    if (tid == 0) {
        slab_m[m * ns + s] = mx;
        slab_s[m * ns + s] = (s_sum[0] + s_sum[1]) + (s_sum[2] + s_sum[3]);
        flag[m * ns + s] = any_bad ? (unsigned)TEV_FLAG_NONFINITE : 0u;
    }
}

// The row merge's floor pool: q = min(K, ceil(2 K / ns)) keys of each of the
// ns slab lists, q ns <= 2 K + ns keys.
constexpr int TB_POOL = 384;
static_assert(2 * TB_MAX_K + TB_MAX_SLABS <= TB_POOL && TB_POOL % 64 == 0, "the floor pool fits the wave");

// One row: the union of its slab lists (ns K <= 8192 keys, 32 per thread) and
// the row's logsumexp from the slab partials.
__global__ __launch_bounds__(TB_THREADS) void k_tb_rows(const unsigned *__restrict__ flag,
                                                        const float *__restrict__ slab_m,
                                                        const double *__restrict__ slab_s,
                                                        const uint64_t *__restrict__ cand, int ns, int K,
                                                        uint64_t *__restrict__ top, double *__restrict__ lse,
                                                        unsigned *__restrict__ row_flag) {
    constexpr int NWV = TB_THREADS / 64;
    constexpr int NK = 8192 / TB_THREADS;
    extern __shared__ __align__(16) uint64_t s_c[];   // NK * K keys, 16 of padding, a spare slot per thread
    __shared__ uint64_t s_tmax[TB_THREADS];
    __shared__ int s_cnt[2 * NWV];                   // per wave, two passes
    const int tid = threadIdx.x, lane = tid & 63;
    const size_t m = blockIdx.x;
    const int nk = ns * K;
    uint64_t key[NK];
#pragma unroll
    for (int j = 0; j < NK; j++) {
        const int i = j * TB_THREADS + tid;
        key[j] = i < nk ? cand[m * (size_t)nk + i] : 0ull;
    }
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
    // A floor for the row's K-th key: every slab list is sorted, best first,
    // so the K-th largest of a pool of each list's first q keys (any K keys of
    // the row) is at most the row's K-th key, and equals it when no list holds
    // more than q of the row's K best.  Every wave selects it from the pool's
    // keys (0 past the pool: never above a key).
    const int q = min(K, (2 * K + ns - 1) / ns);
    const int np = q * ns;                            // <= 2 K + ns <= TB_POOL
    uint64_t pv[TB_POOL / 64];
#pragma unroll
    for (int i = 0; i < TB_POOL / 64; i++) {
        const int e = i * 64 + lane, l = e / q, p = e - l * q;
        pv[i] = e < np ? cand[m * (size_t)nk + (size_t)l * K + p] : 0ull;
    }
    int frem;
    const uint64_t floor_key = (uint64_t)wave_kth_high<TB_POOL / 64>(pv, K, frem) << 32;
    block_top_k<NK>(key, K, s_c, s_tmax, s_cnt, top + m * (size_t)K, floor_key);
}

// Sets the rank of depth d (1-based) in a rank sequence packed big-endian:
// depths 1..8 in hi, 9..16 in lo, one byte each.
__device__ __forceinline__ void set_rank(uint64_t &hi, uint64_t &lo, int d, int r) {
    if (d <= 8) {
        const int sh = 8 * (8 - d);
        hi = (hi & ~(255ull << sh)) | ((uint64_t)r << sh);
    } else {
        const int sh = 8 * (16 - d);
        lo = (lo & ~(255ull << sh)) | ((uint64_t)r << sh);
    }
}

// One emitted node of a mode's search, kept for the merge across modes.
struct StreamRec {
    double key;
    uint64_t hi, lo;        // rank sequence under the mode
    int parent, token, depth, pad;
};

// Frontier slots.  Slot p belongs to node p and holds the next not yet
// emitted child of p: first its rank-0 child, then, each time that child is
// popped, the next sibling.  So a pop changes only the winner's own slot and
// the new node's slot, no slot is searched for, and the parent of a slot's
// entry is the slot's node.
//
// Keys are compared as the order-preserving 64-bit image of the f64 key
// (-0 folded into +0).  Only the high half sits in registers, one word per
// slot (lane p mod 64, register p / 64; 0 = empty); the search takes its wave
// maximum.  The rest of a slot is a record in LDS, read once per pop, so that
// the pop's arithmetic starts from one LDS round trip: the logits of the
// entry's token and of its next sibling's token, the entry's rank and depth,
// the key's low half, the logit sum of the slot node's path, the depth
// constants it needs (C_d, C_{d+1} and the rank-0 and rank-1 logits of depth
// d + 1), and the slot node's rank sequence, parent and rank.  A key is
// recomputed from the record with the arithmetic that made it, so it is the
// same f64 value.
//
// Slots whose high halves tie are ordered exactly, by every tied lane at
// once, in up to three wave maxima: the key's low half with the depth
// (shorter first) and the ranks of depths 1..4 (smaller first), then the rank
// sequence's depths 1..8, then its depths 9..16 (smaller first, as big-endian
// bytes).
__device__ __forceinline__ uint64_t heap_key(double s) { return ord64(s + 0.0); }

// Wave maximum: row maxima by in-row permutes, then row 0's into row 1 and
// row 2's into row 3 (row_bcast:15), then row 1's into row 3 (row_bcast:31),
// so lane 63 holds the maximum.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t x) {
    x = max(x, (uint32_t)wave::dpp_i<wave::kQuadXor1>((int)x));
    x = max(x, (uint32_t)wave::dpp_i<wave::kQuadXor2>((int)x));
    x = max(x, (uint32_t)wave::dpp_i<wave::kRowHalfMirror>((int)x));
    x = max(x, (uint32_t)wave::dpp_i<wave::kRowMirror>((int)x));
    x = max(x, (uint32_t)__builtin_amdgcn_update_dpp((int)x, (int)x, 0x142, 0xA, 0xF, false));
    x = max(x, (uint32_t)__builtin_amdgcn_update_dpp((int)x, (int)x, 0x143, 0xC, 0xF, false));
    return (uint32_t)__builtin_amdgcn_readlane((int)x, 63);
}

__device__ __forceinline__ uint64_t readlane_u64(uint64_t x, int l) {
    return ((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(x >> 32), l) << 32) |
           (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)x, l);
}

template <int CTRL>
__device__ __forceinline__ uint64_t dpp_u64(uint64_t x) {
    return ((uint64_t)(uint32_t)wave::dpp_i<CTRL>((int)(uint32_t)(x >> 32)) << 32) |
           (uint32_t)wave::dpp_i<CTRL>((int)(uint32_t)x);
}
__device__ __forceinline__ uint64_t umax64(uint64_t a, uint64_t b) { return a > b ? a : b; }
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t x) {
    x = umax64(x, dpp_u64<wave::kQuadXor1>(x));
    x = umax64(x, dpp_u64<wave::kQuadXor2>(x));
    x = umax64(x, dpp_u64<wave::kRowHalfMirror>(x));
    x = umax64(x, dpp_u64<wave::kRowMirror>(x));
    return umax64(umax64(readlane_u64(x, 0), readlane_u64(x, 16)), umax64(readlane_u64(x, 32), readlane_u64(x, 48)));
}

__device__ __forceinline__ double as_f64(int lo, int hi) {
    return __builtin_bit_cast(double, ((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo);
}
__device__ __forceinline__ int lo32(double x) { return (int)(uint32_t)__builtin_bit_cast(uint64_t, x); }
__device__ __forceinline__ int hi32(double x) { return (int)(uint32_t)(__builtin_bit_cast(uint64_t, x) >> 32); }

// A slot's record: {entry logit, next sibling's logit, rank | depth << 8, key
// low half}, {logit sum of the slot node's path, C_d}, {C_{d+1}, rank-0 and
// rank-1 logits of depth d + 1}, {the slot node's rank sequence: depths 1..8,
// 9..16}, {the slot node's parent, its rank | depth << 8}.
struct SlotRec {
    int4 a, b, c, h;
    int parent, rd, pad[2];
};
__device__ __forceinline__ uint64_t u64_of(int lo, int hi) { return ((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo; }

// One wave per request; SLOTS = ceil(B / 64) key words per lane.
template <int SLOTS>
__global__ __launch_bounds__(64) void k_tb_heap(const uint64_t *__restrict__ top, const double *__restrict__ lse,
                                                const unsigned *__restrict__ row_flag,
                                                const int32_t *__restrict__ root_tokens, int L, int K, int B,
                                                const float *__restrict__ log_prior, double lp_default,
                                                unsigned *__restrict__ status, int32_t *__restrict__ parents,
                                                int32_t *__restrict__ tokens, double *__restrict__ scores,
                                                StreamRec *__restrict__ stream, int32_t *__restrict__ stream_n) {
    constexpr int NLD = TB_MAX_L * TB_MAX_K / 64;     // top-K entries per lane
    __shared__ float s_tz[TB_MAX_L * TB_MAX_K];
    __shared__ int s_tt[TB_MAX_L * TB_MAX_K];
    __shared__ SlotRec s_rec[TEV_MAX_NODES + 1];     // + a scratch record for the first pop's deferred writes
    __shared__ int4 s_dt[TB_MAX_L + 2];              // per depth e: C_e, rank-0 and rank-1 logits of depth e
    const int lane = threadIdx.x, r = blockIdx.x;
    const float qnan = __builtin_nanf("");
    // the mode's log prior: every key is (logit sum - logsumexp sum) + lp
    const double lp = log_prior ? (double)log_prior[r] : lp_default;
    // every load first, then the LDS stores
    const int LK = L * K;
    uint64_t kv[NLD];
#pragma unroll
    for (int j = 0; j < NLD; j++) {
        const int i = j * 64 + lane;
        kv[j] = i < LK ? top[(size_t)r * LK + i] : 0ull;
    }
    const double lse_l = lane < L ? lse[(size_t)r * L + lane] : 0.0;
    const unsigned rf = lane < L ? row_flag[(size_t)r * L + lane] : 0u;
#pragma unroll
    for (int j = 0; j < NLD; j++) {
        const int i = j * 64 + lane;
        if (i < LK) {
            s_tz[i] = unord32((uint32_t)(kv[j] >> 32));
            s_tt[i] = (int)~(uint32_t)kv[j];
        }
    }
    const unsigned fl = __ballot(rf != 0u) != 0ull ? (unsigned)TEV_FLAG_NONFINITE : 0u;
    // lane e holds C[e] = lse_0 + ... + lse_{e-1} (summed in order; 0 past L)
    double creg = 0.0, c = 0.0;
    for (int j = 0; j < L; j++) {
        c += wave::readlane_d(lse_l, j);
        if (lane == j + 1) creg = c;
    }
    __syncthreads();
    // lane e: the rank-0 and rank-1 logits of depth e (NaN past L)
    const float zr0 = (lane >= 1 && lane <= L) ? s_tz[(lane - 1) * K] : qnan;
    const float zr1 = (lane >= 1 && lane <= L && K > 1) ? s_tz[(lane - 1) * K + 1] : qnan;
    if (lane >= 1 && lane <= L + 1) s_dt[lane] = int4{lo32(creg), hi32(creg), __float_as_int(zr0), __float_as_int(zr1)};
    if (lane == 0) status[r] = fl;
    if (fl) {
        if (stream) {
            if (lane == 0) stream_n[r] = 0;
            return;
        }
        for (int n = lane; n < B; n += 64) {
            parents[(size_t)r * B + n] = -1;
            tokens[(size_t)r * B + n] = -1;
            scores[(size_t)r * B + n] = __builtin_nan("");
        }
        return;
    }
    uint32_t fk[SLOTS];
#pragma unroll
    for (int q = 0; q < SLOTS; q++) fk[q] = 0u;
    {   // the root's slot: its rank-0 child at position 1 (none under a NaN prior)
        const float z0 = wave::readlane_f(zr0, 1), z1 = wave::readlane_f(zr1, 1);
        const double c1 = wave::readlane_d(creg, 1), c2 = wave::readlane_d(creg, 2);
        const float z02 = wave::readlane_f(zr0, 2), z12 = wave::readlane_f(zr1, 2);
        const uint64_t k = heap_key(((0.0 + (double)z0) - c1) + lp);
        if (lane == 0) {
            fk[0] = lp == lp ? (uint32_t)(k >> 32) : 0u;
            s_rec[0] = SlotRec{int4{__float_as_int(z0), __float_as_int(z1), 1 << 8, (int)(uint32_t)k},
                               int4{lo32(0.0), hi32(0.0), lo32(c1), hi32(c1)},
                               int4{lo32(c2), hi32(c2), __float_as_int(z02), __float_as_int(z12)},
                               int4{0, 0, 0, 0}, -1, 0, {0, 0}};
        }
    }
    // Two record parts wait one pop for their LDS loads: the winner's slot
    // (its next sibling's next logit) and the new node's slot (the
    // constants of depth d + 2).  Both are written after the next pop's wave
    // maximum, before it reads any record.
    int pend_p = TEV_MAX_NODES, pend_n = TEV_MAX_NODES, pend_rd = 0, pend_klo = 0;
    bool pend_ok = false;
    float pend_zc = 0.f, pend_zn2 = 0.f;
    int4 pend_dt = int4{0, 0, 0, 0};
    int n = 1;
    for (; n < B; n++) {
        // maximum of the high halves over every slot, then the slots that reach it
        uint32_t lm = fk[0];
#pragma unroll
        for (int q = 1; q < SLOTS; q++) lm = max(lm, fk[q]);
        const uint32_t m = wave_max_u32(lm);
        if (m == 0u) break;                              // the universe is exhausted
        if (lane == 0) {
            s_rec[pend_p].a = int4{__float_as_int(pend_zc), __float_as_int(pend_ok ? pend_zn2 : qnan), pend_rd, pend_klo};
            s_rec[pend_n].c = pend_dt;
        }
        uint64_t hit[SLOTS];
        int nhit = 0;
#pragma unroll
        for (int q = 0; q < SLOTS; q++) {
            hit[q] = __ballot(fk[q] == m);
            nhit += __popcll(hit[q]);
        }
        int wq = SLOTS - 1;
        uint64_t wb = hit[SLOTS - 1];
#pragma unroll
        for (int q = SLOTS - 2; q >= 0; q--) {
            wq = hit[q] ? q : wq;
            wb = hit[q] ? hit[q] : wb;
        }
        int p = wq * 64 + __ffsll((long long)wb) - 1;
        if (nhit > 1) {
            // the exact order of the tied slots' entries, each lane taking
            // the best of its own: (low half, shallower) larger, then rank
            // sequence smaller
            uint64_t b1 = 0ull, bhi = ~0ull, blo = ~0ull;
            int bq = 0;
            bool mine = false;
#pragma unroll
            for (int q = 0; q < SLOTS; q++) {
                if ((hit[q] >> lane) & 1ull) {
                    const SlotRec &R = s_rec[q * 64 + lane];
                    const int4 ra = R.a, rh = R.h;
                    const int ed = ra.z >> 8;
                    uint64_t ehi = u64_of(rh.x, rh.y), elo = u64_of(rh.z, rh.w);
                    set_rank(ehi, elo, ed, ra.z & 255);
                    // key low half, then depth and the ranks of depths 1..4 as
                    // 7-bit digits (ranks < 128), both inverted: smaller first
                    const uint32_t t4 = (uint32_t)(ehi >> 32);
                    const uint32_t dig = ((t4 >> 24) << 21) | (((t4 >> 16) & 255u) << 14) |
                                         (((t4 >> 8) & 255u) << 7) | (t4 & 255u);
                    const uint64_t k1 = ((uint64_t)(uint32_t)ra.w << 32) |
                                        ((uint32_t)(16 - ed) << 28) | (~dig & 0x0FFFFFFFu);
                    if (!mine || k1 > b1 || (k1 == b1 && (ehi < bhi || (ehi == bhi && elo < blo)))) {
                        b1 = k1;
                        bhi = ehi;
                        blo = elo;
                        bq = q;
                        mine = true;
                    }
                }
            }
            uint64_t cand = __ballot(mine);
            const uint64_t m1 = wave_max_u64(mine ? b1 : 0ull);
            cand &= __ballot(b1 == m1);
            if (__popcll(cand) > 1) {
                const bool in = (cand >> lane) & 1ull;
                const uint64_t m2 = wave_max_u64(in ? ~bhi : 0ull);
                cand &= __ballot(~bhi == m2);
                if (__popcll(cand) > 1) {
                    const bool in2 = (cand >> lane) & 1ull;
                    const uint64_t m3 = wave_max_u64(in2 ? ~blo : 0ull);
                    cand &= __ballot(~blo == m3);
                }
            }
            const int l = __ffsll((long long)cand) - 1;      // distinct entries: one lane left
            p = __builtin_amdgcn_readlane(bq, l) * 64 + l;
        }
        p = __builtin_amdgcn_readfirstlane(p);
        // the winner's record: one LDS round trip (broadcast reads)
        const SlotRec rec = s_rec[p];
        __builtin_amdgcn_sched_barrier(0);               // all four parts in flight together
        const int4 ra = rec.a, rb = rec.b, rc = rec.c;
        const float zc = __int_as_float(ra.x), zn = __int_as_float(ra.y);
        const int rd = ra.z, d = rd >> 8, rk = rd & 255;
        const double psz = as_f64(rb.x, rb.y), cd = as_f64(rb.z, rb.w), cd1 = as_f64(rc.x, rc.y);
        const float z0 = __int_as_float(rc.z), z1 = __int_as_float(rc.w);
        // for the new node's slot: the constants of depth d + 2 (clamped);
        // for the winner's slot: the logit after the next sibling (clamped)
        const int4 dt2 = s_dt[min(d + 2, L + 1)];
        const float zn2 = s_tz[(d - 1) * K + min(rk + 2, K - 1)];
        const double wsz = psz + (double)zc;
        // the winner's slot moves on to the next sibling (or empties) ...
        const uint64_t sk = heap_key(((psz + (double)zn) - cd) + lp);
        // ... and node n's slot starts with its rank-0 child (none at depth L)
        const uint64_t ck = heap_key(((wsz + (double)z0) - cd1) + lp);
        const uint32_t sk_hi = rk + 1 < K ? (uint32_t)(sk >> 32) : 0u;
        const uint32_t ck_hi = d < L ? (uint32_t)(ck >> 32) : 0u;
        const int wq2 = p >> 6, wl2 = p & 63, nq = n >> 6, nl = n & 63;
#pragma unroll
        for (int q = 0; q < SLOTS; q++) {
            if ((SLOTS == 1 || q == wq2) && lane == wl2) fk[q] = sk_hi;
            if ((SLOTS == 1 || q == nq) && lane == nl) fk[q] = ck_hi;
        }
        uint64_t nhi = u64_of(rec.h.x, rec.h.y), nlo = u64_of(rec.h.z, rec.h.w);   // node n's rank sequence
        set_rank(nhi, nlo, d, rk);
        if (lane == 0) {
            s_rec[n].a = int4{__float_as_int(z0), __float_as_int(z1), (d + 1) << 8, (int)(uint32_t)ck};
            s_rec[n].b = int4{lo32(wsz), hi32(wsz), rc.x, rc.y};
            s_rec[n].h = int4{(int)(uint32_t)nhi, (int)(uint32_t)(nhi >> 32), (int)(uint32_t)nlo, (int)(uint32_t)(nlo >> 32)};
            s_rec[n].parent = p;
            s_rec[n].rd = rd;
        }
        pend_p = p;
        pend_n = n;
        pend_zc = zn;
        pend_zn2 = zn2;
        pend_ok = rk + 2 < K;
        pend_rd = rd + 1;
        pend_klo = (int)(uint32_t)sk;
        pend_dt = dt2;
    }
    __syncthreads();
    // node i (1 <= i < n): parent and rank in its slot record; its key is
    // (logit sum of its path - C_d) + lp, as it was made when it was an entry
    if (stream) {
        // the mode's pop order, for the merge across modes
        for (int i = 1 + lane; i < n; i += 64) {
            const SlotRec e = s_rec[i];
            const int d = e.rd >> 8;
            StreamRec o;
            o.key = (as_f64(e.b.x, e.b.y) - as_f64(s_dt[d].x, s_dt[d].y)) + lp;
            o.hi = u64_of(e.h.x, e.h.y);
            o.lo = u64_of(e.h.z, e.h.w);
            o.parent = e.parent;
            o.depth = d;
            o.token = s_tt[(d - 1) * K + (e.rd & 255)];
            o.pad = 0;
            stream[(size_t)r * B + i] = o;
        }
        if (lane == 0) stream_n[r] = n;
        return;
    }
    for (int i = lane; i < B; i += 64) {
        const bool ok = i > 0 && i < n;
        const SlotRec e = s_rec[ok ? i : 0];
        const int d = max(e.rd >> 8, 1);
        parents[(size_t)r * B + i] = ok ? e.parent : -1;
        tokens[(size_t)r * B + i] = i == 0 ? (root_tokens ? root_tokens[r] : 0)
                                           : (ok ? s_tt[(d - 1) * K + (e.rd & 255)] : -1);
        scores[(size_t)r * B + i] = i == 0 ? 0.0
                                           : (ok ? (as_f64(e.b.x, e.b.y) - as_f64(s_dt[d].x, s_dt[d].y)) + lp : (double)qnan);
    }
}

// The merge across draft modes ("Multi-Future Drafting", App. B and Prop. 6).
// The merged heap pops every mode's entries in that mode's own order, and all
// entries together in one order: key, then depth, rank sequence, mode.  A
// node is created at the first pop of each distinct prefix, in that order.
// So the merge is a merge of sorted lists and a deduplication, done in
// parallel by one workgroup per request:
//   1. each entry's place in the merged order: its place in its own mode's
//      stream (already in that order) plus, for every other mode, the number
//      of that stream's entries before it (a binary search; entries compare
//      by the order-preserving bits of the key, and by depth, rank sequence
//      and mode only when the keys are equal);
//   2. canonical prefix ids, depth by depth over the entries bucketed by
//      depth: a prefix is (its parent's id, its token), inserted into an LDS
//      hash table; a mode-local parent always has a smaller depth, so its id
//      is known;
//   3. the first merged place of every prefix (LDS atomic minimum); the
//      entries at their prefix's first place are the nodes, numbered by a
//      block prefix sum in merged order; the first B - 1 form the tree.
constexpr int MG_THREADS = 1024;
constexpr int MG_N = TB_MAX_MODES * TEV_MAX_NODES;   // entries
constexpr int MG_HASH = 2 * MG_N;                    // hash slots (load <= 1/2)
constexpr int MG_ROOT = MG_HASH;                     // canonical id of the root prefix
constexpr int MG_EPT = MG_N / MG_THREADS;            // entries (and merged places) per thread

__device__ __forceinline__ double unord64(uint64_t o) {
    return __longlong_as_double((long long)(o ^ ((uint64_t)((int64_t)~o >> 63) | (1ull << 63))));
}

__global__ __launch_bounds__(MG_THREADS) void k_tb_merge(const StreamRec *__restrict__ stream,
                                                         const int32_t *__restrict__ stream_n,
                                                         const unsigned *__restrict__ mode_status,
                                                         const int32_t *__restrict__ root_tokens, int M, int B,
                                                         unsigned *__restrict__ status, int32_t *__restrict__ parents,
                                                         int32_t *__restrict__ tokens, double *__restrict__ scores) {
    __shared__ uint64_t s_pk[MG_N];                   // order-preserving bits of the key
    __shared__ uint64_t s_rhi[MG_N], s_rlo[MG_N];
    __shared__ int s_tok[MG_N];
    __shared__ int16_t s_par[MG_N], s_sidx[MG_N], s_cid[MG_N], s_pcid[MG_N], s_nid[MG_N], s_dlist[MG_N];
    __shared__ uint8_t s_dep[MG_N];
    __shared__ uint64_t s_hkey[MG_HASH];
    __shared__ int s_first[MG_HASH];
    __shared__ int s_len[TB_MAX_MODES];
    __shared__ int s_dcnt[TB_MAX_L + 1], s_doff[TB_MAX_L + 2], s_dfill[TB_MAX_L + 1];
    __shared__ int s_wsum[MG_THREADS / 64];
    __shared__ unsigned s_fl;
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, r = blockIdx.x;
    const StreamRec *st = stream + (size_t)r * M * B;
    if (tid == 0) s_fl = 0u;
    if (tid < M) s_len[tid] = stream_n[(size_t)r * M + tid];
    if (tid <= TB_MAX_L) {
        s_dcnt[tid] = 0;
        s_dfill[tid] = 0;
    }
    __syncthreads();
    if (tid < M && mode_status[(size_t)r * M + tid] != 0u) atomicOr(&s_fl, (unsigned)TEV_FLAG_NONFINITE);
    // entry e = k B + i, i in [1, len_k): mode k's i-th pop
    for (int e = tid; e < MG_N; e += MG_THREADS) {
        const int k = e / B, i = e - k * B;
        const bool ok = e < M * B && i >= 1 && i < s_len[k];
        if (ok) {
            const StreamRec x = st[e];
            s_pk[e] = ord64(x.key + 0.0);
            s_rhi[e] = x.hi;
            s_rlo[e] = x.lo;
            s_tok[e] = x.token;
            s_par[e] = (int16_t)x.parent;
            s_dep[e] = (uint8_t)x.depth;
            atomicAdd(&s_dcnt[x.depth], 1);
        } else {
            s_dep[e] = 0;
        }
    }
    for (int h = tid; h < MG_HASH; h += MG_THREADS) {
        s_hkey[h] = 0ull;
        s_first[h] = 0x7fffffff;
    }
    __syncthreads();
    const unsigned fl = s_fl;
    if (tid == 0) status[r] = fl;
    if (fl) {
        for (int i = tid; i < B; i += MG_THREADS) {
            parents[(size_t)r * B + i] = -1;
            tokens[(size_t)r * B + i] = -1;
            scores[(size_t)r * B + i] = __builtin_nan("");
        }
        return;
    }
    if (tid == 0) {
        int o = 0;
        for (int d = 0; d <= TB_MAX_L; d++) {
            s_doff[d] = o;
            o += s_dcnt[d];
        }
        s_doff[TB_MAX_L + 1] = o;
    }
    __syncthreads();
    int nent = 0;                                     // entries over all modes
#pragma unroll
    for (int k = 0; k < TB_MAX_MODES; k++) nent += k < M ? max(s_len[k] - 1, 0) : 0;
    // 1. merged places.  x before e: larger key, then shorter, then smaller
    //    rank sequence, then smaller mode (x and e in different modes).
    auto tie_before = [&](int x, int e) __attribute__((always_inline)) {
        const int dx = s_dep[x], de = s_dep[e];
        if (dx != de) return dx < de;
        const uint64_t hx = s_rhi[x], he = s_rhi[e];
        if (hx != he) return hx < he;
        const uint64_t lx = s_rlo[x], le = s_rlo[e];
        if (lx != le) return lx < le;
        return x / B < e / B;
    };
    int len[TB_MAX_MODES];
#pragma unroll
    for (int k2 = 0; k2 < TB_MAX_MODES; k2++) len[k2] = k2 < M ? s_len[k2] : 0;
    // c[t][k2]: entries 1..c of mode k2 come before the thread's t-th entry
    // (stream order is the merged order within a mode, so the predicate
    // holds on a prefix); every step loads all its probes before comparing
    int ent[MG_EPT], ek[MG_EPT];
    bool eok[MG_EPT];
    uint64_t pe[MG_EPT];
    int c[MG_EPT][TB_MAX_MODES];
#pragma unroll
    for (int t = 0; t < MG_EPT; t++) {
        const int e = tid + t * MG_THREADS, k = e / B, i = e - k * B;
        ent[t] = e;
        ek[t] = k;
        eok[t] = e < M * B && i >= 1 && i < len[min(k, TB_MAX_MODES - 1)];
        pe[t] = s_pk[e];
#pragma unroll
        for (int k2 = 0; k2 < TB_MAX_MODES; k2++) c[t][k2] = 0;
    }
#pragma unroll
    for (int step = TEV_MAX_NODES / 2; step >= 1; step >>= 1) {
        uint64_t px[MG_EPT][TB_MAX_MODES];
#pragma unroll
        for (int t = 0; t < MG_EPT; t++)
#pragma unroll
            for (int k2 = 0; k2 < TB_MAX_MODES; k2++)
                px[t][k2] = s_pk[k2 * B + min(c[t][k2] + step, max(len[k2] - 1, 0))];
#pragma unroll
        for (int t = 0; t < MG_EPT; t++)
#pragma unroll
            for (int k2 = 0; k2 < TB_MAX_MODES; k2++) {
                const int j = c[t][k2] + step;
                const bool probe = eok[t] && k2 != ek[t] && j < len[k2];
                bool take = probe && px[t][k2] > pe[t];
                if (probe && px[t][k2] == pe[t]) take = tie_before(k2 * B + j, ent[t]);
                c[t][k2] = take ? j : c[t][k2];
            }
    }
#pragma unroll
    for (int t = 0; t < MG_EPT; t++) {
        if (!eok[t]) continue;
        const int e = ent[t];
        int place = e - ek[t] * B - 1;
#pragma unroll
        for (int k2 = 0; k2 < TB_MAX_MODES; k2++) place += c[t][k2];
        s_sidx[place] = (int16_t)e;
        const int d = s_dep[e];
        s_dlist[s_doff[d] + atomicAdd(&s_dfill[d], 1)] = (int16_t)e;
    }
    __syncthreads();
    // 2. canonical prefix ids, one depth at a time
    for (int d = 1; d <= TB_MAX_L; d++) {
        const int n0 = s_doff[d], n1 = s_doff[d + 1];
        if (n0 == n1) continue;                       // uniform: the same for every thread
        for (int q = n0 + tid; q < n1; q += MG_THREADS) {
            const int e = s_dlist[q];
            const int k = e / B;
            const int pl = s_par[e];
            const int pc = pl == 0 ? MG_ROOT : s_cid[k * B + pl];
            const uint64_t key = (((uint64_t)(uint32_t)pc << 32) | (uint32_t)s_tok[e]) + 1ull;
            int h = (int)((key * 0x9E3779B97F4A7C15ull) >> 52) & (MG_HASH - 1);
            for (;;) {
                const uint64_t old = atomicCAS((unsigned long long *)&s_hkey[h], 0ull, (unsigned long long)key);
                if (old == 0ull || old == key) break;
                h = (h + 1) & (MG_HASH - 1);
            }
            s_cid[e] = (int16_t)h;
            s_pcid[e] = (int16_t)pc;
        }
        __syncthreads();
    }
    // 3. first merged place of every prefix, then the nodes in merged order
    for (int pos = tid; pos < nent; pos += MG_THREADS) atomicMin(&s_first[s_cid[s_sidx[pos]]], pos);
    __syncthreads();
    int cnt = 0;
    bool first[MG_EPT];
#pragma unroll
    for (int t = 0; t < MG_EPT; t++) {
        const int pos = tid * MG_EPT + t;
        first[t] = pos < nent && s_first[s_cid[s_sidx[pos]]] == pos;
        cnt += first[t] ? 1 : 0;
    }
    int incl = cnt;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int x = __shfl_up(incl, o);
        if (lane >= o) incl += x;
    }
    if (lane == 63) s_wsum[wv] = incl;
    __syncthreads();
    int base = incl - cnt;
    for (int w = 0; w < wv; w++) base += s_wsum[w];
    int total = 0;
#pragma unroll
    for (int w = 0; w < MG_THREADS / 64; w++) total += s_wsum[w];
#pragma unroll
    for (int t = 0; t < MG_EPT; t++) {
        const int pos = tid * MG_EPT + t;
        s_nid[pos] = (int16_t)(first[t] ? 1 + base : 0);
        base += first[t] ? 1 : 0;
    }
    __syncthreads();
#pragma unroll
    for (int t = 0; t < MG_EPT; t++) {
        const int pos = tid * MG_EPT + t;
        const int nid = s_nid[pos];
        if (nid >= 1 && nid < B) {
            const int e = s_sidx[pos];
            const int pc = s_pcid[e];
            parents[(size_t)r * B + nid] = pc == MG_ROOT ? 0 : s_nid[s_first[pc]];
            tokens[(size_t)r * B + nid] = s_tok[e];
            scores[(size_t)r * B + nid] = unord64(s_pk[e]);
        }
    }
    for (int i = tid; i < B; i += MG_THREADS) {
        if (i == 0) {
            parents[(size_t)r * B] = -1;
            tokens[(size_t)r * B] = root_tokens ? root_tokens[r] : 0;
            scores[(size_t)r * B] = 0.0;
        } else if (i > total) {                       // fewer distinct prefixes than nodes
            parents[(size_t)r * B + i] = -1;
            tokens[(size_t)r * B + i] = -1;
            scores[(size_t)r * B + i] = __builtin_nan("");
        }
    }
}

template <typename T, bool VEC>
hipError_t launch_typed(const void *z, const float *log_prior, double lp_default, const int32_t *root_tokens,
                        int R, int M, int L, int V, int K, int B, int32_t *parents, int32_t *tokens,
                        double *scores, char *ws, hipStream_t st) {
    // M draft modes: the slab, row and search passes treat each (request,
    // mode) as a request of its own; with M > 1 their searches emit streams
    // that the merge combines.
    const TreeModesWs MW = tree_modes_ws_layout(R, M, L, V, K, B);
    const TreeWs W = MW.base;
    char *b = ws + MW.base_off;
    const int G = R * M;
    const int ns = tb_slabs(V);
    unsigned *flag = (unsigned *)(b + W.flag);
    float *slab_m = (float *)(b + W.slab_m);
    double *slab_s = (double *)(b + W.slab_s);
    uint64_t *cand = (uint64_t *)(b + W.cand);
    uint64_t *top = (uint64_t *)(b + W.top);
    double *lse = (double *)(b + W.lse);
    unsigned *row_flag = (unsigned *)(b + W.row_flag);
    k_tb_slabs<T, VEC><<<dim3((unsigned)ns, (unsigned)(G * L)), TB_THREADS, ((size_t)TB_EPT * K + 16 + TB_THREADS) * 8, st>>>(
        static_cast<const T *>(z), V, ns, K, flag, slab_m, slab_s, cand);
    k_tb_rows<<<G * L, TB_THREADS, ((size_t)(8192 / TB_THREADS) * K + 16 + TB_THREADS) * 8, st>>>(flag, slab_m, slab_s, cand, ns, K,
                                                                                  top, lse, row_flag);
    unsigned *hstatus = M == 1 ? (unsigned *)(ws + MW.status) : (unsigned *)(b + W.status);
    StreamRec *strm = M == 1 ? nullptr : (StreamRec *)(ws + MW.stream);
    int32_t *strm_n = M == 1 ? nullptr : (int32_t *)(ws + MW.stream_n);
#define TB_HEAP(SL)                                                                                      \
    k_tb_heap<SL><<<G, 64, 0, st>>>(top, lse, row_flag, root_tokens, L, K, B, log_prior, lp_default, hstatus, \
                                    parents, tokens, scores, strm, strm_n)
    switch ((B + 63) / 64) {
    case 1: TB_HEAP(1); break;
    case 2: TB_HEAP(2); break;
    case 3: TB_HEAP(3); break;
    default: TB_HEAP(4); break;
    }
#undef TB_HEAP
    if (M > 1)
        k_tb_merge<<<R, MG_THREADS, 0, st>>>(strm, strm_n, hstatus, root_tokens, M, B,
                                                                      (unsigned *)(ws + MW.status), parents,
                                                                      tokens, scores);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_build_tree(const void *draft_logits, int dtype, bool vec, const float *log_prior,
                             double lp_default, const int32_t *root_tokens, int R, int M, int L, int V, int K,
                             int B, int32_t *parents, int32_t *tokens, double *scores, char *ws, hipStream_t st) {
#define TB_ARGS draft_logits, log_prior, lp_default, root_tokens, R, M, L, V, K, B, parents, tokens, scores, ws, st
    if (dtype == TEV_BF16)
        return vec ? launch_typed<uint16_t, true>(TB_ARGS) : launch_typed<uint16_t, false>(TB_ARGS);
    return vec ? launch_typed<float, true>(TB_ARGS) : launch_typed<float, false>(TB_ARGS);
#undef TB_ARGS
}

}  // namespace tev
