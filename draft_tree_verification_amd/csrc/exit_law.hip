// exit_law.hip -- the exit law and TEV's two draws on gfx950.
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
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "exit_law_dev.h"
#include "tev_internal.h"
#include "wave_ops.h"

namespace tev {
namespace {

// ----------------------------------------------------------------------------
// k_vocab.  Workgroup (x, rv): 4 / SPLIT consecutive chunks of row rv, SPLIT
// waves per chunk, wave h of a chunk on its part [h * TPW, h * TPW + TPW),
// TPW = 4096 / SPLIT tokens: lane t holds the part's elements
// k*(64*VW) + t*VW + j (coalesced 16-byte vectors).  With two waves per chunk
// (small problems: finer balance over the SIMDs) the pair agrees on the
// chunk's offset M_c through LDS (one barrier), sums its halves against it,
// and the first wave writes the chunk's partials (second barrier); with one
// wave per chunk no barrier is involved.  The row's child tokens inside a part
// are marked in a per-wave LDS bitmap whose word t belongs to lane t (EPW
// bits per lane).  Parts shorter than TPW tokens (the row's tail) take a
// masked path; the rest run without any per-element test.
// ----------------------------------------------------------------------------
template <typename T, bool VEC, int NPLV, int SPLIT>
__global__ __launch_bounds__(VOCAB_THREADS) void k_vocab(
    const T *__restrict__ logits, const int32_t *__restrict__ parents,
    const int32_t *__restrict__ tokens, int B, int V, int nc, float sL, ExitPtrs W) {
    constexpr int TPW = CHUNK / SPLIT;  // tokens per wave
    constexpr int EPW = TPW / 64;       // elements per lane
    constexpr int MW = EPW / 32;        // 32-bit child-mask words per lane
    constexpr int VW = 16 / (int)sizeof(T);
    constexpr int NV = EPW / VW;        // 16-byte vectors per lane
    constexpr int SPAN = 64 * VW;
    constexpr unsigned VMASK = (1u << VW) - 1u;
    static_assert(SPLIT == 1 || SPLIT == 2, "one or two waves per chunk");
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int c = blockIdx.x * (WAVES_PER_WG / SPLIT) + wave / SPLIT;
    const int h = wave % SPLIT;
    const int rv = blockIdx.y;
    const int r = rv / B, v = rv - r * B;
    __shared__ unsigned s_mask[WAVES_PER_WG][64 * MW];
    __shared__ float s_max[WAVES_PER_WG];
    __shared__ double s_sum[WAVES_PER_WG][2];
    __shared__ unsigned s_flag[WAVES_PER_WG];
    const bool live = c < nc;          // uniform per wave; both waves of a chunk agree
    const int c0 = c * CHUNK;
    const int h0 = c0 + h * TPW;
    const int len = live ? min(TPW, V - h0) : 0;   // <= 0: an empty half of the tail chunk
    const int32_t *par = parents + (size_t)r * B;
    const int32_t *tok = tokens + (size_t)r * B;

    // The tree arrays first (a few hundred bytes, cache-resident after the
    // first waves): the child mask below is then built while the logits are
    // still in flight.  Unconditional loads of clamped indices.
    int cpar[NPLV], ctok[NPLV];
#pragma unroll
    for (int k = 0; k < NPLV; k++) {
        const int uc = min(1 + lane + 64 * k, B - 1);
        cpar[k] = par[uc];
        ctok[k] = tok[uc];
    }
    const T *row = logits + (size_t)rv * (size_t)V + h0;
    float x[EPW];
    const bool full = len == TPW;
    if (full) {
#pragma unroll
        for (int k = 0; k < NV; k++) {
            const int idx = k * SPAN + lane * VW;
            if (VEC) {
                load16(row + idx, &x[k * VW]);
            } else {
#pragma unroll
                for (int j = 0; j < VW; j++) x[k * VW + j] = to_f32<T>(row[idx + j]);
            }
        }
    } else if (len > 0) {
        load_chunk_part<T, VEC, EPW>(row, len, lane, x);
    } else {
#pragma unroll
        for (int j = 0; j < EPW; j++) x[j] = -kInf;
    }
#pragma unroll
    for (int q = 0; q < MW; q++) s_mask[wave][MW * lane + q] = 0u;
    wave::lds_sync();
    bool dup = false;
    int mine_o[NPLV];   // half offset of child 1 + lane + 64 k, or -1
    float cval[NPLV];   // that child's logit, loaded now (behind the part's own loads)
#pragma unroll
    for (int k = 0; k < NPLV; k++) {
        // the test is evaluated outside the branch, so that the tree loads
        // cannot sink into it (a load inside the branch would wait for the
        // logits too)
        const int o = ctok[k] - h0;
        const bool hit = (1 + lane + 64 * k < B) & (cpar[k] == v) & (o >= 0) & (o < len);
        mine_o[k] = hit ? o : -1;
        // unconditional load of a valid address (the row's first logit when
        // there is no hit), in flight with the part's loads instead of costing
        // a memory round trip after the sums
        cval[k] = to_f32<T>(logits[(size_t)rv * (size_t)V + (hit ? h0 + o : 0)]);
        if (hit) {
            const int kk = o / SPAN, rem = o - kk * SPAN;
            const int bitpos = kk * VW + (rem % VW);           // 0..EPW-1 within the owner lane
            const unsigned bit = 1u << (bitpos & 31);
            const unsigned old = atomicOr(&s_mask[wave][MW * (rem / VW) + (bitpos >> 5)], bit);
            dup |= (old & bit) != 0u;
        }
    }
    wave::lds_sync();
    uint64_t mybits = s_mask[wave][MW * lane];
    if (MW == 2) mybits |= (uint64_t)s_mask[wave][MW * lane + MW - 1] << 32;
    const bool wave_has_children = __any(mybits != 0ull);

    // chunk maximum: this half's, then the pair's through LDS
    float m = x[0];
#pragma unroll
    for (int j = 1; j + 1 < EPW; j += 2) m = __builtin_elementwise_maximum(__builtin_elementwise_maximum(m, x[j]), x[j + 1]);
    m = __builtin_elementwise_maximum(m, x[EPW - 1]);
    m = wave::max_f32(m);
    float mc = m;
    if (SPLIT == 2) {
        if (lane == 0) s_max[wave] = m;
        __syncthreads();
        mc = __builtin_elementwise_maximum(s_max[wave & ~1], s_max[wave | 1]);
    }
    // Integer offset: every term is below 2, and rescaling between chunk
    // offsets is an exact power of two.
    const float Mc = floorf(mc * sL);
    double accR = 0.0, accC = 0.0;
    if (mc > -kInf) {
        if (!wave_has_children) {
            // common case: no child token of v in this half
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
    const double Rh = wave::sum_f64(accR);
    const double Ch = wave::sum_f64(accC);
    const bool any_dup = __any(dup);
    unsigned f = 0u;
    if (!(m == m) || m == kInf || isnan(Rh) || isnan(Ch)) f |= TEV_FLAG_NONFINITE;
    if (any_dup) f |= TEV_FLAG_TREE;
    if (SPLIT == 1) {
        if (lane == 0 && live) {
            const size_t o = (size_t)rv * nc + c;
            W.flags[o] = f;
            W.part_m[o] = (mc > -kInf) ? Mc : -kInf;
            W.part_r[o] = Rh;
            W.part_c[o] = Ch;
        }
    } else if (lane == 0) {
        s_sum[wave][0] = Rh;
        s_sum[wave][1] = Ch;
        s_flag[wave] = f;
    }
    // Each child token of v lies in exactly one part of v's row: that part
    // records the child's own term (the same f32 operations as the sums) and
    // the chunk offset, so the reach needs no gather of its own.
    if (wave_has_children) {
#pragma unroll
        for (int k = 0; k < NPLV; k++) {
            if (mine_o[k] >= 0) {
                const float t = (mc > -kInf) ? __builtin_amdgcn_exp2f(fmaf(cval[k], sL, -Mc)) : 0.f;
                W.cterm[(size_t)r * B + 1 + lane + 64 * k] = make_float2(t, Mc);
            }
        }
    }
    if (SPLIT == 1) return;
    __syncthreads();
    if (h == 0 && lane == 0 && live) {
        const size_t o = (size_t)rv * nc + c;
        W.flags[o] = s_flag[wave] | s_flag[wave + 1];
        W.part_m[o] = (mc > -kInf) ? Mc : -kInf;
        W.part_r[o] = s_sum[wave][0] + s_sum[wave + 1][0];
        W.part_c[o] = s_sum[wave][1] + s_sum[wave + 1][1];
    }
}

constexpr int REACH_THREADS = 1024;

template <int NB>
__global__ __launch_bounds__(REACH_THREADS) void k_reach(ReachArgs a) {
    reach_wg<NB, REACH_THREADS>(a, (int)blockIdx.x);
}

template <typename T, bool VEC>
__global__ __launch_bounds__(SAMPLE_THREADS) void k_sample(SampleArgs<T> a) {
    sample_wg<T, VEC>(a, (int)blockIdx.x, (int)blockIdx.y);
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
    const double scale = pow2_int(Mc - Mv);
    float x[EPT];
    segment_load<T, VEC>(logits + rb * (size_t)V + c0, len, lane, x);
    const uint64_t bits = segment_child_bits(parents + (size_t)r * B, tokens + (size_t)r * B, B, node,
                                             c0, len, s_mask[wave_id], lane);
    float e[EPT];
    segment_terms(x, sL, Mc, bits, e);
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

// ----------------------------------------------------------------------------
// Predraw-and-follow verification ("Where Draft Trees Lose Target Mass",
// App. A.4.1): every node draws R_v from its full target row p_v (children
// included), then the walk from the root follows the child whose token is
// R_v and stops where none is; the exit node is that node, the bonus token its
// draw.  The rows' chunk partials of the vocabulary pass serve the draws, so a
// node draw reads its row's chunk sums and one chunk.
//
// k_predraw_nodes -- grid (ceil(B / 4), n_draws, R), one wave per node draw:
//   the chunk of the draw from the running sums of (residual + child) chunk
//   sums at the row offset, then an fp64 scan of that chunk's terms (the same
//   f32 terms as the vocabulary pass) in token order.
// k_predraw_walk -- grid (ceil(n_draws / 4), R), one wave per draw: the walk,
//   one ballot over the tree per step (at most B steps).
// ----------------------------------------------------------------------------
template <typename T, bool VEC>
__global__ __launch_bounds__(256) void k_predraw_nodes(
    const T *__restrict__ logits, int B, int V, int nc, float sL, const unsigned *__restrict__ status,
    const float *__restrict__ part_m, const double *__restrict__ part_r,
    const double *__restrict__ part_c, const float *__restrict__ row_m,
    const float *__restrict__ uniforms, int n_draws, int32_t *__restrict__ node_draw) {
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int v = blockIdx.x * 4 + wave;
    const int d = blockIdx.y, r = blockIdx.z;
    if (v >= B) return;
    const size_t k = ((size_t)r * n_draws + d) * B + v;
    const size_t rb = (size_t)r * B + v;
    const unsigned st = status[r];
    const double u = (double)uniforms[k];
    const float Mv = row_m[rb];
    if (st != 0u) {
        if (lane == 0) node_draw[k] = -1;
        return;
    }
    // running sums of the full row's chunk sums, in units of 2^-M_v
    auto chunk_sum = [&](int c) -> double {
        const int cl = min(c, nc - 1);
        const float mc = part_m[rb * nc + cl];
        const double fs = (part_r[rb * nc + cl] + part_c[rb * nc + cl]) * ((mc > -kInf) ? pow2_int(mc - Mv) : 0.0);
        return c < nc ? fs : 0.0;
    };
    double total = 0.0;
    for (int c0 = 0; c0 < nc; c0 += 64) total += wave::sum_f64(chunk_sum(c0 + lane));
    const double t = u * total;
    // chunk: the smallest c with t < W_c (W the running sums)
    int cc = 0;
    double carry = 0.0;
    for (int c0 = 0; c0 < nc; c0 += 64) {
        const double fs = chunk_sum(c0 + lane);
        const double incl = carry + wave::incl_scan_f64(fs, lane);
        cc += wave::sum_i32((c0 + lane < nc && incl <= t) ? 1 : 0);
        carry = wave::readlane_d(incl, 63);
    }
    if (cc >= nc) {   // rounding left no bin: the last chunk with positive mass
        int best = -1;
        for (int c = lane; c < nc; c += 64)
            if (chunk_sum(c) > 0.0) best = max(best, c);
        cc = max(wave::max_i32(best), 0);
    }
    double before = 0.0;
    for (int c0 = 0; c0 < cc; c0 += 64) {
        const int c = c0 + lane;
        before += wave::sum_f64(c < cc ? chunk_sum(c) : 0.0);
    }
    const int c0 = cc * CHUNK;
    const int len = min(CHUNK, V - c0);
    const float Mc = part_m[rb * nc + cc];
    // offsets are integers with Mc <= Mv: the rescale is an exact power of two
    const double target = __builtin_ldexp(t - before, (int)fminf(Mv - Mc, 2000.f));
    float x[EPT];
    segment_load<T, VEC>(logits + rb * (size_t)V + c0, len, lane, x);
    float e[EPT];
    segment_terms(x, sL, Mc, 0ull, e);
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
    if (lane == 0) node_draw[k] = c0 + below;
}

__global__ __launch_bounds__(256) void k_predraw_walk(
    const int32_t *__restrict__ parents, const int32_t *__restrict__ tokens, int B,
    const unsigned *__restrict__ status, const int32_t *__restrict__ node_draw, int n_draws,
    int32_t *__restrict__ exit_node, int32_t *__restrict__ bonus_token) {
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int d = blockIdx.x * 4 + wave, r = blockIdx.y;
    if (d >= n_draws) return;
    const size_t kd = (size_t)r * n_draws + d;
    const int32_t *nd = node_draw + kd * B;
    int cp[NPL], ct[NPL], dr[NPL];
#pragma unroll
    for (int q = 0; q < NPL; q++) {
        const int uq = min(lane + 64 * q, B - 1);
        cp[q] = parents[(size_t)r * B + uq];
        ct[q] = tokens[(size_t)r * B + uq];
        dr[q] = nd[uq];
    }
    if (status[r] != 0u) {
        if (lane == 0) { exit_node[kd] = -1; bonus_token[kd] = -1; }
        return;
    }
    int v = 0, dv = -1;
    for (int step = 0; step < B; step++) {   // a walk visits at most B nodes
        const int q = v >> 6;                 // uniform
        int val = dr[0];
#pragma unroll
        for (int qq = 1; qq < NPL; qq++) val = (q == qq) ? dr[qq] : val;
        dv = __builtin_amdgcn_readlane(val, v & 63);
        int next = -1;
#pragma unroll
        for (int qq = 0; qq < NPL; qq++) {
            const int uq = lane + 64 * qq;
            const bool hit = (uq < B) & (uq > 0) & (cp[qq] == v) & (ct[qq] == dv);
            const unsigned long long bal = __ballot(hit);
            if (next < 0 && bal != 0ull) next = 64 * qq + (int)__builtin_ctzll(bal);
        }
        if (next < 0) break;
        v = next;
    }
    if (lane == 0) {
        exit_node[kd] = v;
        bonus_token[kd] = dv;
    }
}

template <typename T, bool VEC>
hipError_t predraw_impl(const T *logits, const int32_t *parents, const int32_t *tokens, int R,
                        int B, int V, float sL, const char *ws, const float *uniforms,
                        int n_draws, int32_t *node_draw, int32_t *exit_node, int32_t *bonus,
                        hipStream_t st) {
    const ExitWs L = exit_ws_layout(R, B, V);
    const int nc = n_chunks(V);
    const unsigned *status = (const unsigned *)(ws + L.status);
    k_predraw_nodes<T, VEC><<<dim3((B + 3) / 4, n_draws, R), 256, 0, st>>>(
        logits, B, V, nc, sL, status, (const float *)(ws + L.part_m),
        (const double *)(ws + L.part_r), (const double *)(ws + L.part_c),
        (const float *)(ws + L.row_m), uniforms, n_draws, node_draw);
    k_predraw_walk<<<dim3((n_draws + 3) / 4, R), 256, 0, st>>>(parents, tokens, B, status, node_draw,
                                                                  n_draws, exit_node, bonus);
    return hipGetLastError();
}

template <typename T, bool VEC>
void vocab_impl(const T *logits, const int32_t *parents, const int32_t *tokens, int R, int B,
                int V, float sL, char *ws, hipStream_t st) {
    const int nc = n_chunks(V);
    const ExitPtrs W = exit_ptrs(ws, R, B, V);
    // Two waves per chunk while the chunks alone would leave the SIMDs with a
    // few waves each (an uneven last round), one wave per chunk otherwise.
    const bool split = (long)R * B * nc < 4L * 1024;
#define TEV_VOCAB(NP, SP)                                                                          \
    k_vocab<T, VEC, NP, SP><<<dim3((nc + WAVES_PER_WG / SP - 1) / (WAVES_PER_WG / SP), R * B),     \
                              VOCAB_THREADS, 0, st>>>(logits, parents, tokens, B, V, nc, sL, W)
    if (B <= 65) {
        if (split) TEV_VOCAB(1, 2); else TEV_VOCAB(1, 1);
    } else {
        if (split) TEV_VOCAB(NPL, 2); else TEV_VOCAB(NPL, 1);
    }
#undef TEV_VOCAB
}

void reach_impl(const int32_t *parents, const int32_t *tokens, int R, int B, int V, float sL,
                float *rho, float *reach, float *w, float *cov, char *ws, hipStream_t st) {
    const ReachArgs a{parents, tokens, B, V, n_chunks(V), sL, exit_ptrs(ws, R, B, V), rho, reach, w, cov};
    switch (reach_batches(B, REACH_THREADS)) {
        case 1: k_reach<1><<<dim3(R), REACH_THREADS, 0, st>>>(a); break;
        case 2: k_reach<2><<<dim3(R), REACH_THREADS, 0, st>>>(a); break;
        case 3: k_reach<3><<<dim3(R), REACH_THREADS, 0, st>>>(a); break;
        default: k_reach<4><<<dim3(R), REACH_THREADS, 0, st>>>(a); break;
    }
}

template <typename T, bool VEC>
hipError_t sample_impl(const T *logits, const int32_t *parents, const int32_t *tokens, int R,
                       int B, int V, float sL, const char *ws, const float *uniforms,
                       int n_draws, int32_t *exit_node, int32_t *bonus, hipStream_t st) {
    const SampleArgs<T> a = sample_args(logits, parents, tokens, R, B, V, sL, ws, uniforms, n_draws,
                                        exit_node, bonus);
    k_sample<T, VEC><<<dim3(n_draws, R), SAMPLE_THREADS, 0, st>>>(a);
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

hipError_t launch_vocab(const void *logits, int dtype, bool vec, const int32_t *parents,
                        const int32_t *tokens, int R, int B, int V, float sL, char *ws,
                        hipStream_t st) {
    if (dtype == TEV_BF16) {
        const uint16_t *p = (const uint16_t *)logits;
        if (vec) vocab_impl<uint16_t, true>(p, parents, tokens, R, B, V, sL, ws, st);
        else vocab_impl<uint16_t, false>(p, parents, tokens, R, B, V, sL, ws, st);
    } else {
        const float *p = (const float *)logits;
        if (vec) vocab_impl<float, true>(p, parents, tokens, R, B, V, sL, ws, st);
        else vocab_impl<float, false>(p, parents, tokens, R, B, V, sL, ws, st);
    }
    return hipGetLastError();
}

hipError_t launch_exit_law(const void *logits, int dtype, bool vec, const int32_t *parents,
                           const int32_t *tokens, int R, int B, int V, float sL, float *rho,
                           float *reach, float *exit_mass, float *coverage, char *ws,
                           hipStream_t st) {
    const hipError_t e = launch_vocab(logits, dtype, vec, parents, tokens, R, B, V, sL, ws, st);
    if (e != hipSuccess) return e;
    reach_impl(parents, tokens, R, B, V, sL, rho, reach, exit_mass, coverage, ws, st);
    return hipGetLastError();
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

hipError_t launch_predraw(const void *logits, int dtype, bool vec, const int32_t *parents,
                          const int32_t *tokens, int R, int B, int V, float sL, const char *ws,
                          const float *uniforms, int n_draws, int32_t *node_draw,
                          int32_t *exit_node, int32_t *bonus_token, hipStream_t st) {
    if (dtype == TEV_BF16) {
        const uint16_t *p = (const uint16_t *)logits;
        return vec ? predraw_impl<uint16_t, true>(p, parents, tokens, R, B, V, sL, ws, uniforms, n_draws, node_draw, exit_node, bonus_token, st)
                   : predraw_impl<uint16_t, false>(p, parents, tokens, R, B, V, sL, ws, uniforms, n_draws, node_draw, exit_node, bonus_token, st);
    }
    const float *p = (const float *)logits;
    return vec ? predraw_impl<float, true>(p, parents, tokens, R, B, V, sL, ws, uniforms, n_draws, node_draw, exit_node, bonus_token, st)
               : predraw_impl<float, false>(p, parents, tokens, R, B, V, sL, ws, uniforms, n_draws, node_draw, exit_node, bonus_token, st);
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
