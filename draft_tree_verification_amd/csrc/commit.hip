// commit.hip -- KV-cache commit after verification on gfx950.
//
// What is computed ("CAST: Cost-Aware Speculative Trees from One-Pass Block
// Drafters", App. C "Packed verification": after acceptance only the root
// path of the accepted node keeps its cache entries, compacted after the
// prefix; "Where Draft Trees Lose Target Mass", the verifier stage's cache
// commit): with the exit node V of request r and its root path
// 0 = a_0, a_1, ..., a_A = V (A = depth(V) accepted drafted tokens), every
// layer and kv head moves cache row P + a_d to row P + d, d = 0..A, in place.
// Rows 0..P-1 (the prefix) and rows past P + A are left as they are; the new
// cache length is P + A + 1.
//
// k_commit_kv -- grid (L * R * Hkv), 256 threads: the parents go to LDS and
// one lane walks the path up from V; the rows of K and V are then moved in
// batches of increasing d, each batch staged in LDS (16-byte chunks) before
// any of its writes, so no write can overtake a read of the same row
// (a_d >= d, and a_d' = d for some d' < d is possible).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "tev_internal.h"

namespace tev {
namespace {

typedef uint32_t u32x4c __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(256) void k_commit_kv(char *__restrict__ k, char *__restrict__ v,
                                                   const int32_t *__restrict__ parents,
                                                   const int32_t *__restrict__ exit_node, int R,
                                                   int B, int Hkv, int P, int row_bytes,
                                                   int32_t *__restrict__ new_len) {
    __shared__ int s_par[TEV_MAX_NODES];
    __shared__ int s_path[TEV_MAX_NODES];
    __shared__ int s_len;
    constexpr int STAGE = 2048;                        // 16-byte chunks staged per batch (32 KB)
    __shared__ __attribute__((aligned(16))) u32x4c s_rows[STAGE];
    const int tid = threadIdx.x;
    const int b = blockIdx.x;
    const int g = b % Hkv;
    const int r = (b / Hkv) % R;
    const int l = b / (Hkv * R);
    const int32_t *par = parents + (size_t)r * B;
    if (tid < B) s_par[tid] = par[tid];                // B <= 256 = blockDim.x
    __syncthreads();
    if (tid == 0) {
        // walk up from the exit node; a path longer than B or an index out of
        // range means an invalid tree or exit node: nothing is moved
        int vtx = exit_node[r], n = 0;
        bool ok = vtx >= 0 && vtx < B;
        while (ok && vtx != 0) {
            s_path[n++] = vtx;
            const int p = s_par[vtx];
            ok = n < B && p >= 0 && p < vtx;
            vtx = p;
        }
        if (ok) s_path[n++] = 0;   // the root
        s_len = ok ? n : -1;       // path length A + 1, rows listed from V up to the root
        if (ok && l == 0 && g == 0) new_len[r] = P + n;
        if (!ok && l == 0 && g == 0) new_len[r] = -1;
    }
    __syncthreads();
    const int n = s_len;
    if (n <= 0) return;
    const int cpr = row_bytes / 16;                    // 16-byte chunks per row
    const size_t head = (((size_t)l * R + r) * Hkv + g) * (size_t)(P + B) * row_bytes;
    char *kh = k + head, *vh = v + head;
    // Batches of rows d in [d0, d1), increasing: within a batch every read is
    // staged before any write; across batches a later read (row a_d', d' >= d1)
    // never meets an earlier write (rows P + d, d < d1), and a later write
    // (row P + d'', d'' >= d1) comes after the earlier batch's reads finished.
    const int rows_per_batch = STAGE / (2 * cpr);
    for (int d0 = 0; d0 < n; d0 += rows_per_batch) {
        const int nb = min(rows_per_batch, n - d0);
        const int items = 2 * nb * cpr;                // K and V chunks of this batch's rows
        for (int it = tid; it < items; it += 256) {
            const int which = it / (nb * cpr), rest = it - which * nb * cpr;
            const int d = d0 + rest / cpr, c = rest % cpr;
            const int src = P + s_path[n - 1 - d];     // row a_d sits at path slot n - 1 - d
            const char *base = which ? vh : kh;
            s_rows[it] = *reinterpret_cast<const u32x4c *>(base + (size_t)src * row_bytes + c * 16);
        }
        __syncthreads();
        for (int it = tid; it < items; it += 256) {
            const int which = it / (nb * cpr), rest = it - which * nb * cpr;
            const int d = d0 + rest / cpr, c = rest % cpr;
            char *base = which ? vh : kh;
            *reinterpret_cast<u32x4c *>(base + (size_t)(P + d) * row_bytes + c * 16) = s_rows[it];
        }
        __syncthreads();
    }
}

}  // namespace

hipError_t launch_commit_kv(void *k, void *v, int dtype, const int32_t *parents,
                            const int32_t *exit_node, int R, int B, int L, int Hkv, int D, int P,
                            int32_t *new_len, hipStream_t st) {
    const int row_bytes = D * (dtype == TEV_BF16 ? 2 : 4);
    k_commit_kv<<<dim3((unsigned)(L * R * Hkv)), 256, 0, st>>>((char *)k, (char *)v, parents, exit_node,
                                                               R, B, Hkv, P, row_bytes, new_len);
    return hipGetLastError();
}

}  // namespace tev
