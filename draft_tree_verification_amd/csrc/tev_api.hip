// tev_api.hip -- host side of the C ABI declared in include/tev.h: argument
// checks, workspace sizing and kernel dispatch.  Nothing here allocates or
// synchronises except the calls the header marks synchronous.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <mutex>

#include "exit_loss.h"
#include "tev_internal.h"
#include "tree_build.h"

using namespace tev;

namespace {

constexpr long long kMaxV = 1LL << 26;        // 67M tokens per row
constexpr long long kMaxRows = 1LL << 16;      // R * B (grid.y of the vocabulary pass)

bool dtype_ok(int dtype) { return dtype == TEV_F32 || dtype == TEV_BF16; }
size_t esize(int dtype) { return dtype == TEV_BF16 ? 2 : 4; }

tev_status check_exit_shape(int R, int B, int V) {
    if (R < 1 || B < 1 || V < 1) return TEV_ERR_SHAPE;
    if (B > TEV_MAX_NODES || V > kMaxV || (long long)R * B > kMaxRows) return TEV_ERR_SHAPE;
    return TEV_OK;
}

bool vec_ok(const void *logits, int dtype, int V) {
    return ((uintptr_t)logits % 16 == 0) && (((size_t)V * esize(dtype)) % 16 == 0);
}

float log2e_scale(float inv_temperature) {
    return (float)((double)inv_temperature * 1.4426950408889634);
}

bool tree_shape_ok(int R, int M, int L, int V, int K) {
    if (R < 1 || M < 1 || M > TB_MAX_MODES || L < 1 || L > TB_MAX_L || V < 1 || K < 1 || K > TB_MAX_K ||
        K > V)
        return false;
    const long long ns = tb_slabs(V);
    return ns <= TB_MAX_SLABS && ns * K <= 8192 && (long long)R * M * L <= 65535;
}
// K + K^2 + ... + K^L, capped once it reaches `cap`
long long universe_size(int K, int L, long long cap) {
    long long u = 0, pw = 1;
    for (int d = 1; d <= L && u < cap; d++) {
        pw *= K;
        u += pw;
    }
    return u;
}

tev_status hip_status(hipError_t e) { return e == hipSuccess ? TEV_OK : TEV_ERR_HIP; }

// The attention kernels address one head's K / V extent, (P + B) rows of D
// elements, with 32-bit byte offsets (buffer resources): it must stay below 2^31.
bool kv_extent_ok(int P, int B, int D, int dtype) {
    return ((long long)P + B) * D * (long long)esize(dtype) < (1LL << 31);
}

// Device scratch of tev_verify_round_noalloc: one array per GPU the library
// runs on, held until the process ends.  In host code `scratch` names a host-
// side stand-in, never the device memory: kernels and copies receive the
// address hipGetSymbolAddress returns for the current device.
static __device__ __align__(256) unsigned char scratch[TEV_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices] = {};

// The scratch array's device address on the current device, looked up once
// per device (with that device current) and kept.  NULL on a HIP error.
void *scratch_on_current_device() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return nullptr;
        g_scratch_ptr[dev] = ptr;
    }
    return g_scratch_ptr[dev];
}

}  // namespace

extern "C" {

const char *tev_status_str(int s) {
    switch (s) {
        case TEV_OK: return "ok";
        case TEV_ERR_NULL: return "null pointer argument";
        case TEV_ERR_SHAPE: return "size out of range or inconsistent";
        case TEV_ERR_DTYPE: return "unsupported dtype";
        case TEV_ERR_TREE: return "invalid tree (parents/tokens)";
        case TEV_ERR_WORKSPACE: return "workspace too small";
        case TEV_ERR_UNSUPPORTED: return "unsupported configuration";
        case TEV_ERR_HIP: return "HIP runtime error";
        case TEV_ERR_VALUE: return "scalar argument not finite or not positive";
        default: return "unknown status";
    }
}

size_t tev_exit_law_workspace_bytes(int R, int B, int V) {
    if (check_exit_shape(R, B, V) != TEV_OK) return 0;
    return exit_ws_layout(R, B, V).total;
}

tev_status tev_exit_law(const void *logits, int dtype, const int32_t *parents,
                        const int32_t *tokens, int R, int B, int V, float inv_temperature,
                        float *rho, float *reach, float *exit_mass, float *coverage,
                        void *workspace, size_t workspace_bytes, void *stream) {
    if (!logits || !parents || !tokens || !rho || !reach || !exit_mass || !coverage || !workspace)
        return TEV_ERR_NULL;
    if (!dtype_ok(dtype)) return TEV_ERR_DTYPE;
    tev_status s = check_exit_shape(R, B, V);
    if (s != TEV_OK) return s;
    if (!(inv_temperature > 0.f) || !isfinite(inv_temperature)) return TEV_ERR_VALUE;
    if (workspace_bytes < exit_ws_layout(R, B, V).total) return TEV_ERR_WORKSPACE;
    return hip_status(launch_exit_law(logits, dtype, vec_ok(logits, dtype, V), parents, tokens, R,
                                      B, V, log2e_scale(inv_temperature), rho, reach, exit_mass,
                                      coverage, (char *)workspace, (hipStream_t)stream));
}

tev_status tev_sample(const void *logits, int dtype, const int32_t *parents,
                      const int32_t *tokens, int R, int B, int V, float inv_temperature,
                      const void *workspace, size_t workspace_bytes, const float *uniforms,
                      int n_draws, int32_t *exit_node, int32_t *bonus_token, void *stream) {
    if (!logits || !parents || !tokens || !workspace || !uniforms || !exit_node || !bonus_token)
        return TEV_ERR_NULL;
    if (!dtype_ok(dtype)) return TEV_ERR_DTYPE;
    tev_status s = check_exit_shape(R, B, V);
    if (s != TEV_OK) return s;
    if (n_draws < 1 || n_draws > 65535) return TEV_ERR_SHAPE;
    if (!(inv_temperature > 0.f) || !isfinite(inv_temperature)) return TEV_ERR_VALUE;
    if (workspace_bytes < exit_ws_layout(R, B, V).total) return TEV_ERR_WORKSPACE;
    return hip_status(launch_sample(logits, dtype, vec_ok(logits, dtype, V), parents, tokens, R, B,
                                    V, log2e_scale(inv_temperature), (const char *)workspace,
                                    uniforms, n_draws, exit_node, bonus_token,
                                    (hipStream_t)stream));
}

tev_status tev_predraw(const void *logits, int dtype, const int32_t *parents,
                       const int32_t *tokens, int R, int B, int V, float inv_temperature,
                       const void *workspace, size_t workspace_bytes, const float *uniforms,
                       int n_draws, int32_t *node_draw, int32_t *exit_node,
                       int32_t *bonus_token, void *stream) {
    if (!logits || !parents || !tokens || !workspace || !uniforms || !node_draw || !exit_node ||
        !bonus_token)
        return TEV_ERR_NULL;
    if (!dtype_ok(dtype)) return TEV_ERR_DTYPE;
    tev_status s = check_exit_shape(R, B, V);
    if (s != TEV_OK) return s;
    if (R > 65535 || n_draws < 1 || n_draws > 65535) return TEV_ERR_SHAPE;
    if (!(inv_temperature > 0.f) || !isfinite(inv_temperature)) return TEV_ERR_VALUE;
    if (workspace_bytes < exit_ws_layout(R, B, V).total) return TEV_ERR_WORKSPACE;
    return hip_status(launch_predraw(logits, dtype, vec_ok(logits, dtype, V), parents, tokens, R, B,
                                     V, log2e_scale(inv_temperature), (const char *)workspace,
                                     uniforms, n_draws, node_draw, exit_node, bonus_token,
                                     (hipStream_t)stream));
}

tev_status tev_commit_kv(void *k, void *v, int dtype, const int32_t *parents,
                         const int32_t *exit_node, int R, int B, int L, int Hkv, int D, int P,
                         int32_t *new_len, void *stream) {
    if (!k || !v || !parents || !exit_node || !new_len) return TEV_ERR_NULL;
    if (!dtype_ok(dtype)) return TEV_ERR_DTYPE;
    if (R < 1 || B < 1 || B > TEV_MAX_NODES || L < 1 || Hkv < 1 || P < 0) return TEV_ERR_SHAPE;
    if ((long long)L * R * Hkv > 0x7fffffffLL) return TEV_ERR_SHAPE;
    if (D != 64 && D != 128) return TEV_ERR_UNSUPPORTED;
    if ((uintptr_t)k % 16 || (uintptr_t)v % 16) return TEV_ERR_UNSUPPORTED;
    return hip_status(launch_commit_kv(k, v, dtype, parents, exit_node, R, B, L, Hkv, D, P, new_len,
                                       (hipStream_t)stream));
}

size_t tev_exit_loss_workspace_bytes(int R, int B, int H, int V) {
    if (R < 1 || B < 1 || B > TEV_MAX_NODES || H < 1 || H > LOSS_MAX_H || V < 1 || V > kMaxV)
        return 0;
    if ((long long)R * H > 65535) return 0;
    return loss_ws_layout(R, B, H, V).total;
}

tev_status tev_exit_loss(const void *draft_logits, int dtype, const int32_t *parents,
                         const int32_t *tokens, const float *weights, int R, int B, int H, int V,
                         float *loss, float *row_lse, float *row_weight, float *grad,
                         void *workspace, size_t workspace_bytes, void *stream) {
    if (!draft_logits || !parents || !tokens || !weights || !loss || !row_lse || !row_weight ||
        !workspace)
        return TEV_ERR_NULL;
    if (!dtype_ok(dtype)) return TEV_ERR_DTYPE;
    const size_t need = tev_exit_loss_workspace_bytes(R, B, H, V);
    if (need == 0) return TEV_ERR_SHAPE;
    if (workspace_bytes < need) return TEV_ERR_WORKSPACE;
    const bool vec = vec_ok(draft_logits, dtype, V) && ((uintptr_t)grad % 16 == 0);
    return hip_status(launch_exit_loss(draft_logits, dtype, vec, parents, tokens, weights, R, B, H, V,
                                       loss, row_lse, row_weight, grad, (char *)workspace,
                                       (hipStream_t)stream));
}


size_t tev_build_tree_workspace_bytes(int R, int L, int V, int K) {
    if (!tree_shape_ok(R, 1, L, V, K)) return 0;
    return tree_modes_ws_layout(R, 1, L, V, K, 0).total;
}

tev_status tev_build_tree(const void *draft_logits, int dtype, const int32_t *root_tokens, int R,
                          int L, int V, int K, int B, int32_t *parents, int32_t *tokens,
                          double *scores, void *workspace, size_t workspace_bytes, void *stream) {
    if (!draft_logits || !parents || !tokens || !scores || !workspace) return TEV_ERR_NULL;
    if (!dtype_ok(dtype)) return TEV_ERR_DTYPE;
    const size_t need = tev_build_tree_workspace_bytes(R, L, V, K);
    if (need == 0 || B < 1 || B > TEV_MAX_NODES) return TEV_ERR_SHAPE;
    if (universe_size(K, L, B) < B - 1) return TEV_ERR_SHAPE;   // the universe must hold B - 1 prefixes
    if (workspace_bytes < need) return TEV_ERR_WORKSPACE;
    return hip_status(launch_build_tree(draft_logits, dtype, vec_ok(draft_logits, dtype, V), nullptr, 0.0,
                                        root_tokens, R, 1, L, V, K, B, parents, tokens, scores,
                                        (char *)workspace, (hipStream_t)stream));
}

size_t tev_build_tree_modes_workspace_bytes(int R, int M, int L, int V, int K, int B) {
    if (!tree_shape_ok(R, M, L, V, K) || B < 1 || B > TEV_MAX_NODES) return 0;
    return tree_modes_ws_layout(R, M, L, V, K, B).total;
}

tev_status tev_build_tree_modes(const void *draft_logits, int dtype, const float *log_prior,
                                const int32_t *root_tokens, int R, int M, int L, int V, int K, int B,
                                int32_t *parents, int32_t *tokens, double *scores, void *workspace,
                                size_t workspace_bytes, void *stream) {
    if (!draft_logits || !parents || !tokens || !scores || !workspace) return TEV_ERR_NULL;
    if (!dtype_ok(dtype)) return TEV_ERR_DTYPE;
    const size_t need = tev_build_tree_modes_workspace_bytes(R, M, L, V, K, B);
    if (need == 0) return TEV_ERR_SHAPE;
    if ((long long)M * universe_size(K, L, B) < B - 1) return TEV_ERR_SHAPE;
    if (workspace_bytes < need) return TEV_ERR_WORKSPACE;
    // uniform prior: log(1 / M), the same double the host library computes
    const double lp_default = M == 1 ? 0.0 : -log((double)M);
    return hip_status(launch_build_tree(draft_logits, dtype, vec_ok(draft_logits, dtype, V), log_prior,
                                        lp_default, root_tokens, R, M, L, V, K, B, parents, tokens, scores,
                                        (char *)workspace, (hipStream_t)stream));
}

size_t tev_tree_attn_workspace_bytes(int R, int B, int Hq, int Hkv, int D, int P) {
    if (R < 1 || B < 1 || B > TEV_MAX_NODES || Hq < 1 || Hkv < 1 || Hq % Hkv || P < 0) return 0;
    if (D != 64 && D != 128) return 0;
    return attn_ws_layout(R, B, Hq, Hkv, D, P).total;
}

tev_status tev_tree_attn(const void *q, const void *k, const void *v, int dtype,
                         const int32_t *parents, int R, int B, int Hq, int Hkv, int D, int P,
                         float scale, float *out, void *workspace, size_t workspace_bytes,
                         void *stream) {
    if (!q || !k || !v || !parents || !out || !workspace) return TEV_ERR_NULL;
    if (!dtype_ok(dtype)) return TEV_ERR_DTYPE;
    if (R < 1 || B < 1 || B > TEV_MAX_NODES || Hq < 1 || Hkv < 1 || P < 0) return TEV_ERR_SHAPE;
    if (Hq % Hkv) return TEV_ERR_SHAPE;
    if ((long long)R * Hkv > 65535) return TEV_ERR_SHAPE;
    if (D != 64 && D != 128) return TEV_ERR_UNSUPPORTED;
    if (!kv_extent_ok(P, B, D, dtype)) return TEV_ERR_SHAPE;
    if (!(scale > 0.f) || !isfinite(scale)) return TEV_ERR_VALUE;
    if (dtype == TEV_BF16 && (((uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)out) % 16))
        return TEV_ERR_UNSUPPORTED;
    if (workspace_bytes < attn_ws_layout(R, B, Hq, Hkv, D, P).total) return TEV_ERR_WORKSPACE;
    return hip_status(launch_tree_attn(q, k, v, dtype, parents, R, B, Hq, Hkv, D, P, scale, out,
                                       (char *)workspace, (hipStream_t)stream));
}

size_t tev_verify_round_workspace_bytes(int R, int B, int V, int Hq, int Hkv, int D, int P) {
    if (check_exit_shape(R, B, V) != TEV_OK) return 0;
    if (Hq < 1 || Hkv < 1 || Hq % Hkv || P < 0 || (D != 64 && D != 128)) return 0;
    return round_ws_layout(R, B, V, Hq, Hkv, D, P).total;
}

tev_status tev_verify_round_timed(const void *q, const void *k, const void *v, const void *logits,
                            int dtype, const int32_t *parents, const int32_t *tokens, int R, int B,
                            int V, int Hq, int Hkv, int D, int P, float scale,
                            float inv_temperature, const float *uniforms, int n_draws,
                            float *attn_out, float *rho, float *reach, float *exit_mass,
                            float *coverage, int32_t *exit_node, int32_t *bonus_token,
                                  void *workspace, size_t workspace_bytes, void *stream,
                                  void *const *events) {
    if (!q || !k || !v || !logits || !parents || !tokens || !uniforms || !attn_out || !rho ||
        !reach || !exit_mass || !coverage || !exit_node || !bonus_token || !workspace)
        return TEV_ERR_NULL;
    if (!dtype_ok(dtype)) return TEV_ERR_DTYPE;
    tev_status s = check_exit_shape(R, B, V);
    if (s != TEV_OK) return s;
    if (Hq < 1 || Hkv < 1 || P < 0 || Hq % Hkv) return TEV_ERR_SHAPE;
    if ((long long)R * Hkv > 65535) return TEV_ERR_SHAPE;
    if (n_draws < 1 || n_draws > 65535) return TEV_ERR_SHAPE;
    if (D != 64 && D != 128) return TEV_ERR_UNSUPPORTED;
    if (!kv_extent_ok(P, B, D, dtype)) return TEV_ERR_SHAPE;
    if (!(scale > 0.f) || !isfinite(scale)) return TEV_ERR_VALUE;
    if (!(inv_temperature > 0.f) || !isfinite(inv_temperature)) return TEV_ERR_VALUE;
    if (dtype == TEV_BF16 &&
        (((uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)attn_out) % 16))
        return TEV_ERR_UNSUPPORTED;
    if (workspace_bytes < round_ws_layout(R, B, V, Hq, Hkv, D, P).total) return TEV_ERR_WORKSPACE;
    return hip_status(launch_round(q, k, v, logits, dtype, vec_ok(logits, dtype, V), parents, tokens,
                                   R, B, V, Hq, Hkv, D, P, scale, log2e_scale(inv_temperature),
                                   uniforms, n_draws, attn_out, rho, reach, exit_mass, coverage,
                                   exit_node, bonus_token, (char *)workspace, (hipStream_t)stream,
                                   events));
}

tev_status tev_verify_round(const void *q, const void *k, const void *v, const void *logits,
                            int dtype, const int32_t *parents, const int32_t *tokens, int R, int B,
                            int V, int Hq, int Hkv, int D, int P, float scale,
                            float inv_temperature, const float *uniforms, int n_draws,
                            float *attn_out, float *rho, float *reach, float *exit_mass,
                            float *coverage, int32_t *exit_node, int32_t *bonus_token,
                            void *workspace, size_t workspace_bytes, void *stream) {
    return tev_verify_round_timed(q, k, v, logits, dtype, parents, tokens, R, B, V, Hq, Hkv, D, P,
                                  scale, inv_temperature, uniforms, n_draws, attn_out, rho, reach,
                                  exit_mass, coverage, exit_node, bonus_token, workspace,
                                  workspace_bytes, stream, nullptr);
}

tev_status tev_verify_round_noalloc(const void *q, const void *k, const void *v,
                                    const void *logits, int dtype, const int32_t *parents,
                                    const int32_t *tokens, int R, int B, int V, int Hq, int Hkv,
                                    int D, int P, float scale, float inv_temperature,
                                    const float *uniforms, int n_draws, float *attn_out, float *rho,
                                    float *reach, float *exit_mass, float *coverage,
                                    int32_t *exit_node, int32_t *bonus_token, void *stream) {
    if (!q || !k || !v || !logits || !parents || !tokens || !uniforms || !attn_out || !rho ||
        !reach || !exit_mass || !coverage || !exit_node || !bonus_token)
        return TEV_ERR_NULL;
    const size_t need = tev_verify_round_workspace_bytes(R, B, V, Hq, Hkv, D, P);
    if (need == 0) return TEV_ERR_SHAPE;
    if (need > (size_t)TEV_NOALLOC_SCRATCH_BYTES) return TEV_ERR_WORKSPACE;
    // Remaining argument checks run in the round itself, before any launch;
    // the scratch address is looked up only once they could pass.
    if (!dtype_ok(dtype)) return TEV_ERR_DTYPE;
    void *ws = scratch_on_current_device();
    if (!ws) return TEV_ERR_HIP;
    return tev_verify_round_timed(q, k, v, logits, dtype, parents, tokens, R, B, V, Hq, Hkv, D, P,
                                  scale, inv_temperature, uniforms, n_draws, attn_out, rho, reach,
                                  exit_mass, coverage, exit_node, bonus_token, ws,
                                  (size_t)TEV_NOALLOC_SCRATCH_BYTES, stream, nullptr);
}

tev_status tev_validate_tree_host(const int32_t *parents_host, const int32_t *tokens_host, int B,
                                  int V) {
    if (!parents_host || !tokens_host) return TEV_ERR_NULL;
    if (B < 1 || B > TEV_MAX_NODES || V < 1) return TEV_ERR_SHAPE;
    if (parents_host[0] != -1) return TEV_ERR_TREE;
    // per parent: the child tokens seen so far (sibling tokens must differ)
    for (int i = 1; i < B; i++) {
        const int p = parents_host[i];
        if (p < 0 || p >= i) return TEV_ERR_TREE;
        if (tokens_host[i] < 0 || tokens_host[i] >= V) return TEV_ERR_TREE;
        for (int j = 1; j < i; j++)
            if (parents_host[j] == p && tokens_host[j] == tokens_host[i]) return TEV_ERR_TREE;
    }
    return TEV_OK;
}

tev_status tev_read_device_status(const void *workspace, int kind, int R, int B, int V,
                                  uint32_t *flags_host, void *stream) {
    if (!workspace || !flags_host) return TEV_ERR_NULL;
    if (R < 1) return TEV_ERR_SHAPE;
    if (kind < 0 || kind > 4) return TEV_ERR_SHAPE;
    // Every layout places the status words first.
    hipError_t e = hipMemcpyAsync(flags_host, workspace, sizeof(uint32_t) * (size_t)R,
                                  hipMemcpyDeviceToHost, (hipStream_t)stream);
    if (e == hipSuccess) e = hipStreamSynchronize((hipStream_t)stream);
    if (e != hipSuccess || kind != 2) return hip_status(e);
    if (check_exit_shape(R, B, V) != TEV_OK) return TEV_ERR_SHAPE;
    // the round's workspace: the attention part follows the exit-law part
    const size_t off = align_up(exit_ws_layout(R, B, V).total, 256);
    for (int r = 0; r < R; r++) {
        uint32_t fa = 0;
        e = hipMemcpy(&fa, (const char *)workspace + off + sizeof(uint32_t) * r, sizeof(uint32_t),
                      hipMemcpyDeviceToHost);
        if (e != hipSuccess) return TEV_ERR_HIP;
        flags_host[r] |= fa;
    }
    return TEV_OK;
}

tev_status tev_export_exit_cdf(const void *workspace, int R, int B, int V, double *cdf_host,
                               void *stream) {
    if (!workspace || !cdf_host) return TEV_ERR_NULL;
    tev_status s = check_exit_shape(R, B, V);
    if (s != TEV_OK) return s;
    const ExitWs L = exit_ws_layout(R, B, V);
    hipError_t e = hipMemcpyAsync(cdf_host, (const char *)workspace + L.wcum,
                                  sizeof(double) * (size_t)R * B, hipMemcpyDeviceToHost,
                                  (hipStream_t)stream);
    if (e == hipSuccess) e = hipStreamSynchronize((hipStream_t)stream);
    if (e != hipSuccess) return TEV_ERR_HIP;
    for (int r = 0; r < R; r++) {
        const double S = cdf_host[(size_t)r * B + B - 1];
        for (int j = 0; j < B; j++) cdf_host[(size_t)r * B + j] /= S;
    }
    return TEV_OK;
}

tev_status tev_export_residual_cdf(const void *logits, int dtype, const int32_t *parents,
                                   const int32_t *tokens, int R, int B, int V,
                                   float inv_temperature, const void *workspace,
                                   size_t workspace_bytes, int r, int node, double *cdf,
                                   void *stream) {
    if (!logits || !parents || !tokens || !workspace || !cdf) return TEV_ERR_NULL;
    if (!dtype_ok(dtype)) return TEV_ERR_DTYPE;
    tev_status s = check_exit_shape(R, B, V);
    if (s != TEV_OK) return s;
    if (r < 0 || r >= R || node < 0 || node >= B) return TEV_ERR_SHAPE;
    if (!(inv_temperature > 0.f) || !isfinite(inv_temperature)) return TEV_ERR_VALUE;
    if (workspace_bytes < exit_ws_layout(R, B, V).total) return TEV_ERR_WORKSPACE;
    return hip_status(launch_residual_cdf(logits, dtype, vec_ok(logits, dtype, V), parents, tokens,
                                          R, B, V, log2e_scale(inv_temperature),
                                          (const char *)workspace, r, node, cdf,
                                          (hipStream_t)stream));
}

}  // extern "C"
