/*
 * tev.h -- C ABI of the MI355X (gfx950) draft-tree verification library.
 *
 * The library runs the verification stage of tree speculative decoding on one
 * GPU: one layer of ancestor-masked tree attention, the canonical exit law,
 * and Tree Exit Verification (TEV)'s exit-node and bonus-token draws.
 *
 * Conventions shared by every call
 * --------------------------------
 *  - Every array pointer is a DEVICE pointer owned by the caller unless its
 *    comment says "host".  The library never allocates, frees or retains
 *    memory, and holds no global mutable state: calls are reentrant, and
 *    calls on different workspaces may run concurrently.  The one exception
 *    is tev_verify_round_noalloc, whose workspace is a library-owned device
 *    array (see there).
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *    Every call enqueues its kernels on `stream` and returns without
 *    synchronising, except the calls marked "synchronous".
 *  - Inputs are read only.  Outputs are fully overwritten, never accumulated.
 *  - Arrays are row-major and contiguous.  R is the number of independent
 *    requests, B the number of tree nodes per request INCLUDING the root
 *    (node 0), V the vocabulary size.  A tree is given as `parents[r][i]`
 *    (parents[r][0] = -1 and 0 <= parents[r][i] < i for i >= 1, i.e. any
 *    ancestor-before-descendant order) and `tokens[r][i]`, the incoming token
 *    of node i (0 <= tokens[r][i] < V for i >= 1; tokens[r][0] is not read).
 *    Sibling tokens must be distinct.  1 <= B <= TEV_MAX_NODES.
 *  - Errors a host can see (null pointers, bad sizes, unsupported dtype,
 *    workspace too small) return a status before anything is enqueued.
 *    Errors only the device can see (NaN or +inf logits, a row that is
 *    entirely -inf, an invalid tree) set per-request flag bits in the
 *    workspace; that request's float outputs become NaN and its integer
 *    outputs -1.  -inf logits are allowed and mean probability zero.
 *  - No C++ exception crosses this boundary.
 *
 * Sources (titles of the pages the operations are defined on):
 *  [EXIT] "Where Draft Trees Lose Target Mass: Exit-Guided Speculative
 *         Decoding" (arXiv 2610.11750): Sec. 3 Eq. 1-2, Sec. 3.1 Eq. 4,
 *         Lemma 1 Eq. 5, Sec. 3.2 Eq. 6-7, App. B Algorithm 1, Sec. 5
 *         Eq. 14 and App. C.2 Eq. 66-67.
 *  [CAST] "CAST: Cost-Aware Speculative Trees from One-Pass Block Drafters"
 *         (arXiv 2610.00321): App. B Lemma 1, App. C "Candidate
 *         construction" and "Packed verification", Thm. 1,
 *         App. F varlen tree-attention verifier.
 */
#ifndef TEV_H
#define TEV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define TEV_MAX_NODES 256

/* Bytes of the device scratch array behind tev_verify_round_noalloc (32 MiB
 * per GPU, held from the first such call on a GPU until the process ends). */
#define TEV_NOALLOC_SCRATCH_BYTES (32u << 20)

typedef enum {
    TEV_OK = 0,
    TEV_ERR_NULL = 1,        /* a required pointer is NULL                        */
    TEV_ERR_SHAPE = 2,       /* a size is out of range or inconsistent            */
    TEV_ERR_DTYPE = 3,       /* dtype code unknown or unsupported for this call   */
    TEV_ERR_TREE = 4,        /* host-side tree validation failed                  */
    TEV_ERR_WORKSPACE = 5,   /* workspace smaller than *_workspace_bytes()        */
    TEV_ERR_UNSUPPORTED = 6, /* e.g. head_dim not in {64, 128}                    */
    TEV_ERR_HIP = 7,         /* a HIP runtime call or launch failed               */
    TEV_ERR_VALUE = 8        /* a scalar argument is not finite / not positive    */
} tev_status;

typedef enum { TEV_F32 = 0, TEV_BF16 = 1 } tev_dtype;

/* Per-request device flag bits (see tev_read_device_status). */
#define TEV_FLAG_NONFINITE 1u /* NaN or +inf logit, or a row that is all -inf */
#define TEV_FLAG_TREE 2u      /* parents/tokens violate the tree contract      */

/* ------------------------------------------------------------------------
 * Exit law ([EXIT] Eq. 1, 2, 4, 6; Algorithm 1 lines computing rho, w, P).
 *
 * For every request r and node v, with x_a = inv_temperature * logits[r][v][a]:
 *   p_v(a)   = exp(x_a) / sum_b exp(x_b)                       (Eq. 1)
 *   rho(v)   = sum_{a not a child token of v} p_v(a); 1 at a leaf (Eq. 4)
 *   P(0) = 1, P(u) = P(parent(u)) * p_{parent(u)}(tokens[u])    (Eq. 2)
 *   w(v)     = P(v) * rho(v)                                   (Eq. 4)
 *   C        = sum_{u >= 1} P(u); expected block length 1 + C  (Eq. 6)
 *
 * logits    [R][B][V], dtype TEV_F32 or TEV_BF16 (bf16 = upper 16 bits of
 *           an IEEE binary32).  Vector loads are used when V * element size
 *           is a multiple of 16 bytes and `logits` is 16-byte aligned.
 * rho, reach, exit_mass  float [R][B] outputs;  coverage float [R] output.
 * inv_temperature must be finite and > 0 (1.0 = the target's own law).
 * workspace must hold tev_exit_law_workspace_bytes(R, B, V) bytes (any
 * initial contents).  After the call it holds the fp64 exit law and
 * per-chunk row statistics that tev_sample reads.  Its contents are private.
 * Calls that share a workspace must not overlap in time.  Each row of logits
 * is read exactly once.
 * ------------------------------------------------------------------------ */
size_t tev_exit_law_workspace_bytes(int R, int B, int V);

tev_status tev_exit_law(const void *logits, int dtype, const int32_t *parents,
                        const int32_t *tokens, int R, int B, int V, float inv_temperature,
                        float *rho, float *reach, float *exit_mass, float *coverage,
                        void *workspace, size_t workspace_bytes, void *stream);

/* ------------------------------------------------------------------------
 * TEV draws ([EXIT] App. B, Algorithm 1: "Draw V ~ Categorical(w)" and
 * "Draw Y ~ p_V if V is a leaf, otherwise p_V^res"; residual law Eq. 7).
 *
 * uniforms  float [R][n_draws][2]: (u1, u2) in [0, 1), the caller's control
 *           randomness; u1 drives the exit draw and u2 the bonus draw.
 * exit_node, bonus_token  int32 [R][n_draws] outputs.
 * Exit node: the smallest j with u1 * S < W_j, W_j = sum_{i <= j} w(i) in
 * node-index order, S = W_{B-1} (fp64).  Bonus token: the smallest token a
 * with u2 * T < R_a, R_a the running sum in token-id order of node V's
 * residual p_V(a) * [a is not a child token of V], T its total.
 * `workspace` must be the one filled by tev_exit_law for the same logits,
 * tree, sizes and inv_temperature, earlier on the same stream (or ordered
 * before this call).  tev_sample does not modify it.
 * ------------------------------------------------------------------------ */
tev_status tev_sample(const void *logits, int dtype, const int32_t *parents,
                      const int32_t *tokens, int R, int B, int V, float inv_temperature,
                      const void *workspace, size_t workspace_bytes,
                      const float *uniforms, int n_draws,
                      int32_t *exit_node, int32_t *bonus_token, void *stream);

/* ------------------------------------------------------------------------
 * Predraw-and-follow verification ([EXIT] App. A.4.1), the verifier TEV is
 * measured against: same inputs, same law of (exit node, bonus token).
 *
 * Every node v draws R_v from its full target row p_v (children included):
 * the smallest token a with u_v * T_v < R_{v,a}, R_{v,a} the running sum of
 * p_v in token-id order and T_v its total.  The walk starts at the root; at
 * node v it moves to the child whose incoming token equals R_v and stops when
 * none does: exit node v, bonus token R_v.
 *
 * uniforms    float [R][n_draws][B]: u_v in [0, 1) for every node of every draw.
 * node_draw   int32 [R][n_draws][B] output: R_v of every node.
 * exit_node, bonus_token  int32 [R][n_draws] outputs.
 * `workspace` must be the one filled by tev_exit_law for the same logits,
 * tree, sizes and inv_temperature, earlier on the same stream (the draws use
 * its per-chunk row sums); it is not modified.  R <= 65535, n_draws <= 65535.
 * A request flagged by tev_exit_law gets -1 in every output.
 * ------------------------------------------------------------------------ */
tev_status tev_predraw(const void *logits, int dtype, const int32_t *parents,
                       const int32_t *tokens, int R, int B, int V, float inv_temperature,
                       const void *workspace, size_t workspace_bytes, const float *uniforms,
                       int n_draws, int32_t *node_draw, int32_t *exit_node,
                       int32_t *bonus_token, void *stream);

/* ------------------------------------------------------------------------
 * One layer of ancestor-masked tree attention ([CAST] App. B Lemma 1 and
 * App. C "Packed verification": every packed node attends to all P cached
 * prefix entries and to the entries of its own root path, itself included).
 *
 * q     [R][B][Hq][D];  k, v  [R][Hkv][P + B][D]: cache rows 0..P-1 are the
 *       prefix, row P + i holds tree node i (row P is the root); rotary
 *       phases are already applied by the caller.
 * out   float [R][B][Hq][D]:
 *       out[r,i,h,:] = sum_j softmax_j(scale * <q[r,i,h,:], k[r,g,j,:]>) v[r,g,j,:]
 *       over j in {0..P-1} U {P + a : a on the root path of i}, with kv head
 *       g = h / (Hq / Hkv).
 * dtype TEV_BF16 (MFMA kernels, fp32 accumulation) or TEV_F32 (vector-ALU
 * kernel).  D must be 64 or 128; Hq % Hkv == 0; P >= 0; one head's K (and
 * V) extent (P + B) * D * element size must be below 2^31 bytes (the kernels
 * address it with 32-bit offsets), else TEV_ERR_SHAPE; scale must be finite
 * and > 0 (1/sqrt(D) in every workload), else TEV_ERR_VALUE.
 * parents [R][B] as above (tokens are not needed).
 * workspace must hold tev_tree_attn_workspace_bytes(R, B, Hq, Hkv, D, P) bytes
 * (partial results of split-prefix launches and per-request status).
 * ------------------------------------------------------------------------ */
size_t tev_tree_attn_workspace_bytes(int R, int B, int Hq, int Hkv, int D, int P);

tev_status tev_tree_attn(const void *q, const void *k, const void *v, int dtype,
                         const int32_t *parents, int R, int B, int Hq, int Hkv, int D, int P,
                         float scale, float *out, void *workspace, size_t workspace_bytes,
                         void *stream);

/* ------------------------------------------------------------------------
 * One whole verification round: tree attention, exit law and draws.
 *
 * Computes exactly what tev_tree_attn, tev_exit_law and tev_sample compute,
 * in that order, with the arguments of those calls (one dtype for both q/k/v
 * and logits), into the same outputs.  The work is packed into three
 * launches (vocabulary pass; attention beside the reach; draws beside the
 * split combine), so the single-workgroup steps of the exit law overlap the
 * attention instead of following it.
 *
 * workspace must hold tev_verify_round_workspace_bytes(R, B, V, Hq, Hkv, D, P)
 * bytes, any initial contents; calls sharing a workspace must not overlap.
 * Its first tev_exit_law_workspace_bytes(R, B, V) bytes are an exit-law
 * workspace: tev_sample, tev_export_exit_cdf and tev_export_residual_cdf
 * accept it after the round.  tev_read_device_status with kind 2 returns the
 * request's exit-law and attention flags together.
 * Errors: as the three calls (host checks before anything is enqueued),
 * including the attention's limits on scale and on the K / V extent.
 * ------------------------------------------------------------------------ */
size_t tev_verify_round_workspace_bytes(int R, int B, int V, int Hq, int Hkv, int D, int P);

tev_status tev_verify_round(const void *q, const void *k, const void *v, const void *logits,
                            int dtype, const int32_t *parents, const int32_t *tokens, int R,
                            int B, int V, int Hq, int Hkv, int D, int P, float scale,
                            float inv_temperature, const float *uniforms, int n_draws,
                            float *attn_out, float *rho, float *reach, float *exit_mass,
                            float *coverage, int32_t *exit_node, int32_t *bonus_token,
                            void *workspace, size_t workspace_bytes, void *stream);

/* tev_verify_round for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same arguments and outputs, but no workspace argument.
 * Its workspace is a file-scope device array of TEV_NOALLOC_SCRATCH_BYTES
 * bytes per GPU, whose address the first call on a GPU looks up (with that
 * GPU current) and keeps; the call itself allocates nothing.  `stream` must
 * belong to the current device.
 * Errors: as tev_verify_round; TEV_ERR_WORKSPACE when
 * tev_verify_round_workspace_bytes(R, B, V, Hq, Hkv, D, P) exceeds
 * TEV_NOALLOC_SCRATCH_BYTES (checked before anything else touches the GPU);
 * TEV_ERR_HIP if the array's address cannot be obtained.
 * Every call on one GPU shares that GPU's array and leaves its contents
 * behind (the round needs no zeroed workspace, so nothing is cleared):
 * calls that overlap on one GPU -- on different streams, or from several
 * host threads -- race and must not be issued.  Device flags stay in the
 * array; a flagged request shows as NaN / -1 outputs. */
tev_status tev_verify_round_noalloc(const void *q, const void *k, const void *v,
                                    const void *logits, int dtype, const int32_t *parents,
                                    const int32_t *tokens, int R, int B, int V, int Hq, int Hkv,
                                    int D, int P, float scale, float inv_temperature,
                                    const float *uniforms, int n_draws, float *attn_out,
                                    float *rho, float *reach, float *exit_mass, float *coverage,
                                    int32_t *exit_node, int32_t *bonus_token, void *stream);

/* tev_verify_round, and for profiling: events[0..3] (hipEvent_t, created by
 * the caller, any entry may be NULL) are recorded on `stream` before the
 * vocabulary pass, after it, after the attention launch and after the last
 * launch (fp32: before the exit law, after it, after the attention, after the
 * draws), so that the caller can time each launch.  events may be NULL. */
tev_status tev_verify_round_timed(const void *q, const void *k, const void *v,
                                  const void *logits, int dtype, const int32_t *parents,
                                  const int32_t *tokens, int R, int B, int V, int Hq, int Hkv,
                                  int D, int P, float scale, float inv_temperature,
                                  const float *uniforms, int n_draws, float *attn_out,
                                  float *rho, float *reach, float *exit_mass, float *coverage,
                                  int32_t *exit_node, int32_t *bonus_token, void *workspace,
                                  size_t workspace_bytes, void *stream, void *const *events);

/* ------------------------------------------------------------------------
 * KV-cache commit after verification ([CAST] App. C "Packed verification":
 * only the accepted root path keeps its packed cache entries; [EXIT] the
 * verifier stage's cache commit).
 *
 * k, v      [L][R][Hkv][P + B][D] (L layers), dtype TEV_BF16 or TEV_F32,
 *           16-byte aligned; modified IN PLACE.
 * exit_node int32 [R]: the accepted node V of each request (e.g. the first
 *           column of tev_sample's output); its root path is
 *           0 = a_0, a_1, ..., a_A = V with A = depth(V).
 * For every layer, request and kv head, cache row P + a_d moves to row P + d
 * (d = 0..A); rows 0..P-1 and rows past P + A keep their contents.
 * new_len   int32 [R] output: P + A + 1, the committed cache length, or -1
 *           when V is out of range or the parents on its root path violate
 *           the tree contract (nothing of that request is moved).
 * D must be 64 or 128.  Calls on the same cache must not overlap.
 * ------------------------------------------------------------------------ */
tev_status tev_commit_kv(void *k, void *v, int dtype, const int32_t *parents,
                         const int32_t *exit_node, int R, int B, int L, int Hkv, int D, int P,
                         int32_t *new_len, void *stream);

/* ------------------------------------------------------------------------
 * Exit-guided draft-tree loss ([EXIT] Sec. 5 Eq. 14, evaluated per App. C.2
 * Eq. 66-67) and its gradient in the draft logits.
 *
 * draft_logits [R][H][V], TEV_F32 or TEV_BF16: the drafter's position-wise
 *           logits.  Row (r, d - 1) is future draft position d = 1..H of
 *           example r and scores every node of depth d (depth = number of
 *           edges from the root); nodes at one depth share the row.
 * parents, tokens [R][B]: the realised trees (library tree contract; sibling
 *           tokens need not be distinct here).  Every node's depth must be
 *           <= H.
 * weights   float [R][B]: the detached node weights w(v), e.g. the
 *           exit_mass output of tev_exit_law.  weights[r][0] is not read.
 *
 *   loss  = sum_r sum_{v >= 1, w(v) != 0} w(v) (lse_{r,d(v)} - z_{r,d(v),x_v})
 *           / (R (B - 1))                       (0 when B = 1)
 *   lse_m = log sum_a exp(z_{m,a})             natural log, one per row
 * A node with weight exactly 0 contributes nothing.
 *
 * loss        float [1] output.
 * row_lse     float [R][H] output: lse_m of every row.
 * row_weight  float [R][H] output: summed weight of the row's nodes.
 * grad        float [R][H][V] output, or NULL for the loss alone:
 *             d loss / d z_{m,a} = (row_weight_m softmax(z_m)_a
 *                                   - sum_{v in m, x_v = a} w(v)) / (R (B - 1)).
 * workspace   tev_exit_loss_workspace_bytes(R, B, H, V) bytes, any contents;
 *             its first R words are the per-example flag words
 *             (tev_read_device_status kind 3).
 * A flagged example (invalid tree, a node deeper than H, a NaN or +inf logit
 * or an all -inf row in any of its rows) makes its row outputs, its gradient
 * rows and the loss NaN.  Limits: 1 <= H <= 1024, R * H <= 65535.
 * ------------------------------------------------------------------------ */
size_t tev_exit_loss_workspace_bytes(int R, int B, int H, int V);

tev_status tev_exit_loss(const void *draft_logits, int dtype, const int32_t *parents,
                         const int32_t *tokens, const float *weights, int R, int B, int H, int V,
                         float *loss, float *row_lse, float *row_weight, float *grad,
                         void *workspace, size_t workspace_bytes, void *stream);

/* ------------------------------------------------------------------------
 * Best-first draft tree ([CAST] App. C "Candidate construction" and Thm. 1;
 * "Multi-Future Drafting: Mixture Block Drafters for Tree-Verified
 * Speculative Decoding" App. B, the merged heap with one mode = DDTree's
 * builder).
 *
 * draft_logits [R][L][V], TEV_F32 or TEV_BF16: row (r, j) is the drafter's
 *           logits for draft position j + 1 of request r; q_j = its softmax
 *           over the whole vocabulary.
 * root_tokens int32 [R] (device) or NULL: written to tokens[r][0] (0 if NULL).
 * Each position keeps its K most likely tokens (larger logit first, then the
 * smaller token id); the tree is the B - 1 prefixes of that retained universe
 * with the largest plug-in score prod_j q_j(y_j), in pop order (best first):
 *   key s(v) = sum_{j <= d} z_{j, y_j} - sum_{j <= d} lse_j   (d = depth of v)
 * with the logit sum accumulated in f64 along the path (exact for bf16
 * logits); equal keys go to the shorter prefix, then to the lexicographically
 * smaller sequence of ranks.
 *
 * parents, tokens  int32 [R][B] outputs (node 0 = root, parents[r][0] = -1,
 *           parents[r][i] < i): the library's tree contract.
 * scores    double [R][B] output: s(v) = log of the plug-in score (root 0).
 * workspace tev_build_tree_workspace_bytes(R, L, V, K) bytes, any contents;
 *           its first R words are the flag words (tev_read_device_status
 *           kind 4).  A NaN or +inf logit, or an all -inf row, flags the
 *           request: its tokens and parents are -1 and its scores NaN.
 * Limits: 1 <= L <= 16, 1 <= K <= min(128, V), 1 <= B <= 256, B - 1 <= the
 * number of prefixes of the universe (K + K^2 + ... + K^L), V <= 524288 with
 * ceil(V / 8192) * K <= 8192, R * L <= 65535.
 * ------------------------------------------------------------------------ */
size_t tev_build_tree_workspace_bytes(int R, int L, int V, int K);

tev_status tev_build_tree(const void *draft_logits, int dtype, const int32_t *root_tokens, int R,
                          int L, int V, int K, int B, int32_t *parents, int32_t *tokens,
                          double *scores, void *workspace, size_t workspace_bytes, void *stream);

/* ------------------------------------------------------------------------
 * The merged heap over M draft modes ("Multi-Future Drafting" App. B and
 * Prop. 6): the tree of the B - 1 distinct prefixes with the largest
 * best-mode score s(v) = max_k s_k(v), nodes in the order of their first
 * pops.
 *
 * draft_logits [R][M][L][V]: mode k's position-wise logits; mode k keeps its
 *           own K most likely tokens per position (as tev_build_tree).
 * log_prior float [R][M] (device) = log pi_k, or NULL for the uniform prior.
 *   s_k(v) = (sum_j z_{k,j,y_j} - sum_j lse_{k,j}) + log pi_k
 * The merged heap pops entries (k, v) by key s_k(v) (equal keys: shorter
 * prefix, then smaller rank sequence, then smaller k); the first pop of each
 * distinct prefix creates its node, with score s(v).  With M = 1 and no prior
 * this is tev_build_tree.  If the modes' universes hold fewer than B - 1
 * distinct prefixes, the missing nodes get parent and token -1 and score NaN.
 * Outputs, flags and limits as tev_build_tree, with 1 <= M <= 8,
 * R * M * L <= 65535 and M (K + ... + K^L) >= B - 1; the workspace holds
 * tev_build_tree_modes_workspace_bytes(R, M, L, V, K, B) bytes (flag words:
 * tev_read_device_status kind 4).
 * ------------------------------------------------------------------------ */
size_t tev_build_tree_modes_workspace_bytes(int R, int M, int L, int V, int K, int B);

tev_status tev_build_tree_modes(const void *draft_logits, int dtype, const float *log_prior,
                                const int32_t *root_tokens, int R, int M, int L, int V, int K, int B,
                                int32_t *parents, int32_t *tokens, double *scores, void *workspace,
                                size_t workspace_bytes, void *stream);

/* ------------------------------------------------------------------------
 * Host-side helpers.
 * ------------------------------------------------------------------------ */

/* Validates one tree held in HOST memory (parents_host, tokens_host [B])
 * against the contract above.  Touches no GPU.  TEV_OK or TEV_ERR_TREE. */
tev_status tev_validate_tree_host(const int32_t *parents_host, const int32_t *tokens_host,
                                  int B, int V);

/* Copies the R per-request flag words (TEV_FLAG_*) of an exit-law,
 * tree-attention, round or exit-loss workspace into flags_host [R].  `kind`
 * is 0 for an exit-law workspace (sizes R, B, V), 1 for a tree-attention
 * workspace (only R is used), 2 for a tev_verify_round workspace (sizes R, B,
 * V; the two parts' flags are OR-ed), 3 for a tev_exit_loss workspace and 4
 * for a tev_build_tree workspace (only R is used).  Synchronous: waits for
 * `stream`. */
tev_status tev_read_device_status(const void *workspace, int kind, int R, int B, int V,
                                  uint32_t *flags_host, void *stream);

/* Static description of a status code. */
const char *tev_status_str(int status);

/* ------------------------------------------------------------------------
 * Verification exports.  These expose the CDFs the sampler searches, so that
 * a test can bound their deviation from an independent computation.
 * ------------------------------------------------------------------------ */

/* Normalised exit CDF W_j / S of every request, fp64, into cdf_host [R][B]
 * (HOST).  Synchronous. */
tev_status tev_export_exit_cdf(const void *workspace, int R, int B, int V, double *cdf_host,
                               void *stream);

/* Normalised residual CDF of node `node` of request `r`, in token order, as
 * the sampler evaluates it (chunk running sums plus the in-chunk scan), into
 * the DEVICE array cdf [V] (fp64).  Same logits/tree/workspace as tev_sample. */
tev_status tev_export_residual_cdf(const void *logits, int dtype, const int32_t *parents,
                                   const int32_t *tokens, int R, int B, int V,
                                   float inv_temperature, const void *workspace,
                                   size_t workspace_bytes, int r, int node, double *cdf,
                                   void *stream);

#ifdef __cplusplus
}
#endif
#endif /* TEV_H */
