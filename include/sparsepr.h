/*
 * sparsepr.h - C-ABI of the SparsePR per-call sparse attention operator on
 * AMD MI355X (gfx950).
 *
 * SparsePR (arxivdaily 2608.18484, "English abstract"; skillfed article
 * "Partition the Support, Reconstruct the Residual", paragraph on the two
 * components) replaces one attention call:
 *   1. sparsepr_partition  keys are clustered by their responses to sampled
 *                          queries into paired K/V groups;
 *   2. sparsepr_route      queries are grouped by their responses to the
 *                          key-group centroids and each query block is routed
 *                          to its best key groups;
 *   3. sparsepr_attend     attention runs only between each query block and
 *                          its routed groups (softmax renormalised over them);
 *   4. sparsepr_probe_fit  a few query rows per head get exact attention and
 *                          a weighted ridge regression fits an affine map from
 *                          sparse output to the dense-minus-sparse residual,
 *                          inside the probe residuals' principal subspace;
 *   5. sparsepr_apply      the predicted residual is added to every unprobed
 *                          row; probe rows keep their exact output.
 * sparsepr_dense_attention is the exact operator the speedup is measured
 * against.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Every pointer argument except `params` and `workspace_bytes`-style host
 *   outputs is a DEVICE pointer on the current HIP device. The library
 *   allocates nothing and keeps no state between calls; the caller owns all
 *   buffers, including the workspace. (One exception by design:
 *   sparsepr_apply_noalloc keeps its scratch in a fixed device array of the
 *   library, see there.)
 * - Tensors are contiguous, head-major: [H, N, d] means element
 *   (h, i, e) at ((h * N) + i) * d + e. Per-head index arrays are [H, N] etc.
 * - `dtype` selects the element type of Q, K, V, Kp, Vp, the sparse output
 *   S_out and O: SPARSEPR_F32 (IEEE binary32) or SPARSEPR_BF16 (bfloat16).
 *   All other floating arrays are fp32. The apply reads S_out once per row;
 *   the fit reads the probe rows' sparse outputs from S_probe, an fp32 copy
 *   of those rows, so the fitted map sees no storage rounding.
 * - Token index t in [0, N) is a row of Q/K/V. "Query order" position i
 *   refers to token query_perm[h, i].
 * - `stream` is a hipStream_t (NULL = legacy default stream). Work is only
 *   enqueued; results are valid after the stream is synchronised. Calls on
 *   different streams with disjoint buffers may run concurrently. No entry
 *   point allocates, copies, clears memory with a memset or synchronises, so
 *   a sequence of calls can be captured in a HIP graph and replayed.
 * - Errors: validation is done on the host before anything is enqueued. A
 *   non-zero status means nothing was launched, except SPARSEPR_ERR_HIP,
 *   which reports that a launch failed (earlier launches of the same call
 *   may already be enqueued). sparsepr_last_error() gives a message for the
 *   calling thread's last failure. Index arrays living on the device are not
 *   validated on the host: out-of-range entries are clamped into [0, N) by
 *   the kernels (never read out of bounds) and give meaningless results.
 * - The softmax scale `scale[h]` (tau, fp32 on the device) may be any finite
 *   value, negative or zero included; the attention kernels keep their
 *   exponentials in range for any span of the scaled logits.
 */
#ifndef SPARSEPR_H
#define SPARSEPR_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* 2: S_out has the element type `dtype` (fp32 on both paths in 1); the
   probe rows' sparse outputs go to S_probe (fp32), which stage 4 reads.
   3: sparsepr_attend, sparsepr_attend_subset and sparsepr_dense_attention
   take an optional work-queue buffer (queue, queue_bytes) before `stream`.
   4: sparsepr_params ends with an optional `probe_pos` array. */
#define SPARSEPR_ABI_VERSION 4

/* Bytes of the optional work-queue buffer of the attention entry points. */
#define SPARSEPR_QUEUE_BYTES 1024

/* status codes */
#define SPARSEPR_OK 0
#define SPARSEPR_ERR_INVALID_ARG 1  /* a parameter or pointer is invalid */
#define SPARSEPR_ERR_UNSUPPORTED 2  /* valid but not supported (e.g. head_dim) */
#define SPARSEPR_ERR_WORKSPACE 3    /* workspace missing or too small */
#define SPARSEPR_ERR_HIP 4          /* a HIP launch failed */

/* element types */
#define SPARSEPR_F32 0
#define SPARSEPR_BF16 1

/* partition modes */
#define SPARSEPR_RESPONSE_COUPLED 0
#define SPARSEPR_RANDOM_BLOCK 1     /* ablation without response-coupled partitioning */
#define SPARSEPR_SEMANTIC 2         /* comparator: k-means on raw key (and query) features */

/*
 * Parameters of one call. The executed-pair budget follows the pages' rule
 * that probe rows are counted in the density (skillfed article, results
 * paragraph): every probe costs N pairs and each query row of the sparse
 * pass may use kappa = floor(density * N - n_probes) keys, computed in
 * double precision; kappa must be >= 1.
 */
typedef struct sparsepr_params {
  int32_t heads;          /* 1 <= H <= 65535 */
  int32_t n_tokens;       /* N >= 1 */
  int32_t head_dim;       /* d in {64, 128} */
  int32_t dtype;          /* SPARSEPR_F32 or SPARSEPR_BF16 */
  int32_t q_block;        /* B_q in {64, 128}: query rows per routed block */
  int32_t n_groups;       /* G, 1 <= G <= min(N, 1024): key groups */
  int32_t n_samples;      /* S, 1 <= S <= N: sampled queries (response-coupled mode) */
  int32_t kmeans_iters;   /* T >= 1: Lloyd iterations (response-coupled mode) */
  double density;         /* rho in (0, 1]: executed-pair density including probes */
  int32_t n_probes;       /* m, 0 <= m <= N: exact probe rows per head */
  int32_t rank;           /* k, 0 <= k <= d: residual subspace rank */
  double ridge_lambda;    /* lambda > 0: ridge penalty (bias unpenalised) */
  int32_t partition_mode; /* SPARSEPR_RESPONSE_COUPLED, SPARSEPR_RANDOM_BLOCK or SPARSEPR_SEMANTIC */
  int32_t reserved;       /* must be 0 */
  /* Probe positions p_i in the query order, shared by every head: NULL for
     p_i = floor((i + 1/2) N / m) (the default), or a DEVICE array of m int32
     that the caller owns and keeps unchanged from stage 3 to stage 5 (the
     three stages must see the same positions). It must be strictly
     increasing with every entry in [0, N). The library does not read it on
     the host: entries outside [0, N) are clamped into it, and an array that
     is not strictly increasing gives unspecified outputs (every access
     stays inside the caller's buffers). Ignored when m = 0. */
  const int32_t* probe_pos;
} sparsepr_params;

/* Version of this ABI (SPARSEPR_ABI_VERSION). */
int32_t sparsepr_abi_version(void);

/* Static, NUL-terminated name of a status code. */
const char* sparsepr_status_string(int32_t status);

/* Message describing the calling thread's last non-zero status ("" if none). */
const char* sparsepr_last_error(void);

/* Validates `params` and returns the number of workspace bytes that every
 * stage below needs at most (one workspace serves all stages; stages on one
 * stream may share it). Host-only: launches nothing. */
int32_t sparsepr_workspace_bytes(const sparsepr_params* params, size_t* bytes);

/*
 * Stage 1 - response-coupled partitioning of the keys (arxivdaily 2608.18484,
 * English abstract: keys grouped by how they respond to sampled queries;
 * cpu3d summary: the groups are paired K/V groups).
 *
 * Response mode: key j's response profile is r_j = tau * Q[sample_idx] k_j
 * (one scaled logit per sampled query). Lloyd k-means with T iterations
 * clusters the profiles; centroid g starts at the profile of key
 * init_idx[g]; each assignment takes the lowest g among equal distances; an
 * emptied group keeps its previous centroid. Because profiles are linear in
 * k the work is done with key-space centroids under the metric
 * M = tau^2 Q_s^T Q_s.
 * Random-block mode: the permutation rand_key_perm is cut into G runs,
 * run g = positions floor(gN/G) .. floor((g+1)N/G)-1; sample_idx, init_idx
 * are ignored.
 * Semantic mode, the comparator the pages measure against (arxivdaily
 * 2608.18484, English abstract: semantic block-sparse attention without
 * residual correction): the same Lloyd k-means on the raw key rows, i.e.
 * metric M = I and centroid g starting at K[init_idx[g]]; Q, scale and
 * sample_idx are ignored. Run with K := Q it clusters the queries, and its
 * key_perm is then the semantic query order for sparsepr_route.
 *
 * Inputs : Q, K, V [H,N,d] dtype; scale [H] fp32 (tau per head);
 *          sample_idx [S] int32 and init_idx [G] int32 (response mode;
 *          distinct token indices shared by all heads);
 *          rand_key_perm [N] int32 (random-block mode, else may be NULL).
 * Outputs: key_label [H,N] int32 final group of each key token;
 *          key_perm [H,N] int32 group-contiguous key order: keys sorted by
 *            (group, token index);
 *          group_off [H,G+1] int32 group g = key_perm[group_off[g] ..
 *            group_off[g+1]-1]; empty groups have equal offsets;
 *          key_centroid [H,G,d] fp32 mean key of each group (for an empty
 *            group: its last centroid; it is excluded downstream);
 *          Kp, Vp [H,N,d] dtype: K and V rows gathered in key_perm order
 *            (both NULL: no gather; V is then not read and may be NULL);
 *          dbg_assign_scores [H,N,G] fp32 or NULL: the scores the final
 *            assignment took its argmin over, score(j,g) = ||r_j - c_g||^2
 *            - ||r_j||^2 (argmin over g of these is key_label).
 */
int32_t sparsepr_partition(const sparsepr_params* params, const void* Q, const void* K,
                           const void* V, const float* scale, const int32_t* sample_idx,
                           const int32_t* init_idx, const int32_t* rand_key_perm,
                           int32_t* key_label, int32_t* key_perm, int32_t* group_off,
                           float* key_centroid, void* Kp, void* Vp, float* dbg_assign_scores,
                           void* workspace, size_t workspace_bytes, void* stream);

/*
 * Stage 2 - query coordinates and shared routing (arxivdaily 2608.18484,
 * English abstract: queries grouped by their responses to the key-group
 * centroids for shared sparse routing; peercurrent abstract: centroids
 * induce query-response coordinates).
 *
 * C[q,g] = tau * q . kbar_g over non-empty groups. Response mode: each
 * query's dominant group g1 = argmax_g C (lowest g on ties) and value
 * v = C[q,g1]; queries are ordered by (g1 ascending, v descending, token
 * ascending). Random-block mode: the order is rand_query_perm. Semantic
 * mode: the order is given per head in rand_query_perm [H,N] (the key_perm
 * of sparsepr_partition run in semantic mode on the queries: queries sorted
 * by (query cluster, token)). The order is
 * cut into blocks of B_q (the last may be shorter). Each block b scores
 * groups by sigma[b,g] = tau * qbar_b . kbar_g (qbar_b = the block's mean
 * query, equal to the block mean of C), ranks non-empty groups by (sigma
 * descending, g ascending), and takes the longest ranked prefix whose total
 * key count is <= kappa (at least one group).
 *
 * Inputs : Q [H,N,d]; scale [H]; key_centroid [H,G,d]; group_off [H,G+1];
 *          rand_query_perm [N] int32 (random-block mode) or [H,N] int32
 *          (semantic mode), else may be NULL.
 * Outputs: query_perm [H,N] int32 position -> query token;
 *          block_ptr [H,nb+1] int32 and block_groups [H, nb*G] int32: CSR of
 *            the selected groups of each block, ascending; head h's offsets
 *            index block_groups + h*nb*G; nb = ceil(N / B_q);
 *          executed_pairs [H] int64: sum_b n_b |K(b)| + m N;
 *          dbg_coords [H,N,G] fp32 or NULL: C (empty groups -inf);
 *          dbg_dominant [H,N] int32 / dbg_dominant_val [H,N] fp32 or NULL:
 *            g1 and v per token (response mode);
 *          dbg_block_score [H,nb,G] fp32 or NULL: sigma.
 */
int32_t sparsepr_route(const sparsepr_params* params, const void* Q, const float* scale,
                       const float* key_centroid, const int32_t* group_off,
                       const int32_t* rand_query_perm, int32_t* query_perm, int32_t* block_ptr,
                       int32_t* block_groups, int64_t* executed_pairs, float* dbg_coords,
                       int32_t* dbg_dominant, float* dbg_dominant_val, float* dbg_block_score,
                       void* workspace, size_t workspace_bytes, void* stream);

/*
 * Stage 3 - block-sparse attention over the routed groups (arxivdaily
 * 2608.18484, English abstract, first sentence; skillfed article: the error
 * arises after the softmax is renormalised over the kept keys).
 *
 * For query position i in block b = i / B_q with token q = query_perm[i]:
 *   S_out[i] = sum_{j in K(b)} softmax_{K(b)}(tau q . k_j) v_j,
 *   lse[i]   = log sum_{j in K(b)} exp(tau q . k_j),
 * where K(b) = the keys of the block's selected groups, read from the
 * group-contiguous Kp/Vp. Needs no workspace. On the bf16 path the
 * probabilities are rounded to bf16 for the product with V, and both the
 * normalisation and lse use the sum of those rounded values, so lse is within
 * log(1 + 2^-9) < 2e-3 of the exact value.
 *
 * Inputs : Q [H,N,d]; Kp, Vp [H,N,d] (from stage 1); scale [H];
 *          group_off [H,G+1]; query_perm [H,N]; block_ptr, block_groups.
 * Outputs: S_out [H,N,d] dtype in QUERY ORDER; S_probe [H,m,d] fp32, row i =
 *          S_out at probe position p_i (stage 4) before rounding to dtype
 *          (may be NULL when m = 0); lse [H,N] fp32 (query order).
 * Work queue (optional): queue = SPARSEPR_QUEUE_BYTES of 4-byte aligned
 *          device memory, or NULL. On the bf16 path the call then keeps only
 *          as many workgroups as the GPU holds at once and they take query
 *          blocks from per-XCD counters in `queue`, so that faster XCDs take
 *          over the last blocks of slower ones; with NULL each block gets its
 *          own workgroup on a fixed XCD. The results are the same bit for bit
 *          either way (each block is computed the same way wherever it runs).
 *          The call clears the counters itself (with a kernel on `stream`)
 *          and their contents afterwards mean nothing. Calls that may run at
 *          the same time need distinct queue buffers; the fp32 path ignores it.
 *          Errors: SPARSEPR_ERR_INVALID_ARG for a misaligned queue,
 *          SPARSEPR_ERR_WORKSPACE for queue_bytes < SPARSEPR_QUEUE_BYTES.
 */
int32_t sparsepr_attend(const sparsepr_params* params, const void* Q, const void* Kp,
                        const void* Vp, const float* scale, const int32_t* group_off,
                        const int32_t* query_perm, const int32_t* block_ptr,
                        const int32_t* block_groups, void* S_out, float* S_probe, float* lse,
                        void* queue, size_t queue_bytes, void* stream);

/*
 * Stage 3 on a subset of the query blocks, so that the probe fit can start
 * before the whole sparse output exists (stage 4 reads only S_probe, the
 * probe positions p_i of its own description):
 *   SPARSEPR_BLOCKS_ALL              every block (= sparsepr_attend);
 *   SPARSEPR_BLOCKS_WITH_PROBE       only blocks holding some probe position;
 *   SPARSEPR_BLOCKS_WITHOUT_PROBE    only the other blocks.
 * Running subset 1 then subset 2 writes exactly what sparsepr_attend writes
 * (the blocks are disjoint and each is computed the same way). Between the
 * two, sparsepr_probe_fit may run on another stream; it touches the workspace
 * and this stage does not. Errors: as sparsepr_attend, and
 * SPARSEPR_ERR_INVALID_ARG for another subset value.
 */
#define SPARSEPR_BLOCKS_ALL 0
#define SPARSEPR_BLOCKS_WITH_PROBE 1
#define SPARSEPR_BLOCKS_WITHOUT_PROBE 2
int32_t sparsepr_attend_subset(const sparsepr_params* params, const void* Q, const void* Kp,
                               const void* Vp, const float* scale, const int32_t* group_off,
                               const int32_t* query_perm, const int32_t* block_ptr,
                               const int32_t* block_groups, void* S_out, float* S_probe,
                               float* lse, int32_t subset, void* queue, size_t queue_bytes,
                               void* stream);

/*
 * Stage 4 - exact probe rows and the probe-fitted map (arxivdaily 2608.18484,
 * English abstract: exact attention on a few rows, weighted ridge fit of the
 * dense-minus-sparse differences; skillfed article and peercurrent abstract:
 * per head, call-specific, restricted to the probe residuals' subspace).
 *
 * Probe i < m is the query at position p_i of the query order:
 * params->probe_pos[i] when given, else floor((i + 1/2) N / m).
 * o_i = dense attention of that query over all N keys; the keys may be
 * given in any order (e.g. Kp, Vp). With s_i = S_probe[i] (the
 * sparse output at p_i, in fp32):
 *   r_i = o_i - s_i;  w_i = ||o_i||^-2 / sum ||o||^-2 (0 where o_i = 0);
 *   Sigma = sum_i w_i r_i r_i^T;  U = eigenvectors of Sigma's k_eff largest
 *   eigenvalues, k_eff = min(k, m, d), or 0 when trace(Sigma) = 0;
 *   the map reads the subspace coordinates z_i = U^T s_i (skillfed article:
 *   a small linear map from the sparse output; peercurrent abstract: within
 *   the output subspace of the probe residuals): B solves
 *   (Z^T W Z + lambda_eff I~) B = Z^T W (R U) with Z = [z_i, 1],
 *   I~ = diag(1,..,1,0) (unpenalised bias) and lambda_eff = lambda times the
 *   mean weighted variance of the k_eff input coordinates (so the correction
 *   scales with V). Theta = [U B[0:k_eff]; B[k_eff]] is the same map written
 *   on [s; 1]: Theta^T [s; 1] = B^T [U^T s; 1].
 *
 * Inputs : Q [H,N,d]; K, V [H,N,d] (any key order); scale [H];
 *          query_perm [H,N]; S_probe [H,m,d] fp32 (from stage 3).
 * Outputs: O_probe [H,m,d] fp32 exact probe outputs;
 *          U [H,d,k] fp32 (columns >= k_eff are zero); Theta [H,d+1,k] fp32
 *          (row d is the bias; columns >= k_eff zero); rank_eff [H] int32.
 * m = 0 or k = 0 gives k_eff = 0 (no correction).
 */
int32_t sparsepr_probe_fit(const sparsepr_params* params, const void* Q, const void* K,
                           const void* V, const float* scale, const int32_t* query_perm,
                           const float* S_probe, float* O_probe, float* U, float* Theta,
                           int32_t* rank_eff, void* workspace, size_t workspace_bytes,
                           void* stream);

/*
 * Stage 5 - residual apply and return to token order (arxivdaily 2608.18484,
 * English abstract: the fitted map predicts a residual for each unprobed
 * query, added to its sparse output).
 *
 * For query position i with token q = query_perm[i]:
 *   O[q] = s_i + U Theta^T [s_i; 1]   if i is not a probe position,
 *   O[q] = O_probe[probe index]       if it is.
 * Inputs : S_out [H,N,d] dtype; query_perm [H,N]; O_probe [H,m,d]; U; Theta;
 *          rank_eff [H]; workspace (the shared one; this stage keeps the
 *          per-head matrix Theta U^T there). Output: O [H,N,d] dtype in TOKEN
 *          ORDER. Errors: as the other stages (NULL arguments, a workspace
 *          smaller than sparsepr_workspace_bytes).
 */
int32_t sparsepr_apply(const sparsepr_params* params, const void* S_out,
                       const int32_t* query_perm, const float* O_probe, const float* U,
                       const float* Theta, const int32_t* rank_eff, void* O, void* workspace,
                       size_t workspace_bytes, void* stream);

/*
 * Stage 5 without a workspace, for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation). Computes exactly what sparsepr_apply computes, with the same
 * kernels, arguments and errors, except that the per-head matrix Theta U^T
 * and bias live in a fixed device array inside the library instead of the
 * caller's workspace. That array holds SPARSEPR_APPLY_SCRATCH_BYTES on each
 * device the library runs on, until the process ends; its address is looked
 * up on a device's first call. The bf16 path needs H * (4 d^2 + 4 d) bytes
 * (256-byte aligned parts): up to 127 heads at d = 128, 503 at d = 64; the
 * fp32 path needs none. Larger calls are rejected with
 * SPARSEPR_ERR_WORKSPACE before anything is launched. Nothing is allocated,
 * freed or cleared. All calls on one device share the array and leave their
 * contents there: calls that may overlap on one device (other streams,
 * other threads) race and must be serialised by the caller.
 */
#define SPARSEPR_APPLY_SCRATCH_BYTES ((size_t)8 << 20)
int32_t sparsepr_apply_noalloc(const sparsepr_params* params, const void* S_out,
                               const int32_t* query_perm, const float* O_probe, const float* U,
                               const float* Theta, const int32_t* rank_eff, void* O,
                               void* stream);

/*
 * Support and mass diagnostics of sampled query blocks of one head (skillfed
 * article, the two problem paragraphs: queries that share a block route may
 * prefer different keys, and keeping most attention mass need not keep the
 * output; arxivdaily 2608.18484, English abstract: the partition decides how
 * much the grouped queries' preferred supports overlap). Not a stage of the
 * call: it measures one, after sparsepr_route.
 *
 * For row r of sampled block blocks[i] (query position p = blocks[i] B_q + r,
 * token q = query_perm[p]), with logits x_j = tau q . k_j over ALL N keys
 * (fp32) and probabilities p_j = softmax_j(x):
 *   lse[i B_q + r]            = log sum_j exp(x_j)
 *   routed_mass[i B_q + r]    = sum of p_j over the block's routed keys K(b)
 *                               (keys whose key_label is a routed group)
 *   theta                     = the largest logit t with sum_{x_j >= t} p_j >= mass
 *   support[i B_q + r]        = #{j : x_j >= theta}: the fewest keys that hold
 *                               the given mass (keys tied at theta all count)
 *   support_routed[i B_q + r] = #{j in K(b) : x_j >= theta}
 *   pooled[i]                 = |union over the block's rows of {j : x_j >= theta}|
 *   pooled_routed[i]          = the part of that union inside K(b).
 * Rows past N (ragged last block) give lse = -inf and zeros. Sums over keys
 * are accumulated in fp64.
 *
 * Inputs : head in [0, H); Q, K [H,N,d] dtype in TOKEN order; scale [H];
 *          key_label [H,N] (stage 1); query_perm, block_ptr, block_groups
 *          (stage 2); blocks [n_blocks] int32 device array of block indices
 *          (1 <= n_blocks <= nb); mass in (0, 1]; N <= 16776960 (else
 *          SPARSEPR_ERR_UNSUPPORTED).
 * Outputs: lse, routed_mass [n_blocks B_q] fp32; support, support_routed
 *          [n_blocks B_q] int32; pooled, pooled_routed [n_blocks] int32.
 * Workspace: at least 4 n_blocks B_q (N + 1) bytes (the rows' logits and
 *          thresholds); its own, not the stages' workspace size.
 */
int32_t sparsepr_support_stats(const sparsepr_params* params, int32_t head, const void* Q,
                               const void* K, const float* scale, const int32_t* key_label,
                               const int32_t* query_perm, const int32_t* block_ptr,
                               const int32_t* block_groups, const int32_t* blocks,
                               int32_t n_blocks, double mass, float* lse, float* routed_mass,
                               int32_t* support, int32_t* support_routed, int32_t* pooled,
                               int32_t* pooled_routed, void* workspace, size_t workspace_bytes,
                               void* stream);

/*
 * Exact softmax attention over all keys, the operator SparsePR replaces
 * (arxivdaily 2608.18484, English abstract: speedups are over dense
 * attention). O[q] = softmax(tau q K^T) V, lse[q] = log sum exp(tau q K^T),
 * token order. Uses only heads, n_tokens, head_dim, dtype and q_block from
 * params. lse may be NULL. Needs no workspace; queue and queue_bytes as in
 * sparsepr_attend (optional work queue, same results with or without).
 */
int32_t sparsepr_dense_attention(const sparsepr_params* params, const void* Q, const void* K,
                                 const void* V, const float* scale, void* O, float* lse,
                                 void* queue, size_t queue_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* SPARSEPR_H */
