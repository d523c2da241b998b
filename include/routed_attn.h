/*
 * routed_attn.h -- C ABI of the MI355X (gfx950) routed sparse attention
 * library: the routing-attention layer of the Routing Transformer (Roy,
 * Saffar, Vaswani, Grangier, "Efficient Content-Based Sparse Attention with
 * Routing Transformers", TACL 9, 2021).
 *
 * Page citations are to the paperlayer.ai "Source-linked AI summary" of that
 * paper ("summary §N") and to its arXiv abstract.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Every tensor pointer is a DEVICE pointer to contiguous row-major memory
 *    owned by the caller, aligned to 16 bytes (the kernels use 16-byte vector
 *    accesses); a required pointer that is NULL or misaligned returns
 *    RT_EINVAL.  Optional pointers (documented as such) may be NULL.  Token tensors are [B][H][n][d] (d fastest);
 *    centroids [H][k][d] float32; inverse norms [B][H][n] float32;
 *    memberships idx [B][H][k][w] int32; lse [B][H][k][w] float32;
 *    scores [B][H][k][n] float32.
 *  - `dtype` is RT_F32 (float32) or RT_BF16 (bfloat16 bit patterns); it
 *    applies to every token tensor of the call.  Arithmetic is float32
 *    (bf16 matrix products accumulate in float32).
 *  - `stream` is a hipStream_t (NULL = the legacy default stream).  Every
 *    call only enqueues work on it and returns; device faults surface at the
 *    caller's next synchronisation.  The library never synchronises, never
 *    allocates, keeps no state between calls and may be called from several
 *    host threads at once.
 *  - Scratch memory is caller-provided: `ws` must point to at least
 *    rt_workspace_bytes(op, ...) bytes of device memory (any alignment of 256
 *    bytes or more), or may be NULL when that size is 0.  The workspace's
 *    contents need not be initialised and are garbage afterwards.  Two calls
 *    in flight at once must not share a workspace.
 *  - All argument checks happen on the host before anything is enqueued; a
 *    failed check returns RT_EINVAL or RT_EUNSUPPORTED and enqueues nothing.
 *    A failed kernel launch returns RT_EHIP.  The text of the last error of
 *    the calling thread is available from rt_last_error().
 *  - Supported shapes: d in {16, 32, 64, 128}; 1 <= w <= n; 1 <= k <= 256;
 *    n < 2^31 / d.  The in-cluster kernels keep a whole cluster in on-chip
 *    memory, which bounds w (beyond it the call returns RT_EUNSUPPORTED):
 *      rt_routed_attn, bf16, shared q/k:    w <= 512 (d <= 64), 256 (d = 128)
 *      rt_routed_attn, bf16, distinct q/k:  w <= 256 (d <= 64), 128 (d = 128)
 *      rt_routed_attn, float32:             w <= 1024
 *      rt_routed_attn_bwd, bf16, shared:    w <= 256 (d <= 64), 128 (d = 128)
 *      rt_routed_attn_bwd, bf16, distinct:  w <= 128 (d <= 64),  64 (d = 128)
 *      rt_routed_attn_bwd, float32:         w <= 64
 */
#ifndef ROUTED_ATTN_H
#define ROUTED_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    RT_OK = 0,
    RT_EINVAL = 1,        /* a null pointer, a non-positive size, w > n, ... */
    RT_EUNSUPPORTED = 2,  /* a legal request outside what the kernels cover  */
    RT_EHIP = 3           /* the HIP runtime refused a launch                 */
} rt_status;

typedef enum { RT_F32 = 0, RT_BF16 = 1 } rt_dtype;

/* Operation ids for rt_workspace_bytes. */
typedef enum {
    RT_OP_ROUTE = 0,
    RT_OP_ROUTED_ATTN = 1,
    RT_OP_LOCAL_ATTN = 2,
    RT_OP_CENTROID_UPDATE = 3,
    RT_OP_ROUTED_ATTN_BWD = 4,
    RT_OP_LOCAL_ATTN_BWD = 5,
    RT_OP_CENTROID_UPDATE_ARGMAX = 6,
    RT_OP_ROUTE_PARTITION = 7,
    RT_OP_ATTN_JS = 8,
    RT_OP_ROUTED_ATTN_UPDATE = 9
} rt_op;

/*
 * rt_route -- normalise, score against the centroids, balanced top-w.
 *   Summary §4 ("Routing attention with clustering"): queries/keys are
 *   unit-normalised and compared with k shared centroids (the O(nkd) routing
 *   comparisons); balanced clusters give each centroid the same number of
 *   tokens.  Summary §1/§2: nearest centroid approximates maximum inner
 *   product search.
 *
 *   qk        [B][H][n][d] dtype, the shared query/key vectors (raw).
 *   mu        [H][k][d] float32 centroids (read only).
 *   inv_norm  out [B][H][n] float32: 1 / max(||qk_t||_2, 1e-12).
 *   idx       out [B][H][k][w] int32: for centroid c, the w positions whose
 *             unit vector has the largest inner product with mu_c (equal
 *             scores: lower position first), listed in ascending position.
 *             Scores are float32-accurate (the bf16 path splits mu into three
 *             bf16 terms so that no precision is lost in the products).
 *   member_mask  optional out (NULL to skip) [B][H][n][ceil(k/32)] uint32: bit
 *             c of token t is set iff t is a member of cluster c (the input
 *             rt_routed_attn would otherwise build from idx).
 *   qk_hat    optional out (NULL to skip) [B][H][n][d] dtype: qk * inv_norm.
 *   scores    optional out (NULL to skip) [B][H][k][n] float32: the inner
 *             products <qk_t * inv_norm_t, mu_c>.  When NULL the scores live
 *             in the workspace.
 *   ws        rt_workspace_bytes(RT_OP_ROUTE, ...) bytes (0 when scores != NULL).
 */
rt_status rt_route(const void *qk, int dtype, const float *mu, int B, int H, int n, int d, int k,
                   int w, float *inv_norm, int32_t *idx, uint32_t *member_mask, void *qk_hat,
                   float *scores, void *ws, size_t ws_bytes, void *stream);

/*
 * rt_route_noalloc -- rt_route without a workspace, for callers that cannot
 *   allocate device memory: code under HIP graph capture, tight serving loops,
 *   harnesses that forbid allocation.  Same kernels and results as rt_route
 *   (bit for bit); the scores live in a static device array of
 *   RT_ROUTE_NOALLOC_MAX_SCORES float32 (64 MiB) that the library holds on
 *   every GPU it runs on until the process ends.  The array's address is looked
 *   up on the first call on each device; the stream must belong to the current
 *   device.
 *   Arguments as rt_route (no scores output, no workspace).
 *   B*H*k*n above RT_ROUTE_NOALLOC_MAX_SCORES: RT_EUNSUPPORTED, nothing
 *   launched.  Calls that overlap on one GPU (other streams, other threads)
 *   share the array and race: serialise them.  No allocation of any kind.
 */
#define RT_ROUTE_NOALLOC_MAX_SCORES (16 * 1024 * 1024)
rt_status rt_route_noalloc(const void *qk, int dtype, const float *mu, int B, int H, int n, int d,
                           int k, int w, float *inv_norm, int32_t *idx, uint32_t *member_mask,
                           void *qk_hat, void *stream);

/*
 * rt_routed_attn -- attention inside each cluster, scatter-added back.
 *   Summary §3: softmax-normalised attention over the permitted keys, the
 *   output is the weighted sum of values, and an autoregressive query sees no
 *   later position.  Summary §4: only query-key pairs of the same cluster are
 *   considered.  Queries and keys are used unit-normalised: the logit of
 *   members (r, s) is scale * <q_r, k_s> * q_inv[r] * k_inv[s].
 *
 *   q, kk, v   [B][H][n][d] dtype.  kk may equal q (shared query/key).
 *   q_inv, k_inv  [B][H][n] float32 inverse norms (e.g. from rt_route);
 *              pass NULL for both to attend with q and kk as given.
 *   idx        [B][H][k][w] int32 memberships: each row strictly increasing
 *              positions in [0, n) (rows that are not give unspecified
 *              results; out-of-range values are clamped, never dereferenced).
 *   member_mask   optional [B][H][n][ceil(k/32)] uint32 membership bits
 *              consistent with idx (as rt_route emits them); NULL: built from
 *              idx in the workspace.  The bits decide how many rows each
 *              token gets: bits that are not those of this idx give wrong
 *              outputs, and a smaller buffer is read out of bounds (the
 *              library sees only the pointer).
 *   causal     1: member s is visible to member r iff pos(s) <= pos(r);
 *              0: every member sees every member.
 *   out        out [B][H][n][d] of element type out_dtype (RT_F32 or RT_BF16,
 *              independent of dtype): for each token, the sum of its output
 *              rows over the clusters that hold it, in ascending centroid
 *              order (float32 accumulation, one final rounding); 0 for a
 *              token that no cluster holds.  Must not alias an input.  The
 *              bf16 output is exactly the round-to-nearest-even of the
 *              float32 output.
 *   lse        optional out (NULL to skip) [B][H][k][w] float32: natural log
 *              of each row's softmax denominator, max + log(sum exp).
 *   sum_q, sum_k  optional outs (NULL to skip) [B][H][k][d] float32: per
 *              cluster, the sum over its members of q*q_inv (resp. kk*k_inv),
 *              the input of rt_centroid_update_sums.
 *   ws         rt_workspace_bytes(RT_OP_ROUTED_ATTN, ...) bytes: membership
 *              bits and float32 partial rows of tokens that several clusters
 *              hold.
 *   Deterministic: repeated calls give bit-identical results.
 */
rt_status rt_routed_attn(const void *q, const void *kk, const void *v, int dtype,
                         const float *q_inv, const float *k_inv, const int32_t *idx,
                         const uint32_t *member_mask, int B, int H, int n, int d, int k, int w,
                         float scale, int causal, void *out, int out_dtype, float *lse,
                         float *sum_q, float *sum_k, void *ws, size_t ws_bytes, void *stream);

/*
 * rt_routed_attn_update -- rt_routed_attn followed by the centroid update of
 *   rt_centroid_update_sums from the same memberships, with the update run in
 *   the launch that scatters the output (one launch fewer than the two calls).
 *   Summary §4 (online k-means: the centroids move towards the mean of their
 *   members as an exponential moving average): the member sums of the queries
 *   and keys (q*q_inv, kk*k_inv over each cluster's rows, all batch rows) give
 *       mu_c <- lambda * mu_c + (1 - lambda)/2 * (S_Q[c] + S_K[c]).
 *   The attention uses idx, computed with mu before the update; results are
 *   those of rt_routed_attn then rt_centroid_update_sums, bit for bit.
 *   mu         [H][k][d] float32, updated in place; lambda in [0, 1].
 *   Other arguments as rt_routed_attn (no sum outputs).
 *   ws: rt_workspace_bytes(RT_OP_ROUTED_ATTN_UPDATE, ...) bytes.
 */
rt_status rt_routed_attn_update(const void *q, const void *kk, const void *v, int dtype,
                                const float *q_inv, const float *k_inv, const int32_t *idx,
                                const uint32_t *member_mask, int B, int H, int n, int d, int k,
                                int w, float scale, int causal, void *out, int out_dtype,
                                float *lse, float *mu, float lambda, void *ws, size_t ws_bytes,
                                void *stream);

/*
 * rt_cluster_attn, rt_scatter_rows -- rt_routed_attn in its two stages, for
 *   callers that schedule them apart (e.g. other work between them) and for
 *   timing each.  The Spec names the stages: attention inside each cluster,
 *   then the scatter-add of the cluster rows back to token order.
 *
 * rt_cluster_attn: gathers each cluster's rows and runs the in-cluster
 *   attention (Summary §3, §4 as for rt_routed_attn).  Rows of tokens that
 *   one cluster holds are written to `out` (final); rows of tokens that
 *   several clusters hold go to the workspace for rt_scatter_rows.  Rows of
 *   tokens that no cluster holds are not written.  member_mask is required
 *   (the bits rt_route wrote for idx).  Other arguments as rt_routed_attn.
 *
 * rt_scatter_rows: completes `out` after rt_cluster_attn with the same
 *   member_mask, ws, B, H, n, d, k, w, dtype (the attention's input dtype)
 *   and out_dtype: tokens held by several clusters get the sum of their rows
 *   in ascending centroid order, tokens held by none get zeros.  With mu !=
 *   NULL it also applies rt_centroid_update_sums's update from sum_q (and
 *   sum_k; NULL counts sum_q twice), both [B][H][k][d] float32 as
 *   rt_cluster_attn wrote them; lambda in [0, 1].
 *   The two calls in this order, on one stream, give rt_routed_attn's (and,
 *   with mu, rt_routed_attn_update's) results bit for bit.
 *   ws: rt_workspace_bytes(RT_OP_ROUTED_ATTN, ...) bytes, the same buffer for
 *   both calls, untouched in between.
 */
rt_status rt_cluster_attn(const void *q, const void *kk, const void *v, int dtype,
                          const float *q_inv, const float *k_inv, const int32_t *idx,
                          const uint32_t *member_mask, int B, int H, int n, int d, int k, int w,
                          float scale, int causal, void *out, int out_dtype, float *lse,
                          float *sum_q, float *sum_k, void *ws, size_t ws_bytes, void *stream);
rt_status rt_scatter_rows(const uint32_t *member_mask, int dtype, int B, int H, int n, int d,
                          int k, int w, void *out, int out_dtype, float *mu, const float *sum_q,
                          const float *sum_k, float lambda, void *ws, size_t ws_bytes,
                          void *stream);

/*
 * rt_routed_attn_split -- rt_routed_attn for queries and keys routed on their
 *   own (distinct query and key vectors, each given to rt_route with the same
 *   centroids).
 *   Summary §4: queries and keys are clustered by shared centroids and only
 *   pairs in the same cluster are considered; content-based sparsity also
 *   serves data with no order, so there is no causal mask here.  Cluster c's
 *   queries (idx_q[c]) attend to cluster c's keys and values (idx_k[c]) with
 *   logit scale * <q_r, k_s> * q_inv[r] * k_inv[s].
 *   idx_q, idx_k  [B][H][k][w] int32 memberships as in rt_routed_attn (each row
 *              strictly increasing; out-of-range values are clamped).
 *   q_mask     optional membership bits of idx_q (the queries' rt_route);
 *              NULL: built from idx_q in the workspace.
 *   out        out [B][H][n][d] out_dtype: for each query token, the sum of its
 *              rows over the clusters whose queries hold it (ascending centroid
 *              order); 0 for a token that no query cluster holds.
 *   lse        optional out [B][H][k][w]: per query row, as in rt_routed_attn.
 *   sum_q, sum_k  optional outs [B][H][k][d]: sums of the unit query rows of
 *              idx_q and of the unit key rows of idx_k (rt_centroid_update_sums).
 *   Other arguments, the workspace (RT_OP_ROUTED_ATTN) and the limits on w are
 *   those of rt_routed_attn with distinct q and kk.  Deterministic.
 */
rt_status rt_routed_attn_split(const void *q, const void *kk, const void *v, int dtype,
                               const float *q_inv, const float *k_inv, const int32_t *idx_q,
                               const int32_t *idx_k, const uint32_t *q_mask, int B, int H, int n,
                               int d, int k, int w, float scale, void *out, int out_dtype,
                               float *lse, float *sum_q, float *sum_k, void *ws, size_t ws_bytes,
                               void *stream);

/*
 * rt_local_attn -- sliding-window attention for the non-routed heads.
 *   Abstract and summary §6: local attention over a window of recent
 *   positions (windows 512 and 1024 are the ones the pages report).
 *   out_i = sum_j softmax_j(scale * <q_i, k_j>) v_j over j in
 *   [max(0, i-window+1), i] (causal = 1).  causal = 0 uses the symmetric band
 *   |i - j| < window.
 *
 *   q, kk, v  [B][H][n][d] dtype (raw, not normalised).
 *   out       [B][H][n][d] of element type out_dtype (RT_F32 or RT_BF16); must
 *             not alias an input.  window >= 1.  No workspace.
 */
rt_status rt_local_attn(const void *q, const void *kk, const void *v, int dtype, int B, int H,
                        int n, int d, int window, float scale, int causal, void *out,
                        int out_dtype, void *stream);

/*
 * rt_centroid_update -- one online k-means step of the shared centroids.
 *   Summary §2/§4: centroids are shared by queries and keys and across
 *   sequences and are learned online by mini-batch spherical k-means.  The
 *   pages do not print the update; this library applies the exponential
 *   moving average
 *       mu_c <- lambda * mu_c + (1 - lambda)/2 * (S_Q[c] + S_K[c]),
 *   S_Q[c] = sum over every batch row b and every member t of cluster c of
 *   q_t * q_inv_t (likewise S_K with kk, k_inv), without renormalisation.
 *
 *   mu      in/out [H][k][d] float32, updated in place.
 *   q, q_inv   [B][H][n][d] dtype and [B][H][n] float32.
 *   kk, k_inv  the key side; pass kk = NULL (and k_inv = NULL) when keys are
 *              the queries (shared QK): then S_K = S_Q.
 *   idx     [B][H][k][w] int32 memberships (as for rt_routed_attn).
 *   lambda  in [0, 1].  Deterministic (fixed summation order).  No workspace.
 */
rt_status rt_centroid_update(float *mu, const void *q, const float *q_inv, const void *kk,
                             const float *k_inv, int dtype, const int32_t *idx, int B, int H, int n,
                             int d, int k, int w, float lambda, void *stream);

/*
 * rt_centroid_update_sums -- the same update as rt_centroid_update from the
 *   per-cluster member sums rt_routed_attn emits (sum_q, sum_k [B][H][k][d]
 *   float32, summed here over b in ascending order); sum_k = NULL when keys
 *   are the queries (then S_K = S_Q).  mu [H][k][d] updated in place.
 */
rt_status rt_centroid_update_sums(float *mu, const float *sum_q, const float *sum_k, int B, int H,
                                  int k, int d, float lambda, void *stream);

/*
 * rt_routed_attn_bwd -- gradients of rt_routed_attn with respect to its
 *   attention inputs, for a fixed membership (routing is a discrete choice
 *   and the centroids move by the update above, not by gradient).
 *
 *   dout            [B][H][n][d] dtype (the dtype of q), gradient of `out`.
 *   lse             [B][H][k][w] float32 from the forward call with the same
 *                   inputs (the softmax is rebuilt from it, not renormalised).
 *   dq_hat, dk_hat  out [B][H][n][d] float32: gradients w.r.t. the
 *                   normalised vectors q*q_inv and kk*k_inv (token order,
 *                   summed over clusters).  With shared QK the gradient of
 *                   the shared normalised vector is dq_hat + dk_hat; pass
 *                   dk_hat = NULL (shared QK only: q == kk, q_inv == k_inv)
 *                   to receive that sum in dq_hat directly (one gradient
 *                   fewer to scatter; summed per cluster row in float32).
 *   dv              out [B][H][n][d] float32.
 *   member_mask     [B][H][n][ceil(k/32)] uint32 or NULL, as for rt_routed_attn:
 *                   the membership bits rt_route wrote for this idx (saves
 *                   building them again); NULL builds them from idx in ws.
 *   The three gradients are float32, distinct, and alias no input.  Tokens
 *   held by no cluster get zero rows.  Other arguments as for rt_routed_attn.
 *   ws: rt_workspace_bytes(RT_OP_ROUTED_ATTN_BWD, ...) bytes (membership bits
 *   and the float32 partial rows of tokens that several clusters hold).
 *   Deterministic: clusters are summed per token in ascending centroid order.
 */
rt_status rt_routed_attn_bwd(const void *q, const void *kk, const void *v, int dtype,
                             const float *q_inv, const float *k_inv, const int32_t *idx,
                             const uint32_t *member_mask, const float *lse, const void *dout, int B, int H, int n, int d, int k,
                             int w, float scale, int causal, float *dq_hat, float *dk_hat,
                             float *dv, void *ws, size_t ws_bytes, void *stream);

/*
 * rt_in_proj -- the heads' inputs of one layer from the layer input.
 *   Summary §3: a self-attention layer maps n vectors of dimension d_model
 *   to queries, keys and values with learned linear maps; here one product
 *   gives the shared query/key and the values of the R routed heads and the
 *   queries, keys and values of the L local heads:
 *       [qk | v | q_l | k_l | v_l] = x W_in^T   (bf16, float32 accumulation,
 *                                                one rounding per element).
 *   x      [B][n][dm] bf16 (token-major layer input).
 *   w_in   [(2R + 3L) d][dm] bf16: rows R*d of qk heads, R*d of v heads, then
 *          L*d each of local q, k and v heads (head h, dim i = row h*d + i).
 *   qk, v  out [B][R][n][d] bf16; q_l, k_l, v_l out [B][L][n][d] bf16 (NULL
 *          when L = 0).  Outputs must not alias x or w_in.  No workspace.
 *   Sizes: d in {16, 32, 64, 128}, dm a positive multiple of 8, R >= 1,
 *   L >= 0, B*n*max(dm, (2R+3L)d) < 2^31.
 */
rt_status rt_in_proj(const void *x, const void *w_in, int B, int n, int dm, int d, int R, int L,
                     void *qk, void *v, void *q_l, void *k_l, void *v_l, void *stream);

/*
 * rt_out_proj -- the layer output: y = x + [o_r | o_l] W_o^T.
 *   The heads' outputs (routed heads, then local heads, concatenated per
 *   token) mapped back to d_model and added to the residual stream
 *   (summary §3, §5: a stack of such layers).
 *   o_r    [B][R][n][d] bf16 (routed heads' outputs); o_l [B][L][n][d] bf16
 *          (NULL when L = 0).
 *   w_o    [dm][(R + L) d] bf16.
 *   x      [B][n][dm] bf16 residual, or NULL for none.  y [B][n][dm] bf16
 *          out; y may be x (each element's residual is read before it is
 *          written), must not alias o_r, o_l or w_o.  Float32 accumulation
 *          and residual add, one rounding per element.  No workspace.
 */
rt_status rt_out_proj(const void *o_r, const void *o_l, const void *w_o, const void *x, int B,
                      int n, int dm, int d, int R, int L, void *y, void *stream);

/*
 * The layer's backward (gradients of one layer for the gradient dy of its
 * output, membership held fixed): rt_out_proj_bwd -> rt_routed_attn_bwd on
 * the routed heads and rt_local_attn_bwd on the local heads ->
 * rt_normalize_bwd (the routed heads' shared q/k) -> rt_in_proj_bwd.
 */

/*
 * rt_local_attn_bwd -- gradients of rt_local_attn with respect to q, k, v.
 *   Summary §3 (softmax attention) over the local band of rt_local_attn.  For
 *   the output gradient dout and P the softmax rows:
 *     dv_j = sum_i P_ij dout_i,
 *     dl_ij = P_ij (<dout_i, v_j> - sum_j' P_ij' <dout_i, v_j'>),
 *     dq_i = scale sum_j dl_ij k_j,   dk_j = scale sum_i dl_ij q_i.
 *   q, kk, v, dout  [B][H][n][d] bf16 (RT_BF16 only), d in {64, 128}.
 *   dq, dk, dv      out [B][H][n][d] float32, distinct, aliasing no input.
 *   The softmax is rebuilt from q, k (no state from the forward call); P and
 *   dl are rounded to bf16 for the products, accumulation is float32.
 *   ws: rt_workspace_bytes(RT_OP_LOCAL_ATTN_BWD, B, H, n, d, 1, 1) bytes
 *   (each query's log-sum-exp and sum_j P dP).  Deterministic (no atomics).
 */
rt_status rt_local_attn_bwd(const void *q, const void *kk, const void *v, const void *dout,
                            int dtype, int B, int H, int n, int d, int window, float scale,
                            int causal, float *dq, float *dk, float *dv, void *ws,
                            size_t ws_bytes, void *stream);

/*
 * rt_normalize_bwd -- gradient through the unit normalisation of rt_route.
 *   Summary §4: queries and keys are used unit-normalised,
 *   x^ = x / max(||x||, 1e-12).  For the gradients g1 and g2 (NULL for none)
 *   of x^ (shared query/key: the query's and the key's gradients add),
 *   with g = g1 + g2:  dx = (g - x^ <x^, g>) / ||x||, and dx = g / 1e-12 on
 *   rows whose norm is below 1e-12 (the clamp is then constant).
 *   x         [rows][d] dtype (the raw vectors given to rt_route).
 *   inv_norm  [rows] float32 from rt_route.
 *   g1, g2    [rows][d] float32.   dx out [rows][d] float32; dx may be g1 or
 *             g2 (a row is read whole before it is written), not x.
 */
rt_status rt_normalize_bwd(const void *x, int dtype, const float *inv_norm, const float *g1,
                           const float *g2, long rows, int d, float *dx, void *stream);

/*
 * rt_out_proj_bwd -- gradients of rt_out_proj.
 *   For dy, the gradient of y = x + [o_r | o_l] W_o^T:
 *     do = dy W_o (split into the routed and the local heads, head-major),
 *     dw_o = dy^T [o_r | o_l];
 *   the gradient of the residual x is dy itself (rt_in_proj_bwd adds it).
 *   dy     [B][n][dm] bf16.  o_r, o_l, w_o as in rt_out_proj.
 *   do_r   out [B][R][n][d] bf16; do_l out [B][L][n][d] bf16 (NULL when
 *          L = 0): rounded once, as rt_routed_attn_bwd and rt_local_attn_bwd
 *          take them.   dw_o out [dm][(R + L) d] float32.
 *   bf16 products, float32 accumulation; outputs alias no input.
 *   ws     optional float32 workspace (NULL: none) of ws_bytes: with room for
 *          at least two dm x (R + L) d partial products, dw_o's contraction
 *          over the B n tokens is split over more workgroups and the parts
 *          are added in a fixed order (results independent of scheduling;
 *          rt_proj_bwd_workspace_bytes gives the size that lets both layer
 *          gradients split fully).
 */
rt_status rt_out_proj_bwd(const void *dy, const void *o_r, const void *o_l, const void *w_o,
                          int B, int n, int dm, int d, int R, int L, void *do_r, void *do_l,
                          float *dw_o, void *ws, size_t ws_bytes, void *stream);

/*
 * rt_in_proj_bwd -- gradients of rt_in_proj.
 *   For the heads' gradients dC = [dqk | dv | dq_l | dk_l | dv_l] (laid out
 *   as rt_in_proj writes the heads):
 *     dx = dC W_in + dres,   dw_in = dC^T x.
 *   x, w_in  as in rt_in_proj.
 *   dqk, dv  [B][R][n][d] float32; dq_l, dk_l, dv_l [B][L][n][d] float32
 *            (NULL when L = 0).  dC is rounded to bf16 as the products'
 *            operand; float32 accumulation.
 *   dres     [B][n][dm] bf16 or NULL: a gradient added to dx (the residual's,
 *            i.e. the dy given to rt_out_proj_bwd).
 *   dx       out [B][n][dm] float32;  dw_in out [(2R + 3L) d][dm] float32.
 *   ws       optional workspace as in rt_out_proj_bwd, for dw_in.
 *   Outputs alias no input.
 */
rt_status rt_in_proj_bwd(const void *x, const void *w_in, const float *dqk, const float *dv,
                         const float *dq_l, const float *dk_l, const float *dv_l, const void *dres,
                         int B, int n, int dm, int d, int R, int L, float *dx, float *dw_in,
                         void *ws, size_t ws_bytes, void *stream);

/* Workspace in bytes that lets the weight gradients of rt_out_proj_bwd and
 * rt_in_proj_bwd split their contraction fully at these sizes (0: they would
 * not split; (size_t)-1: invalid sizes). */
size_t rt_proj_bwd_workspace_bytes(int B, int n, int dm, int d, int R, int L);

/*
 * Variants: readings the pages leave open, built beside the main path.
 */

/*
 * rt_local_attn_blocked -- blocked (chunked) local attention.
 *   The local heads' attention (arXiv abstract; summary §6) with the window
 *   taken as blocks: the sequence is cut into blocks of `block` positions and
 *   position i sees the positions of its own block and of the `lookback`
 *   blocks before it that are not later than i (causal).  Softmax attention as
 *   in rt_local_attn; arguments, layouts and limits as there.
 */
rt_status rt_local_attn_blocked(const void *q, const void *kk, const void *v, int dtype, int B,
                                int H, int n, int d, int block, int lookback, float scale,
                                void *out, int out_dtype, void *stream);

/*
 * rt_centroid_update_argmax -- the centroid update with nearest-centroid
 *   assignments instead of the balanced memberships.
 *   Summary §2, §4 (online spherical k-means): each unit-normalised query and
 *   each key counts once, for the centroid with the largest inner product
 *   (ties: the lower index); S_Q[c], S_K[c] are those sums over the whole
 *   batch (ascending batch row and position) and
 *       mu_c <- lambda * mu_c + (1 - lambda)/2 * (S_Q[c] + S_K[c]).
 *   mu      [H][k][d] float32, updated in place.
 *   q, kk   [B][H][n][d] dtype, raw; kk NULL (or == q) for shared q/k.
 *   ws: rt_workspace_bytes(RT_OP_CENTROID_UPDATE_ARGMAX, B, H, n, d, k, 1)
 *   bytes.  Deterministic (fixed summation order, no atomics).
 */
rt_status rt_centroid_update_argmax(float *mu, const void *q, const void *kk, int dtype, int B,
                                    int H, int n, int d, int k, float lambda, void *ws,
                                    size_t ws_bytes, void *stream);

/*
 * rt_route_partition -- partition-style balanced routing: every token in
 *   exactly one cluster, every cluster w = n / k tokens.
 *   Summary §4 (a token's assigned cluster; balanced clusters; the routing
 *   cost of a sort): the tokens of a (batch, head) are ordered by (nearest
 *   centroid, descending score against it, position) and cut into k
 *   consecutive groups of w; group c is cluster c.
 *   qk, mu, inv_norm as in rt_route.  idx out [B][H][k][n/k] int32, each row in
 *   ascending position; member_mask optional out as in rt_route (one bit per
 *   token).  n a multiple of k, n <= 16384, k <= 256.
 *   ws: rt_workspace_bytes(RT_OP_ROUTE_PARTITION, ...) bytes.
 */
rt_status rt_route_partition(const void *qk, int dtype, const float *mu, int B, int H, int n,
                             int d, int k, float *inv_norm, int32_t *idx, uint32_t *member_mask,
                             void *ws, size_t ws_bytes, void *stream);

/*
 * ---- Incremental decode ------------------------------------------------------------------
 * Summary Appendix A generates one token at a time; Summary §3 (autoregressive
 * factorisation: a query sees only earlier positions) and §4 (routing by the
 * nearest shared centroid) say what one step computes.  The pages define no
 * decode step, so this reading is used: the new token joins the one cluster
 * whose centroid is nearest (largest inner product of the unit vectors, ties to
 * the lower index); its raw key row, inverse norm, value and position are
 * appended to that cluster's cache; its query attends, with the routed logit
 * scale * <q_hat, k_hat>, to every entry of that cache (all earlier positions
 * or itself).  The local heads keep the last `window` keys and values in a ring.
 *
 * Every decode entry point takes bfloat16 rows (no dtype argument) and keeps
 * them in bfloat16 caches owned by the caller:
 *   cache_k    [B][H][k][cap][d] bf16  raw key rows of each cluster
 *   cache_inv  [B][H][k][cap]    float32 their inverse norms 1 / max(|x|, 1e-12)
 *   cache_v    [B][H][k][cap][d] bf16  values
 *   cache_pos  [B][H][k][cap]    int32 positions
 *   cache_len  [B][H][k]         int32 entries in use (the first cache_len rows)
 *   ring_k, ring_v [B][H][window][d] bf16: position p at slot p % window.
 * cap and window are at most 16384 (the step keeps its logits on chip).  A
 * step with B*H pieces of work is bound by launch latency; steps on one stream
 * run in order, which is what the cache updates need.
 */

/*
 * rt_decode_fill -- cluster caches from a prefill membership.
 *   qk, v      [B][H][n][d] bf16, the prefill's shared query/key rows and values.
 *   inv_norm   [B][H][n] float32 and idx [B][H][k][w] int32 as written by rt_route
 *              (or rt_route_partition with w = n / k).
 *   Writes rows 0..w-1 of every cluster's cache (row r: position idx[.., c, r])
 *   and cache_len = w; rows w..cap-1 are left as they are.  cap >= w.
 */
rt_status rt_decode_fill(const void *qk, const float *inv_norm, const void *v, const int32_t *idx,
                         int B, int H, int n, int d, int k, int w, int cap, void *cache_k,
                         float *cache_inv, void *cache_v, int32_t *cache_pos, int32_t *cache_len,
                         void *stream);

/*
 * rt_decode_ring_fill -- the local heads' rings from a prefill: slot s gets the
 *   key and value of the last position p < n with p % window == s (slots with no
 *   such position are left as they are).
 *   kk, v  [B][H][n][d] bf16 (the local heads' keys and values).
 */
rt_status rt_decode_ring_fill(const void *kk, const void *v, int B, int H, int n, int d,
                              int window, void *ring_k, void *ring_v, void *stream);

/*
 * rt_decode_routed -- one routed decode step for the token at position t.
 *   qk_t, v_t  [B][H][d] bf16: the new token's shared query/key row and value.
 *   mu         [H][k] unit rows of d float32 (the centroids; not changed).
 *   The caches are read and appended to in place (see above).
 *   out        out [B][H][d] of element type out_dtype (RT_F32 or RT_BF16).
 *   label      optional out [B][H] int32: the chosen cluster.
 *   A cluster whose cache is full (cache_len >= cap) is not written: that
 *   (batch, head) gets label -1 and an all-NaN output row, and its caches are
 *   unchanged; the other (batch, head) pairs are unaffected.  The caller keeps
 *   room (cap >= fill + steps bounds every cluster).
 */
rt_status rt_decode_routed(const void *qk_t, const void *v_t, const float *mu, int B, int H, int d,
                           int k, int cap, void *cache_k, float *cache_inv, void *cache_v,
                           int32_t *cache_pos, int32_t *cache_len, int t, float scale, void *out,
                           int out_dtype, int32_t *label, void *stream);

/*
 * rt_decode_local -- one local decode step for the token at position t >= 0:
 *   writes k_t, v_t ([B][H][d] bf16) to slot t % window of the rings, then the
 *   query q_t attends with logit scale * <q, k> (raw rows) to positions
 *   max(0, t - window + 1) .. t, which the rings must hold (Summary §6, Abstract:
 *   the local heads' sliding window).
 *   out  out [B][H][d] of element type out_dtype.
 */
rt_status rt_decode_local(const void *q_t, const void *k_t, const void *v_t, int B, int H, int d,
                          int window, void *ring_k, void *ring_v, int t, float scale, void *out,
                          int out_dtype, void *stream);

/*
 * rt_attn_js -- Jensen-Shannon divergence between local and routed attention,
 *   a diagnostic (Summary §6 compares the two by this divergence, natural log,
 *   at most ln 2).  For each row r of each cluster c, with i = idx[c][r]:
 *     P = the local attention distribution of query i (softmax over i's window
 *         of scale_l * <q_l[i], k_l[j]>, as rt_local_attn computes it),
 *     Q = the routed distribution of that row (softmax over the cluster's keys
 *         row r sees of scale_r * <qk[i], qk[s]> * q_inv[i] * q_inv[s]),
 *     js[c][r] = 1/2 KL(P || M) + 1/2 KL(Q || M), M = (P + Q) / 2.
 *   qk         [B][H][n][d] bf16, the routing heads' shared query/key rows;
 *              q_inv [B][H][n] float32 and idx [B][H][k][w] as from rt_route.
 *   q_l, k_l   [B][H][n][d] bf16, a local head's queries and keys (head h of
 *              the local heads is compared with head h of the routing heads).
 *   causal     1: row r sees the cluster's rows 0..r and i's window is
 *              [i - window + 1, i]; 0: all rows and |i - j| < window.
 *   js         out [B][H][k][w] float32, in [0, ln 2].
 *   ws: rt_workspace_bytes(RT_OP_ATTN_JS, B, H, n, d, k, w) bytes (the local
 *   heads' log-denominators and a discarded attention output).
 *   Limits: w <= 128 at d = 128, 256 at d = 64, 512 below.  P's denominator
 *   is the local kernel's (bf16 probabilities summed in float32), so values
 *   agree with an exact evaluation to a few 1e-3.
 */
rt_status rt_attn_js(const void *qk, const float *q_inv, const int32_t *idx, const void *q_l,
                     const void *k_l, int B, int H, int n, int d, int k, int w, int window,
                     float scale_r, float scale_l, int causal, float *js, void *ws,
                     size_t ws_bytes, void *stream);

/* Workspace size in bytes for operation `op` at these sizes (0 if none,
 * (size_t)-1 if the sizes are invalid). */
size_t rt_workspace_bytes(int op, int B, int H, int n, int d, int k, int w);

/* Static text for a status code. */
const char *rt_status_string(int status);

/* Text of the calling thread's last error ("" if none). */
const char *rt_last_error(void);

/* Library version as MAJOR*10000 + MINOR*100 + PATCH. */
int rt_version(void);

#ifdef __cplusplus
}
#endif

#endif /* ROUTED_ATTN_H */
