/*
 * losa.h -- C ABI of the retained-mass block-sparse self-attention library
 * (gfx950 / MI355X).
 *
 * The three calls follow page 1, "LoSA: Near-Lossless Sparse Attention for
 * Training-Free Video Diffusion Acceleration":
 *
 *   losa_block_mass   exact block attention masses      (Motivation Summary;
 *                     Methodology Summary, one-time pattern construction)
 *   losa_select       retained-mass (top-p) key-block lists, CSR
 *                     (Methodology Summary, one-time pattern construction)
 *   losa_sparse_attn  softmax attention over the frozen lists only
 *                     (Methodology Summary, sparse attention with a frozen
 *                     pattern)
 *
 * The further calls below (each cites the page it follows) build the
 * patterns in other ways or maintain them: dense attention with the masses
 * in one pass, masses within given lists, pooled proxy masses, online block
 * thresholding, the query-key drift that triggers a refresh, and the
 * per-head merge of refreshed lists.
 *
 * Conventions shared by every call
 * --------------------------------
 * Memory.  Every pointer named Q, K, V, O, M, P, row_ptr, col_idx, order,
 *   ws, kept, kept_count, kept_mask, Q_ref, K_ref, drift, refresh, take_b
 *   (and the _a/_b list sets) is DEVICE memory owned by the caller; the
 *   library allocates nothing and keeps no pointer after a call returns.  The
 *   only host pointers are the losa_shape, the p arrays of losa_select and
 *   losa_select_noalloc, the theta arrays of losa_select_threshold and
 *   losa_sparse_attn_threshold and the size_t out-parameters.
 * Streams.  Work is enqueued on `stream` (0 = the null stream) and the call
 *   returns without waiting.  Outputs are valid once the stream reaches them.
 * Errors.  Argument checks run on the host before any HIP call; a failed
 *   check returns its status and enqueues nothing.  LOSA_ERR_HIP reports a
 *   failed launch (hipGetLastError after the launches).  After any error the
 *   contents of the output buffers are unspecified.  No call throws.
 * Threads.  Calls are thread-safe.  The only mutable global state is the
 *   per-device address of losa_select_noalloc's scratch array, looked up
 *   once per device under a lock.  Calls on one stream run in order; two
 *   calls writing the same buffers on different streams race.
 *
 * Tensor layout.  Q, K, V (and O) are [batch, heads, tokens_alloc, head_dim]
 *   with the element strides given in losa_shape (batch, head, token), the
 *   head_dim axis contiguous.  Rows tokens..tokens_alloc-1 are padding: they
 *   are never keys, never counted as queries, and O is written as 0 there.
 *   Base pointers must be 16-byte aligned and strides multiples of 8 (bf16)
 *   or 4 (f32) elements.
 * Blocks.  n_q = ceil(tokens / q_block) query blocks and n_k = ceil(tokens /
 *   k_block) key blocks per (batch, head); the last block of each may be
 *   partial.  A row r = (b * heads + h) * n_q + i names query block i of
 *   head h of batch b.
 */
#ifndef LOSA_H
#define LOSA_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define LOSA_ABI_VERSION 1
/* Largest n_k accepted (key blocks per head), and largest head count that may
 * carry its own p in losa_select. */
#define LOSA_MAX_KEY_BLOCKS 4096
#define LOSA_MAX_HEADS_P 128
/* Size of the device scratch array behind losa_select_noalloc (32 MiB). */
#define LOSA_SELECT_SCRATCH_BYTES ((size_t)32 << 20)

typedef enum losa_status {
  LOSA_OK = 0,
  LOSA_ERR_NULL = 1,        /* a required pointer is NULL                       */
  LOSA_ERR_INVALID_ARG = 2, /* a size, stride, alignment or parameter is wrong  */
  LOSA_ERR_UNSUPPORTED = 3, /* well-formed but outside what is implemented      */
  LOSA_ERR_WORKSPACE = 4,   /* workspace smaller than the matching query says   */
  LOSA_ERR_CAPACITY = 5,    /* col_idx capacity below batch*heads*n_q*n_k       */
  LOSA_ERR_HIP = 6          /* a HIP launch failed                              */
} losa_status;

typedef enum losa_dtype { LOSA_F32 = 0, LOSA_BF16 = 1 } losa_dtype;

typedef struct losa_shape {
  int32_t batch;         /* >= 1                                                 */
  int32_t heads;         /* >= 1                                                 */
  int32_t tokens;        /* N, valid tokens per (batch, head), >= 1               */
  int32_t tokens_alloc;  /* rows allocated per (batch, head), >= n_q*R and n_k*C  */
  int32_t head_dim;      /* d: 64 or 128                                          */
  int32_t q_block;       /* R: 32, 64 or 128                                      */
  int32_t k_block;       /* C: 32, 64 or 128                                      */
  losa_dtype dtype;      /* element type of Q, K and V                            */
  float softmax_scale;   /* <= 0 selects 1/sqrt(head_dim) (the page's scaling)    */
  int32_t reserved;      /* must be 0                                             */
  int64_t q_stride[3];   /* element strides: batch, head, token                   */
  int64_t k_stride[3];
  int64_t v_stride[3];
  int64_t o_stride[3];   /* read by losa_sparse_attn only                         */
} losa_shape;

/* ABI version of the loaded library (LOSA_ABI_VERSION it was built with). */
int32_t losa_abi_version(void);

/* Static, human-readable name of a status code (never NULL). */
const char* losa_status_string(losa_status status);

/* ------------------------------------------------------------------------
 * Exact block attention masses.
 * Motivation Summary (block attention mass M(i, j) = sum over the query
 * rows of block i and the key columns of block j of softmax(Q K^T scale)),
 * in row-mean form: M[b, h, i, j] = that sum divided by the number of valid
 * rows of query block i, so each row of blocks sums to 1.
 *
 * bf16 matrix-core path (head_dim 64/128, q_block 64/128): one pass over
 * K -- per query row and key block, the sum of exp(s - m) against one fixed
 * per-row reference m (the largest score among the first keys each wave of
 * the row's 64-row group reads) goes to the workspace; the row total is the sum
 * of those sums, and M the sums divided by it.  Rows whose sums leave a safe
 * range (a later score far above m) are redone against their exact maximum.
 * Other shapes: two passes over K (the row maximum and the sum against it,
 * then exp(s - max) summed per key block).  Arithmetic: products and sums in
 * fp32 (bf16 inputs are exact in fp32), exponentials in fp32.
 *
 * Dynamic range: m is a score of the row, hence at most its log-sum-exp, so
 * every key whose attention probability is at least 2^-126 (fp32's smallest
 * normal number) contributes a normal fp32 term; keys of smaller probability
 * may be flushed to zero, which changes a mass by at most k_block * 2^-126.
 * Masses at or above about 2^-110 * k_block / 64 are therefore exact to
 * fp32 rounding (relative error far below 1e-3), and smaller ones to
 * k_block * 2^-126 absolute.
 *
 * M: fp32 [batch, heads, n_q, n_k], contiguous (written completely).
 * ws: at least *bytes from losa_block_mass_workspace.  bf16 matrix-core path:
 *    per-(query row, key block) partial sums, 4 * batch*heads*n_q*q_block*n_k
 *    bytes, then K repacked in 32-token chunks.  The partial sums grow with
 *    the square of the token count: 0.81 GB for 12 heads x 32760 tokens
 *    (64-token blocks), 14.3 GB for 40 heads x 75600 tokens (64-token
 *    blocks), 10.6 GB for 24 heads x 118800 tokens (128-token blocks) and
 *    42.4 GB for the same layer with 128-token query and 32-token key blocks.
 *    Other paths: the row maximum and sum, 8 * batch*heads*tokens_alloc bytes.
 * ------------------------------------------------------------------------ */
losa_status losa_block_mass_workspace(const losa_shape* shape, size_t* bytes);
losa_status losa_block_mass(const losa_shape* shape, const void* Q, const void* K, float* M,
                            void* ws, size_t ws_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------
 * Retained-mass block selection.
 * Methodology Summary (one-time pattern construction): per row, sort key
 * blocks by decreasing mass and keep the shortest prefix whose cumulative
 * mass reaches p times the row total.  Exact rules (the page leaves these
 * open):
 *   - ties in mass: the lower block index comes first;
 *   - non-finite, negative and -0 masses count as 0;
 *   - the cumulative sum is evaluated exactly in integers, so the result does
 *     not depend on summation order: with e the binary exponent of the row
 *     maximum (max = f * 2^e, 1/2 <= f < 1), each mass becomes
 *     q_j = ceil(m_j * 2^(51 - e)); P = floor(p * 2^32 + 1/2);
 *     T = ceil(P * sum_j q_j / 2^32); the kept count s is the least prefix
 *     length whose integer sum is >= T (s >= 1; an all-zero row keeps block 0);
 *   - p = 1 (P = 2^32) keeps every block.
 *
 * M: fp32 [batch, heads, n_q, n_k] contiguous (e.g. from losa_block_mass).
 * p: HOST array of n_p doubles in (0, 1]; n_p = 1 (one p for all heads) or
 *    n_p = heads (head h uses p[h]; heads <= LOSA_MAX_HEADS_P).
 * row_ptr: int32 [batch*heads*n_q + 1]; row r's kept blocks are
 *    col_idx[row_ptr[r] .. row_ptr[r+1]-1], in ascending block order.
 * col_idx: int32, col_capacity >= batch*heads*n_q*n_k entries (the worst
 *    case; the used length is row_ptr[last], read back by the caller).
 * order: int32 [batch*heads*n_q] or NULL.  When given, receives the work
 *    order losa_sparse_attn takes: the rows of each head g = b*heads + h are
 *    ranked by kept-block count, descending, ties by row index; the ranks
 *    are cut into groups of 32 (a head's last group may be shorter); the
 *    groups run longest first by their first row's count, ties by head and
 *    then group, each group's rows in rank order.  Per-head budgets are
 *    uneven (HASTE page, head-wise adaptive top-p; Sol-Attn page,
 *    imbalanced dynamic budgets), so long work starts first; a group is one
 *    head's rows, which the workgroups running side by side on one XCD then
 *    share keys and values for.
 * ws: at least *bytes from losa_select_workspace.
 * ------------------------------------------------------------------------ */
losa_status losa_select_workspace(const losa_shape* shape, size_t* bytes);
losa_status losa_select(const losa_shape* shape, const float* M, const double* p, int32_t n_p,
                        int32_t* row_ptr, int32_t* col_idx, int64_t col_capacity, int32_t* order,
                        void* ws, size_t ws_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------
 * Retained-mass block selection that allocates nothing.
 * For callers that cannot allocate device memory or take a workspace: code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation.  Same arguments, rules and results as losa_select (bit for
 * bit), without ws/ws_bytes: the selector's scratch lives in a file-scope
 * device array of LOSA_SELECT_SCRATCH_BYTES in the library, one per GPU the
 * library runs on, held until the process ends.  Its address is looked up
 * (hipGetSymbolAddress) on the first call on each device, with that device
 * current; the stream must belong to the current device.  Nothing in the
 * array needs to start at zero (the kernels clear what they count in).
 *
 * Shapes whose losa_select_workspace exceeds LOSA_SELECT_SCRATCH_BYTES are
 * rejected with LOSA_ERR_WORKSPACE before any HIP call.  Every call on one
 * GPU shares that GPU's array: calls that overlap on one GPU (on different
 * streams, or from different threads without ordering) race and give
 * unspecified lists; calls ordered on one stream are safe.
 * ------------------------------------------------------------------------ */
losa_status losa_select_noalloc(const losa_shape* shape, const float* M, const double* p, int32_t n_p,
                                int32_t* row_ptr, int32_t* col_idx, int64_t col_capacity, int32_t* order,
                                hipStream_t stream);

/* ------------------------------------------------------------------------
 * Frozen-pattern block-sparse attention.
 * Methodology Summary (sparse attention with a frozen pattern): for each
 * query q of query block i, O(q) = sum over retained keys k of
 * exp(s_qk) / sum over retained keys k' of exp(s_qk') * v_k with
 * s = q.k * scale; the retained keys are the valid tokens of the blocks
 * listed for q's row; discarded keys are absent from the denominator; no
 * block is added.  A row with an empty list gets O = 0.
 *
 * row_ptr/col_idx: CSR as produced by losa_select (any order of indices is
 *    accepted; each index must lie in [0, n_k) and occur at most once in a
 *    row -- a repeated index gives an unspecified O, never an access outside
 *    the buffers).
 * order: NULL (rows in index order) or a permutation of the rows giving the
 *    order in which work is dispatched (losa_select's work order).  The
 *    result does not depend on it.
 * O: [batch, heads, tokens_alloc, head_dim] with shape->o_stride, element
 *    type o_dtype (LOSA_BF16 or LOSA_F32).
 * ws: at least *bytes from losa_sparse_attn_workspace (bf16 matrix-core
 *    path: K and V repacked in 32-token chunks as matrix-core operands, zero
 *    beyond the last valid token; 0 bytes otherwise).
 * Arithmetic: bf16 inputs use bf16 matrix products with fp32 accumulation,
 * the probabilities rounded to bf16 for the P.V product; softmax statistics
 * in fp32.  f32 inputs use fp32 throughout.
 * ------------------------------------------------------------------------ */
losa_status losa_sparse_attn_workspace(const losa_shape* shape, size_t* bytes);
losa_status losa_sparse_attn(const losa_shape* shape, const void* Q, const void* K, const void* V,
                             const int32_t* row_ptr, const int32_t* col_idx, const int32_t* order,
                             void* O, losa_dtype o_dtype, void* ws, size_t ws_bytes,
                             hipStream_t stream);

/* ------------------------------------------------------------------------
 * Sparse attention with on-the-fly block thresholding.
 * Sol-Attn page (abstract): the key blocks a query block attends to are
 * chosen while the online softmax runs, by comparing each block's proxy
 * score with a threshold, without materialising a proxy map.  The page gives
 * no rule; this library's reading: the proxy of key block j for query block
 * i is a_j = scale * qbar_i . kbar_j + ln|B_j| -- the pooled score of the
 * block means over valid tokens (see losa_pooled_mass), weighted by the
 * block's valid keys -- and, visiting blocks in index order as the online
 * pass does, block j is kept when a_j >= ln(theta) + max(a_0 .. a_j).  That
 * is losa_select_threshold's rule applied to the pooled proxy masses with
 * their normaliser cancelled, so no proxy matrix is formed or stored: each
 * workgroup decides its row's blocks in LDS, then skips the dropped blocks'
 * K/V loads and products.  O is the softmax attention over the kept blocks'
 * valid tokens (as losa_sparse_attn computes it); the page's correction for
 * the skipped blocks is not applied.  The decision is taken in fp64 (bf16
 * block sums are exact there; the fp32 softmax scale is widened exactly);
 * ln(theta) and the two block-size logarithms are computed on the host.
 *
 * bf16 matrix-core shapes only (head_dim 64/128, q_block 64/128); others
 * return LOSA_ERR_UNSUPPORTED.
 * theta: HOST array of n_theta doubles in (0, 1]; n_theta = 1 or heads.
 * O: as for losa_sparse_attn (rows beyond tokens written as 0).
 * kept_count: int32 [batch*heads*n_q] or NULL: the kept blocks per row.
 * kept_mask: uint32 [batch*heads*n_q][ceil(n_k/32)] or NULL: bit j%32 of
 *    word j/32 of row r is set when block j is kept.
 * ws: at least *bytes from losa_sparse_attn_threshold_workspace: fp64 block
 *    means of Q and K (8 * batch*heads*(n_q + n_k)*head_dim bytes), K and V
 *    repacked as for losa_sparse_attn, then one slot per 64-query tile for
 *    its list of kept blocks (4 * batch*heads*n_q*(q_block/64)*n_k bytes;
 *    only the kept blocks' indices are written).  Nothing of the proxy
 *    scores is stored.
 * ------------------------------------------------------------------------ */
losa_status losa_sparse_attn_threshold_workspace(const losa_shape* shape, size_t* bytes);
losa_status losa_sparse_attn_threshold(const losa_shape* shape, const void* Q, const void* K, const void* V,
                                       const double* theta, int32_t n_theta, void* O, losa_dtype o_dtype,
                                       int32_t* kept_count, uint32_t* kept_mask, void* ws, size_t ws_bytes,
                                       hipStream_t stream);

/* ------------------------------------------------------------------------
 * Dense attention with exact block masses, in one pass (the construction
 * step).  LoSA page, Methodology Summary: the pattern is built once, at a
 * dense step, from exact block masses; Experiments Summary: the
 * construction step's kernel is a full attention pass that also sums the
 * exact block masses.
 * O(q) = softmax over all valid keys of s = q.k * scale, times V (rows in
 * [tokens, n_q*q_block) written as 0, rows beyond not touched); M = exactly
 * what losa_block_mass computes.
 *
 * M: fp32 [batch, heads, n_q, n_k], contiguous (written completely).
 * O: [batch, heads, tokens_alloc, head_dim] with shape->o_stride, element
 *    type o_dtype (LOSA_BF16 or LOSA_F32).
 * ws: at least *bytes from losa_dense_attn_mass_workspace.  bf16
 *    matrix-core path: packed K and V, per-(query row, key block) partial
 *    sums (4 * batch*heads*n_q*q_block*n_k bytes) and, for q_block = 128, two
 *    partial copies of M; other paths: the losa_block_mass workspace.
 * Arithmetic as losa_sparse_attn for O and as losa_block_mass for M.
 * ------------------------------------------------------------------------ */
losa_status losa_dense_attn_mass_workspace(const losa_shape* shape, size_t* bytes);
losa_status losa_dense_attn_mass(const losa_shape* shape, const void* Q, const void* K, const void* V,
                                 float* M, void* O, losa_dtype o_dtype, void* ws, size_t ws_bytes,
                                 hipStream_t stream);

/* ------------------------------------------------------------------------
 * Frozen-pattern sparse attention with the exact masses within the lists.
 * GSRS card (Sparse Attention for Video Generation Acceleration via Growing
 * Sparsity and Reduced Search): after the first top-p search, later ones
 * look only among the blocks an earlier search kept, and the weights they
 * rank are the exact ones the attention pass itself produces.  Reading (the
 * card gives no formula): O is exactly losa_sparse_attn's, and for each row i with listed blocks L
 *   M[b,h,i,j] = (1/valid rows of block i) * sum over valid rows q of block i
 *                and valid keys k of block j of
 *                exp(s_qk) / sum over the valid keys k' of L of exp(s_qk')
 * for j in L (the softmax of the sparse attention itself, summed per block),
 * and 0 for j outside L.  A row with a non-empty list sums to 1; with every
 * block listed M is losa_block_mass's.  losa_select on M with a target p'
 * then keeps a subset of L (for p' < 1) -- the reduced search.
 *
 * Supported: bf16, head_dim 64 or 128, q_block 64 or 128 (the matrix-core
 *    shapes); other shapes return LOSA_ERR_UNSUPPORTED before any HIP call,
 *    from this call and from its workspace query.
 * row_ptr/col_idx/order: as losa_sparse_attn (indices in [0, n_k), each at
 *    most once in a row -- a repeated index gives an unspecified O and M,
 *    never an access outside the buffers).
 * M: fp32 [batch, heads, n_q, n_k], contiguous (written completely).
 * O: [batch, heads, tokens_alloc, head_dim] with shape->o_stride, element
 *    type o_dtype (LOSA_BF16 or LOSA_F32).
 * ws: at least *bytes from losa_sparse_attn_mass_workspace (the sizes of
 *    losa_dense_attn_mass's matrix-core path).
 * Arithmetic as losa_dense_attn_mass.
 * ------------------------------------------------------------------------ */
losa_status losa_sparse_attn_mass_workspace(const losa_shape* shape, size_t* bytes);
losa_status losa_sparse_attn_mass(const losa_shape* shape, const void* Q, const void* K, const void* V,
                                  const int32_t* row_ptr, const int32_t* col_idx, const int32_t* order,
                                  float* M, void* O, losa_dtype o_dtype, void* ws, size_t ws_bytes,
                                  hipStream_t stream);

/* ------------------------------------------------------------------------
 * Pooled proxy masses: the coarse block-mass estimate of per-step top-p
 * methods, which the LoSA page contrasts with exact masses (Motivation
 * Summary: the estimates SVG2 and SpargeAttn use lose accuracy just where
 * 99% recall is wanted; the pages give no formula).  Reading:
 *   P[b,h,i,j] = |B_j| exp(qbar_i . kbar_j * scale)
 *                / sum_j' |B_j'| exp(qbar_i . kbar_j' * scale),
 * qbar_i, kbar_j the means over the valid tokens of query block i and key
 * block j, |B_j| the valid keys of block j.  Rows sum to 1 like losa_block_
 * mass's M, so losa_select turns P into lists; P = M whenever the scores are
 * constant on every (query block, key block) pair.
 *
 * P: fp32 [batch, heads, n_q, n_k], contiguous (written completely).
 * ws: at least *bytes from losa_pooled_mass_workspace (the block means, fp32).
 * Arithmetic: fp32 means, dot products and softmax, for bf16 and f32 inputs
 * and every supported block shape.
 * ------------------------------------------------------------------------ */
losa_status losa_pooled_mass_workspace(const losa_shape* shape, size_t* bytes);
losa_status losa_pooled_mass(const losa_shape* shape, const void* Q, const void* K, float* P, void* ws,
                             size_t ws_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------
 * Retained mass of a pattern (for Recall, Motivation Summary).
 * kept: fp32 [2 * batch*heads*n_q]: kept[2r] = sum of M[r, j] over the
 * listed blocks of row r, kept[2r+1] = sum of M[r, j] over all j.  Recall
 * follows by weighting row r with its number of valid query rows.
 * ------------------------------------------------------------------------ */
losa_status losa_retained_mass(const losa_shape* shape, const float* M, const int32_t* row_ptr,
                               const int32_t* col_idx, float* kept, hipStream_t stream);

/* ------------------------------------------------------------------------
 * Online block thresholding.
 * Sol-Attn page: which blocks matter is decided while the online softmax
 * runs, each block's proxy score tested against a threshold, so the budget
 * varies by row; the page gives no rule.  Read here as: visiting a row's
 * key blocks in index order (the order an online pass visits them), block j
 * is kept when M[r, j] >= theta * max(M[r, 0 .. j]) -- in scores, within
 * ln(1/theta) of the running maximum.  Masses are sanitised as in
 * losa_select (NaN, inf, negatives and -0 count as 0); the comparison is
 * made in fp64, so the lists are exact.  Block 0 is always kept.
 *
 * M: fp32 [batch, heads, n_q, n_k], contiguous: exact masses
 *    (losa_block_mass) or proxies (losa_pooled_mass).
 * theta: host array of n_theta values in (0, 1]; n_theta = 1 (all heads) or
 *    heads (head h uses theta[h]; heads <= LOSA_MAX_HEADS_P).
 * row_ptr/col_idx/col_capacity/order: as losa_select (indices ascending;
 *    the same work order).
 * ws: at least *bytes from losa_select_threshold_workspace.
 * ------------------------------------------------------------------------ */
losa_status losa_select_threshold_workspace(const losa_shape* shape, size_t* bytes);
losa_status losa_select_threshold(const losa_shape* shape, const float* M, const double* theta, int32_t n_theta,
                                  int32_t* row_ptr, int32_t* col_idx, int64_t col_capacity, int32_t* order, void* ws,
                                  size_t ws_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------
 * Query-key drift since a reference step, and the heads to refresh.
 * HASTE page (temporal mask reuse): mask prediction is skipped while the
 * queries and keys have drifted little since it was last made.  The page
 * gives no measure; read here as, for head g = b*heads + h over its valid
 * tokens,
 *   drift[2g]     = ||Q_g - Q_ref_g||_F / ||Q_ref_g||_F,
 *   drift[2g + 1] = ||K_g - K_ref_g||_F / ||K_ref_g||_F
 * (0/0 = 0, x/0 = +inf for x > 0, NaN when a valid token holds NaN), and
 * refresh[g] = 1 when drift[2g] > tau or drift[2g + 1] > tau, else 0.
 * Q_ref/K_ref are the queries and keys of the step at which head g's lists
 * were built; a refreshed head takes the current ones as its new reference
 * (a device copy by the caller).
 *
 * Q, K, Q_ref, K_ref: as for losa_block_mass; Q_ref uses q_stride and K_ref
 *    k_stride.  Padding rows are not read.
 * tau: any value but NaN (LOSA_ERR_INVALID_ARG).
 * drift: fp64 [2 * batch*heads], 8-byte aligned.
 * refresh: int32 [batch*heads], or NULL (not written).
 * ws: at least *bytes from losa_qk_drift_workspace (per-workgroup partial
 *    sums, 32 bytes per 8192 elements of each tensor).
 * Arithmetic: differences, squares and sums in fp64, in a fixed order (no
 * atomics): the result is the same on every run.
 * ------------------------------------------------------------------------ */
losa_status losa_qk_drift_workspace(const losa_shape* shape, size_t* bytes);
losa_status losa_qk_drift(const losa_shape* shape, const void* Q, const void* K, const void* Q_ref,
                          const void* K_ref, double tau, double* drift, int32_t* refresh, void* ws, size_t ws_bytes,
                          hipStream_t stream);

/* ------------------------------------------------------------------------
 * Per-head merge of two list sets: the lists of the heads refreshed by a
 * drift-triggered rebuild (set b) replace theirs in the frozen set (set a);
 * the other heads keep set a's lists.  Row r of head g = r / n_q takes its
 * list from set b when take_b[g] != 0, from set a otherwise.
 *
 * take_b: int32 [batch*heads] (e.g. losa_qk_drift's refresh).
 * row_ptr_a/col_idx_a, row_ptr_b/col_idx_b: CSR lists as losa_select writes
 *    them (counts outside [0, n_k] are clamped to it); neither may overlap
 *    the outputs.
 * row_ptr/col_idx/col_capacity/order: outputs, as for losa_select; order
 *    receives the work order of the merged lists.
 * ws: at least *bytes from losa_merge_lists_workspace.
 * ------------------------------------------------------------------------ */
losa_status losa_merge_lists_workspace(const losa_shape* shape, size_t* bytes);
losa_status losa_merge_lists(const losa_shape* shape, const int32_t* take_b, const int32_t* row_ptr_a,
                             const int32_t* col_idx_a, const int32_t* row_ptr_b, const int32_t* col_idx_b,
                             int32_t* row_ptr, int32_t* col_idx, int64_t col_capacity, int32_t* order, void* ws,
                             size_t ws_bytes, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* LOSA_H */
