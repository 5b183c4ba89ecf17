/*
 * lsa.h -- C ABI of the Latent Sparse Attention (LSA) indexer for AMD MI355X
 * (gfx950).
 *
 * The indexer picks, for every query head of every query token, the cached
 * keys that sparse attention will read.  Keys are projected into a latent
 * space and clustered into a bucket hierarchy; a query scores the bucket
 * centroids level by level, descends into its best buckets, scores the member
 * keys and keeps the best k, together with the attention-sink tokens and a
 * local causal window.  (Page "Latent Sparse Attention (LSA): The 72.4x and
 * 22.7x Speedups, and What They Compare Against", section "How does LSA
 * work?", steps 1-3; page "Latent Sparse Attention: tree search over keys for
 * 10M-token context", TL;DR and flowchart.)
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Pointers named as device pointers point to GPU memory owned by the
 *    caller; the library never allocates or frees device memory and never
 *    synchronises: every call only enqueues work on `stream` (a hipStream_t
 *    passed as void*, NULL = the null stream) and returns.  Calls are
 *    therefore capturable in a HIP graph.  (lsa_pca_map is the exception: it
 *    works on host memory only, synchronously, and touches no device.)
 *  - Every argument is validated on the host before anything is enqueued.
 *    On any error nothing is enqueued, the status is returned and
 *    lsa_last_error() describes it.  No call aborts, exits or throws.
 *  - Status codes: lsa_status.  LSA_ERR_HIP reports a launch failure (read
 *    from the thread's HIP last-error state after the launches, so an error
 *    the caller's own earlier HIP calls left pending is reported here too);
 *    faults inside kernels surface at the caller's next synchronisation.
 *  - Device status of a select call (lsa_select, lsa_flat_select): the host
 *    cannot read the device-resident blob without a synchronisation, so the
 *    first kernel of the call compares the blob's header (magic, version,
 *    n_keys, n_kv_heads, d_head, d_latent, dtypes, n_levels, fanouts, build
 *    status, total bytes) with what `desc` implies, before it reads anything
 *    else of the blob.  The result, an int32 lsa_status, lands in bytes
 *    [0, 4) of the workspace: LSA_OK, or LSA_ERR_BAD_INDEX on a mismatch.  On
 *    LSA_ERR_BAD_INDEX no kernel reads past the header, every output row is
 *    all -1, scores are -inf and leaves -1.  The caller reads the word after
 *    synchronising.  The blob must hold at least its 256-byte header.
 *  - Query head hq reads KV head hq / G with G = n_q_heads / n_kv_heads.
 *  - Dtypes: keys and queries are fp32 or bf16 (the same for both); the
 *    latent store is fp32 or bf16.  All dot products accumulate in fp32.
 *
 * Limits (LSA_ERR_UNSUPPORTED otherwise): 1 <= n_keys < 2^31; n_kv_heads <=
 * 1024; d_head in {64, 128, 256}; d_latent in {32, 64}; 1 <= n_levels <= 4;
 * 2 <= fanout <= 256; at most 65535 nodes above the leaf level; product of
 * fanouts <= 2^22; per-parent beam: b <= fanout at every level and
 * b^n_levels <= 4096; global beam: b <= 64; 1 <= k <= 4096; n_q_heads <=
 * 65535; the flat scan needs n_q_heads / n_kv_heads in {1, 2, 4}.
 *
 * The k-means member sums are 64-bit fixed point: a latent value x enters as
 * round(x * 2^s) with s = 61 - c - e, where every |latent| < 2^e and
 * N <= 2^c (s clamped to [-100, 100]).  No sum can overflow whatever the
 * data's scale; each value is quantised to 2^-(61-c) of the largest magnitude
 * (2^-37 at 10M keys).  A non-finite latent value marks the index bad (header
 * word 15), and select then refuses it.
 */
#ifndef LSA_H
#define LSA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  LSA_OK = 0,
  LSA_ERR_INVALID_ARG = 1,      /* null pointer, negative size, inconsistent shapes */
  LSA_ERR_UNSUPPORTED = 2,      /* outside the limits above                          */
  LSA_ERR_BUFFER_TOO_SMALL = 3, /* index or workspace smaller than required          */
  LSA_ERR_BAD_INDEX = 4,        /* descriptor does not describe a valid index        */
  LSA_ERR_HIP = 5               /* a HIP launch failed                               */
} lsa_status;

typedef enum { LSA_F32 = 0, LSA_BF16 = 1 } lsa_dtype;

/* Beam rule of the descent.  PER_PARENT: every kept node keeps its best b
 * children (frontier b^l at level l).  GLOBAL: each level keeps the best b
 * children over the whole frontier. */
typedef enum { LSA_BEAM_PER_PARENT = 0, LSA_BEAM_GLOBAL = 1 } lsa_beam;

/* Shape of an index.  Filled by the caller; the same descriptor must be
 * passed to every call on that index (a copy is stored in the blob header). */
typedef struct {
  int64_t n_keys;       /* N: cached keys (token positions 0..N-1)               */
  int32_t n_kv_heads;   /* Hkv                                                   */
  int32_t d_head;       /* key / query width                                     */
  int32_t d_latent;     /* latent width                                          */
  int32_t key_dtype;    /* lsa_dtype of keys and queries                         */
  int32_t latent_dtype; /* lsa_dtype of latent keys and of the scoring centroids */
  int32_t n_levels;     /* L                                                     */
  int32_t fanout[4];    /* F_1..F_L (children per node at each level)            */
  int32_t kmeans_iters; /* Lloyd (assign, update) rounds per node                */
  uint64_t seed;        /* seeds the k-means initial centroids                   */
} lsa_index_desc;

typedef struct {
  int32_t b;      /* buckets kept per level (per parent, or globally)          */
  int32_t k;      /* long-range keys kept per query head                       */
  int32_t sink;   /* attention-sink positions 0..sink-1                        */
  int32_t window; /* local window: the last `window` positions up to p         */
  int32_t beam;   /* lsa_beam                                                  */
} lsa_select_params;

/* ------------------------------------------------------------------------
 * The index blob: one caller-owned device buffer of lsa_index_bytes(desc)
 * bytes, little-endian, every section aligned to 256 bytes.
 *
 *   header (256 bytes)
 *     0  char[4]   "LSA1"            4  uint32  version = 1
 *     8  int64     n_keys
 *    16  int32     n_kv_heads, d_head, d_latent, key_dtype, latent_dtype,
 *                  n_levels, fanout[4], kmeans_iters, build status (0 = good,
 *                  1 = a latent value was not finite)
 *    64  uint64    seed              72  uint64  total bytes
 *    80  uint64    offset of W       88  uint64  offset of perm
 *    96  uint64    offset of latent
 *   104  uint64[4] offsets of centroids[l]   (0 for absent levels)
 *   136  uint64[4] offsets of cscore[l]
 *   168  uint64[4] offsets of offsets[l]
 *   sections, in this order:
 *     W            fp32   [Hkv][d_head][d_latent]        the latent map
 *     centroids[l] fp32   [Hkv][P_l][d_latent]            P_l = F_1*...*F_l
 *     cscore[l]    latent [Hkv][P_l][d_latent]            scoring copy (RNE)
 *     offsets[l]   int32  [Hkv][P_l + 1]                  CSR row ranges
 *     perm         int32  [Hkv][N]                        key index of CSR row
 *     latent       latent [Hkv][N][d_latent]              row r = key perm[r]
 *
 * Node ids: child c of node p at level l has id p*F_l + c (the root is node
 * 0 of level 0).  Rows [offsets[l][n], offsets[l][n+1]) of a head hold the
 * keys of node n of level l, in ascending key index within each leaf; the
 * ranges of a node's children tile the node's range.  A node with no member
 * is empty: it is never selected.  A child that received no initial centroid
 * (its parent had fewer members than the fanout) has zero centroids.
 * ------------------------------------------------------------------------ */

/* Bytes of the index blob for `desc`; 0 if the descriptor is invalid (then
 * lsa_last_error() says why). */
size_t lsa_index_bytes(const lsa_index_desc* desc);

/* Bytes of device workspace lsa_build_index needs; 0 if invalid. */
size_t lsa_build_workspace_bytes(const lsa_index_desc* desc);

/* Build the index (step 1 of "How does LSA work?": keys are clustered into a
 * hierarchy of buckets in a latent space).
 *   keys      device [N][Hkv][d_head], key_dtype (the KV cache's key layout)
 *   W         device [Hkv][d_head][d_latent] fp32, latent map (copied into
 *             the blob; queries use the same map)
 *   index     device, index_bytes >= lsa_index_bytes(desc); fully written
 *   workspace device, workspace_bytes >= lsa_build_workspace_bytes(desc);
 *             scratch, contents undefined afterwards
 * Latent keys are round(K.W) (fp32 accumulation, one RNE rounding to the
 * latent dtype).  Level l splits every node of level l-1 into F_l children by
 * Lloyd k-means on the node's own members: seeded initial centroids (distinct
 * members drawn with splitmix64), kmeans_iters rounds of (assign to the
 * nearest centroid, ties to the lowest child; move every non-empty centroid
 * to its members' mean), then a final assignment against the stored
 * centroids.  Deterministic: the same inputs give the same bytes. */
int lsa_build_index(const lsa_index_desc* desc, const void* keys, const float* W, void* index,
                    size_t index_bytes, void* workspace, size_t workspace_bytes, void* stream);

/* Width of one output row: sink + k + window. */
int32_t lsa_select_out_width(const lsa_select_params* params);

/* Bytes of device workspace lsa_select needs for this shape; 0 if invalid. */
size_t lsa_select_workspace_bytes(const lsa_index_desc* desc, const lsa_select_params* params,
                                  int32_t n_tokens, int32_t n_q_heads);

/* Tree selection (steps 2 and 3 of "How does LSA work?").
 *   index      device blob written by lsa_build_index (or to the same layout)
 *   queries    device [T][Hq][d_head], key_dtype
 *   q_pos      device int32 [T], position p of each query token, 0 <= p < N
 *              (a row whose position is out of range is written as all -1)
 *   out_idx    device int32 [T][Hq][sink + k + window]:
 *                [0, sink)          positions 0..min(sink, p+1)-1, then -1
 *                [sink, sink+k)     selected long-range keys, ascending, -1 padded
 *                [sink+k, width)    positions max(sink, p-window+1)..p, then -1
 *   out_scores device fp32 [T][Hq][k] or NULL: score of each selected key,
 *              aligned with its slot, -inf padded
 *   out_leaves device int32 [T][Hq][b^L] (b for GLOBAL) or NULL: the leaf
 *              buckets the query descended into, -1 padded
 * The query's latent is round(q.W_h).  Level by level the children of every
 * kept node are scored by the inner product with their scoring centroid
 * (empty children never kept) and the best b are kept (ties: lower id).  The
 * members of the kept leaves whose index lies in [sink, p - window] are
 * scored by the inner product of latents, and the best k (ties: lower index)
 * are returned; fewer candidates than k return all of them. */
int lsa_select(const lsa_index_desc* desc, const void* index, const void* queries, const int32_t* q_pos,
               int32_t n_tokens, int32_t n_q_heads, const lsa_select_params* params, int32_t* out_idx,
               float* out_scores, int32_t* out_leaves, void* workspace, size_t workspace_bytes,
               void* stream);

/* lsa_select without a workspace argument, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc).  The workspace is a fixed scratch buffer of
 * LSA_NOALLOC_SCRATCH_BYTES inside the library: one copy per GPU, set up on
 * the first call on that device and held until the process ends.  The call
 * allocates nothing.  Same arguments (minus the workspace), kernels and
 * results as lsa_select.
 * Errors: those of lsa_select; LSA_ERR_UNSUPPORTED when the batch needs more
 * workspace than the scratch holds (lsa_select_workspace_bytes tells; decode
 * batches of the 1M and 10M configurations need about 13 MiB); LSA_ERR_HIP if
 * the scratch cannot be located.  Every call on a GPU uses that GPU's one
 * scratch: calls that overlap on one GPU (concurrent streams, or threads)
 * race and must be serialised by the caller.  The scratch keeps the last
 * call's contents; the kernels clear what they need.  The device status word
 * of a call sits in the scratch, so a mismatched index shows only as all -1
 * rows here. */
#define LSA_NOALLOC_SCRATCH_BYTES (32u << 20)
int lsa_select_noalloc(const lsa_index_desc* desc, const void* index, const void* queries, const int32_t* q_pos,
                       int32_t n_tokens, int32_t n_q_heads, const lsa_select_params* params, int32_t* out_idx,
                       float* out_scores, int32_t* out_leaves, void* stream);

/* How lsa_select computes a batch of this shape (same result either way):
 *   LSA_PATH_PER_QUERY_HEAD  every query head descends and gathers on its own
 *                            (decode and small batches)
 *   LSA_PATH_NODE_MAJOR      every tree node is visited once with all the
 *                            query heads that kept its parent, centroids and
 *                            keys scored on bf16 matrix tiles (large batches:
 *                            at least 256 query heads per KV head, bf16
 *                            latent, per-parent beam, fanouts <= 64,
 *                            b <= 16, k <= 2048)
 * Returns -1 (and sets lsa_last_error) for invalid arguments. */
typedef enum {
  LSA_PATH_PER_QUERY_HEAD = 0,
  LSA_PATH_NODE_MAJOR = 1,
  LSA_PATH_ROW_TILED = 2
} lsa_select_path_kind;
int32_t lsa_select_path(const lsa_index_desc* desc, const lsa_select_params* params, int32_t n_tokens,
                        int32_t n_q_heads);

/* Which kernels lsa_flat_select runs for this shape (same results either way):
 *   LSA_PATH_PER_QUERY_HEAD  a streaming scan per (token, KV head) that reads
 *                            every key once for the head's G query heads
 *   LSA_PATH_ROW_TILED       a scan on the matrix cores: 256 query heads of a
 *                            KV head per workgroup against every key, with a
 *                            sampled per-query-head threshold (at least 256
 *                            query heads per KV head, bf16 latent, k <= 2048)
 * Returns -1 (and sets lsa_last_error) for invalid arguments. */
int32_t lsa_flat_select_path(const lsa_index_desc* desc, const lsa_select_params* params, int32_t n_tokens,
                             int32_t n_q_heads);

/* Bytes of device workspace lsa_flat_select needs; 0 if invalid. */
size_t lsa_flat_workspace_bytes(const lsa_index_desc* desc, const lsa_select_params* params,
                                int32_t n_tokens, int32_t n_q_heads);

/* Full-scan baseline: the indexer that scores every key (the dashed, quadratic
 * path of the flowchart on "Latent Sparse Attention: tree search over keys for
 * 10M-token context").  Same arguments and output rows as lsa_select, with
 * every key in [sink, p - window] a candidate; params->b and ->beam are
 * ignored.  Equal to lsa_select with b = fanout at every level. */
int lsa_flat_select(const lsa_index_desc* desc, const void* index, const void* queries,
                    const int32_t* q_pos, int32_t n_tokens, int32_t n_q_heads,
                    const lsa_select_params* params, int32_t* out_idx, float* out_scores,
                    void* workspace, size_t workspace_bytes, void* stream);

/* ---- incremental upkeep: keys that arrive after the build --------------------------
 * Every decode step adds a key to the cache, and the cache stays full length
 * (page "Latent Sparse Attention: tree search over keys for 10M-token
 * context", section "Gaps"); decode runs in a captured loop ("Latent Sparse
 * Attention (LSA): The 72.4x and 22.7x Speedups, and What They Compare
 * Against", section "Can I run LSA?").  The pages do not say how new keys
 * enter the index.  Reading: a new key joins the tree without changing it.
 * Its latent is computed as the build computes every key's; it descends from
 * the root, at every level to the child of the current node whose stored
 * centroid is nearest (the build's assignment arithmetic) among the children
 * that hold keys, ties to the lowest child, and joins the leaf it reaches.
 * Centroids and earlier keys do not move; re-clustering is a new build.  The
 * i-th appended key of every KV head is the key at position n_keys + i.
 *
 * The append pool: one caller-owned device buffer of
 * lsa_append_pool_bytes(desc, capacity) bytes, sections 256-byte aligned:
 *     leaf    int32  [Hkv][capacity]              leaf each appended key joined
 *                                                 (-1: the index was refused)
 *     latent  latent [Hkv][capacity][d_latent]    its latent
 * Slot i of a head holds the key at position n_keys + i.  The caller keeps
 * count of the slots in use (every call appends the same tokens to every
 * KV head).  Limits: capacity >= 1, n_keys + capacity < 2^31. */

/* Bytes of an append pool of `capacity` keys per KV head; 0 if invalid. */
size_t lsa_append_pool_bytes(const lsa_index_desc* desc, int32_t capacity);

/* Append n_new keys (device [n_new][Hkv][d_head], key_dtype: the new tokens'
 * keys) to slots [first, first + n_new) of `pool` (device, capacity keys per
 * head), for every KV head.  Reads the index (device blob); a blob whose
 * header does not match desc leaves the slots' leaves at -1.  Asynchronous on
 * `stream`; allocates nothing.  Errors: LSA_ERR_INVALID_ARG (NULL pointer,
 * slots outside [0, capacity)), LSA_ERR_UNSUPPORTED (descriptor, capacity),
 * LSA_ERR_HIP; nothing is enqueued on a validation error. */
int lsa_append_keys(const lsa_index_desc* desc, const void* index, const void* keys, int32_t n_new, int32_t first,
                    void* pool, int32_t capacity, void* stream);

/* Bytes of device workspace lsa_select_appended needs; 0 if invalid. */
size_t lsa_select_appended_workspace_bytes(const lsa_index_desc* desc, const lsa_select_params* params,
                                           int32_t n_tokens, int32_t n_q_heads);

/* lsa_select over the index plus the first n_appended keys of the pool
 * (positions n_keys .. n_keys + n_appended - 1): an appended key is a
 * candidate of a query head iff its leaf is one the head kept and its
 * position lies in [sink, p - window].  Query positions may be up to
 * n_keys + n_appended - 1.  Same outputs, device status word and errors as
 * lsa_select; n_appended outside [0, capacity] is LSA_ERR_INVALID_ARG.  Every
 * batch runs the per-query-head kernels, which read each leaf once per query
 * head: meant for decode between re-builds. */
int lsa_select_appended(const lsa_index_desc* desc, const void* index, const void* pool, int32_t capacity,
                        int32_t n_appended, const void* queries, const int32_t* q_pos, int32_t n_tokens,
                        int32_t n_q_heads, const lsa_select_params* params, int32_t* out_idx, float* out_scores,
                        int32_t* out_leaves, void* workspace, size_t workspace_bytes, void* stream);

/* ---- training-free latent map ------------------------------------------------
 * "Latent Sparse Attention (LSA): The 72.4x and 22.7x Speedups, and What They
 * Compare Against", section "How does LSA work?", lists a PCA map as the option
 * that needs no training.  Reading: for every KV head h, the d_latent leading
 * eigenvectors of the covariance of the keys of h (mean-centred, divided by N)
 * are the columns of W_h, in descending order of eigenvalue, each signed so
 * that its entry of largest magnitude (the lowest row on a tie) is positive.
 * The result is the W that lsa_build_index takes.  Two calls: the covariance on
 * the device, then the eigenvectors on the host (the caller copies the
 * covariance to host memory in between). */

/* Bytes of device workspace lsa_pca_covariance needs; 0 if the descriptor is
 * invalid.  Only n_keys, n_kv_heads, d_head and key_dtype matter. */
size_t lsa_pca_workspace_bytes(const lsa_index_desc* desc);

/* Per KV head the key covariance, into cov: DEVICE float64 [Hkv][d_head][d_head],
 * row-major, caller-owned.  keys: DEVICE [N][Hkv][d_head] of desc->key_dtype.
 * Sums of products are fp32 over chunks of at most max(4096, N / 256) keys of
 * one head (each key shifted by the head's first key), chunks are added in
 * fp64.  Asynchronous on `stream`; the workspace is scratch for the call.
 * Errors: LSA_ERR_INVALID_ARG (NULL pointer), LSA_ERR_UNSUPPORTED (descriptor),
 * LSA_ERR_BUFFER_TOO_SMALL, LSA_ERR_HIP (launch); nothing is enqueued on a
 * validation error. */
int lsa_pca_covariance(const lsa_index_desc* desc, const void* keys, double* cov, void* workspace,
                       size_t workspace_bytes, void* stream);

/* The latent map from a covariance, on the host: cov HOST float64
 * [Hkv][d_head][d_head] (as lsa_pca_covariance writes it; it is symmetrised
 * first), W HOST fp32 [Hkv][d_head][d_latent] (out), eigenvalues HOST float64
 * [Hkv][d_latent] (out, descending; NULL to skip).  Eigenvectors come from
 * cyclic Jacobi rotations in float64.  Synchronous; touches no device.
 * Errors: LSA_ERR_INVALID_ARG (NULL cov or W), LSA_ERR_UNSUPPORTED
 * (descriptor). */
int lsa_pca_map(const lsa_index_desc* desc, const double* cov, float* W, double* eigenvalues);

/* ---- exact sparse attention over the selected keys ------------------------------
 * "Latent Sparse Attention (LSA): The 72.4x and 22.7x Speedups, and What They
 * Compare Against", section "How does LSA work?", step 3: a query reads the
 * far keys the indexer chose, the sink positions and its recent window, and
 * the attention computation is the ordinary one.  For every (token t, query head hq):
 *   out[t][hq] = sum_j softmax_j(scale * q . k_j) v_j
 * over the entries j of row idx[t][hq] (an lsa_select output row, or any list);
 * an entry outside [0, N) is padding, an entry listed twice counts twice, and a
 * row with no key gives zeros.  Query head hq reads KV head hq / G.
 *   queries  DEVICE [T][Hq][d_head], desc->key_dtype
 *   keys     DEVICE [N][Hkv][d_head], desc->key_dtype (the KV cache's keys)
 *   values   DEVICE [N][Hkv][d_head], desc->key_dtype (the KV cache's values)
 *   idx      DEVICE int32 [T][Hq][width], 1 <= width <= 32768
 *   out      DEVICE fp32 [T][Hq][d_head]
 *   workspace DEVICE, lsa_sparse_attention_workspace_bytes bytes (0 for many
 *            rows; few rows split each row over several workgroups, whose
 *            partial results go here); scratch for the call
 * Only n_keys, n_kv_heads, d_head and key_dtype of desc are used.  Scores,
 * softmax and the weighted sum are fp32.  Asynchronous on `stream`.
 * Errors: LSA_ERR_INVALID_ARG (NULL pointer, shape, scale not finite),
 * LSA_ERR_UNSUPPORTED (descriptor, width), LSA_ERR_BUFFER_TOO_SMALL,
 * LSA_ERR_HIP (launch); nothing is enqueued on a validation error. */
size_t lsa_sparse_attention_workspace_bytes(const lsa_index_desc* desc, int32_t width, int32_t n_tokens,
                                            int32_t n_q_heads);
int lsa_sparse_attention(const lsa_index_desc* desc, const void* queries, const void* keys, const void* values,
                         const int32_t* idx, int32_t width, int32_t n_tokens, int32_t n_q_heads, float scale,
                         float* out, void* workspace, size_t workspace_bytes, void* stream);

/* Stages of a select call that can be timed by the caller. */
typedef enum {
  LSA_STAGE_PROJECT = 1, /* query latent projection                         */
  LSA_STAGE_DESCEND = 2, /* centroid scoring and descent                    */
  LSA_STAGE_GATHER = 3,  /* gather-and-score with top-k (lsa_select)       */
  LSA_STAGE_MERGE = 4,   /* merge of split top-k lists                      */
  LSA_STAGE_FLAT = 5,    /* full scan with top-k (lsa_flat_select)         */
  LSA_STAGE_SAMPLE = 6   /* node-major path: sampled scores and per-query
                            thresholds (between DESCEND and GATHER)        */
} lsa_stage;

/* Instrumentation: until reset, every lsa_select / lsa_flat_select call on
 * this thread records `start` (a hipEvent_t) on its stream before the first
 * kernel of `stage` and `stop` after the last one.  NULL events switch the
 * stage off.  Nothing is allocated and nothing synchronises; the caller owns
 * the events. */
int lsa_set_profile_events(int32_t stage, void* start, void* stop);

/* Message of the last failed call on this thread ("" if none).  Valid until
 * the next lsa_* call on the same thread. */
const char* lsa_last_error(void);

/* ABI version (1). */
int32_t lsa_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* LSA_H */
