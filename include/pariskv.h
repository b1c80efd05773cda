/*
 * pariskv.h -- C ABI of the MI355X (gfx950) ParisKV decode-step retrieval
 * library: KV-cache index build and incremental append, two-stage top-k
 * retrieval (collision votes -> candidates -> RSQ-IP rerank -> exact top-k)
 * and split-K sparse attention over the selected full-precision rows.
 *
 * Method source: "Technical Summary: ParisKV" (gist.science/paper/2602.07721),
 * cited below as [TS] with its section names, and "ParisKV: Fast and
 * Drift-Robust KV-Cache Retrieval for Long-Context LLMs" (ICML 2026 poster
 * abstract).  Each entry point cites the passage that defines its operation.
 *
 * Conventions (all entry points):
 *   - Status codes: PARISKV_OK (0) or a negative PARISKV_ERR_*.  No C++
 *     exception crosses this boundary.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *     Work is enqueued asynchronously; nothing synchronises the device except
 *     the pariskv_debug_* calls, which are documented as synchronous.
 *   - The library allocates NO device memory.  The caller owns every device
 *     buffer (index, workspace, inputs, outputs); the only library-owned
 *     object is the small host-side index handle.
 *   - Device pointers must be device-accessible (HBM, or mapped pinned host
 *     memory where stated).  Inputs must be finite; NaN/Inf behaviour is
 *     undefined (no checking pass: it would cost a full read of the cache).
 *   - Argument errors are detected on the host, synchronously, before any
 *     launch.  Asynchronous device faults surface as PARISKV_ERR_HIP on a
 *     later call or at the caller's stream synchronisation.
 *   - One index handle must not be used from two streams at once; distinct
 *     handles are independent.
 */
#ifndef PARISKV_H
#define PARISKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PARISKV_API __attribute__((visibility("default")))

/* status codes */
#define PARISKV_OK               0
#define PARISKV_ERR_INVALID_ARG (-1)   /* bad pointer, size, shape or k      */
#define PARISKV_ERR_UNSUPPORTED (-2)   /* valid for the method, not built    */
#define PARISKV_ERR_CAPACITY    (-3)   /* append/build beyond capacity       */
#define PARISKV_ERR_WORKSPACE   (-4)   /* workspace or index buffer too small */
#define PARISKV_ERR_HIP         (-5)   /* a HIP runtime call failed          */
#define PARISKV_ERR_NOMEM       (-6)   /* host allocation of the handle failed */

/* element types of K, V, Q and the attention output */
#define PARISKV_DTYPE_BF16 0
#define PARISKV_DTYPE_FP32 1

/*
 * Method parameters and shapes.  Validated by every call that takes it.
 *   head_dim     d, a power of two (this build: 128).
 *   n_subspaces  B; m = d / B contiguous coordinates per subspace, each
 *                with 2^m sign-pattern centroids ([TS] Coarse Candidate
 *                Generation; this build: m = 8, B = 16, or m = 4, B = 32).
 *   rho          centroids the query keeps per subspace, 1..8.
 *   tier_w[s]    vote weight of the query's (s+1)-th ranked centroid,
 *                0..255, with B * max(tier_w) <= 255 (the tiered votes of
 *                [TS] Coarse Candidate Generation).
 *   cand_num/den candidate fraction f = num/den, 0 < num <= den (the pages
 *                keep the top 5 to 10 per cent).
 *                C = min(E, max(k', ceil(E f))), E = N - S, k' = k - S.
 *   n_sink       S: keys [0, S) are always selected and are not scored.
 *   batch, n_kv_heads, n_q_heads   n_q_heads % n_kv_heads == 0; the
 *                G = n_q_heads / n_kv_heads query heads of a KV head share
 *                one retrieval whose query is their mean (this build:
 *                G in {1, 2, 4, 8}).  batch * n_kv_heads <= 65535.
 *   key_dtype    PARISKV_DTYPE_BF16 or _FP32, the dtype of K and Q.
 *   capacity     maximum keys per (batch, KV head) the index can hold.
 *   per_query_head  0: one retrieval per (batch, KV head) with the group's
 *                mean query (the default).  1: unshared retrieval, one per
 *                (batch, query head) with that head's own query, over its KV
 *                head's index; out_idx / out_est then hold n_q_heads rows per
 *                batch entry.  batch * n_q_heads <= 65535.
 */
typedef struct pariskv_config {
    int32_t head_dim;
    int32_t n_subspaces;
    int32_t rho;
    int32_t tier_w[8];
    int32_t cand_num;
    int32_t cand_den;
    int32_t n_sink;
    int32_t batch;
    int32_t n_kv_heads;
    int32_t n_q_heads;
    int32_t key_dtype;
    int64_t capacity;
    int32_t per_query_head;
} pariskv_config;

typedef struct pariskv_index pariskv_index;   /* opaque host-side handle */
typedef struct pariskv_window pariskv_window; /* opaque host-side handle */

/* Number of stages that pariskv_retrieve_topk_profiled brackets. */
#define PARISKV_RETRIEVE_STAGES 6

/* ---------------------------------------------------------------------- */
/* Sizing.                                                                 */
/* ---------------------------------------------------------------------- */

/* Bytes of the device index buffer for `cfg`: per key and (b, h), 16 B of
 * bucket ids (byte s = the sign bits of coordinates 8 s .. 8 s + 7: one id
 * for m = 8, two 4-bit ids for m = 4) and a 128-byte record holding the
 * 64 B of RSQ-IP codes and the B fp16 calibration factors (32 B for m = 8,
 * 64 B for m = 4; one aligned line per key, so a rerank gather touches one
 * line), for `capacity` keys.
 * Errors: INVALID_ARG / UNSUPPORTED for a bad config. */
PARISKV_API int32_t pariskv_index_bytes(const pariskv_config *cfg,
                                        size_t *bytes);

/* Bytes of the device workspace pariskv_retrieve_topk needs for any index
 * size up to cfg->capacity and this k. */
PARISKV_API int32_t pariskv_retrieve_workspace_bytes(const pariskv_config *cfg,
                                                     int32_t k, size_t *bytes);

/* Bytes of the device workspace pariskv_sparse_attn needs. */
PARISKV_API int32_t pariskv_attn_workspace_bytes(int32_t batch,
                                                 int32_t n_q_heads, int32_t k,
                                                 int32_t head_dim,
                                                 size_t *bytes);

/* ---------------------------------------------------------------------- */
/* Index build and append.                                                 */
/* [TS] Core Algorithmic Innovations 1 (normalisation + shared SRHT        */
/* rotation; analytic sign-pattern centroids, data independent, so decode  */
/* keys join the index without re-clustering) and 2 (bucket id per         */
/* subspace; 4-bit RSQ-IP code per coordinate; calibration w_{i,b}         */
/* computed when the key is encoded).                                      */
/* ---------------------------------------------------------------------- */

/* Creates a handle over the caller's `index_buf` (device, >= index_bytes,
 * 256-byte aligned, must outlive the handle) and encodes keys [0, n_keys)
 * of every (b, h), asynchronously on `stream`.
 *   srht_signs   host array of head_dim int8 values, each +1 or -1: the
 *                random diagonal D of the rotation c * H * diag(D).  Copied.
 *   K            device-accessible (HBM, or mapped pinned host memory read
 *                over the host link), key_dtype, element (b, h, i, j) at
 *                K[((b * n_kv_heads + h) * k_rows_per_head + i) * d + j].
 *   k_rows_per_head   row stride between consecutive (b, h), >= n_keys.
 * Errors: INVALID_ARG (null pointer, signs not +-1, stride < n_keys),
 * UNSUPPORTED, WORKSPACE (index_bytes too small), CAPACITY (n_keys >
 * capacity), NOMEM, HIP.  On error *out is NULL. */
PARISKV_API int32_t pariskv_build_index(const pariskv_config *cfg,
                                        const int8_t *srht_signs,
                                        void *index_buf, size_t index_bytes,
                                        const void *K, int64_t k_rows_per_head,
                                        int64_t n_keys, void *stream,
                                        pariskv_index **out);

/* Encodes n_new keys per (b, h) and appends them at positions [N, N+n_new)
 * where N is the current size; the host-side size is updated at once, so
 * later calls know N without a device synchronisation.
 *   K_new        device-accessible (HBM or mapped pinned host memory),
 *                element (b, h, r, j) at
 *                K_new[((b * n_kv_heads + h) * new_rows_per_head + r) * d + j]
 *                for r < n_new (a pointer into the KV cache at row N with
 *                new_rows_per_head = the cache's rows per head works).
 * A decode step's few keys (n_new <= 48) are encoded lazily: by the first
 * kernel of the next pariskv_retrieve_topk, on that call's stream (which the
 * caller orders after the writes of K_new, as any retrieval that must see the
 * new keys requires, whether or not it is the append's stream), or, if
 * something else comes first (another append, pariskv_debug_export,
 * pariskv_index_destroy), by a kernel launched then on this call's stream.
 * K_new must stay valid and unmodified until then.
 * Larger appends are encoded at once on `stream`.
 * Errors: INVALID_ARG, CAPACITY (N + n_new > capacity), HIP. */
PARISKV_API int32_t pariskv_append_keys(pariskv_index *index,
                                        const void *K_new,
                                        int64_t new_rows_per_head,
                                        int64_t n_new, void *stream);

/* Current number of keys per (b, h), or -1 for a NULL handle. */
PARISKV_API int64_t pariskv_index_size(const pariskv_index *index);

/* Encodes any deferred appended keys (on the stream they were appended on),
 * then frees the host handle (never the caller's index buffer). */
PARISKV_API void pariskv_index_destroy(pariskv_index *index);

/* ---------------------------------------------------------------------- */
/* Retrieval.                                                              */
/* [TS] Core Algorithmic Innovations 2, "Two-Stage GPU-Native Retrieval    */
/* Pipeline": per subspace the query's top-rho centroids cast tiered votes */
/* summed into an integer coarse score; the top fraction of keys is kept   */
/* and reranked with the RSQ-IP estimator                                  */
/* ||q|| sum_b w_{i,b} <v_{i,b}, q~_b>; the exact top-k of the estimates is */
/* returned.  Key Contributions 2: the whole selection runs on the GPU.    */
/* ---------------------------------------------------------------------- */

/* For every (b, h): out_idx[(b * n_kv_heads + h) * k + t], t < k, receives
 * the selected key positions in ascending order: the S sinks 0..S-1 followed
 * by the k - S reranked winners (ties broken towards the lower position).
 *   Q        device, key_dtype, [batch][n_q_heads][d] contiguous.
 *   out_est  optional (NULL to skip): device float [b][h][k - S], the RSQ-IP
 *            estimate of each non-sink selected key, aligned with
 *            out_idx[S..k).
 *   ws       device workspace of >= pariskv_retrieve_workspace_bytes(k),
 *            256-byte aligned; its contents need not be initialised.
 * No host synchronisation and no allocation: capturable in a HIP graph.
 * Errors: INVALID_ARG (k <= S or k > N, null pointers), WORKSPACE,
 * UNSUPPORTED (more than 4,194,304 candidates per (b, h)), HIP. */
PARISKV_API int32_t pariskv_retrieve_topk(const pariskv_index *index,
                                          const void *Q, int32_t k,
                                          int32_t *out_idx, float *out_est,
                                          void *ws, size_t ws_bytes,
                                          void *stream);

/* Bytes of the library's own device scratch per GPU, used by
 * pariskv_retrieve_topk_noalloc. */
#define PARISKV_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)

/* For callers that cannot allocate device memory or pass a workspace (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation): pariskv_retrieve_topk with the workspace taken from a
 * library-owned device array of PARISKV_NOALLOC_SCRATCH_BYTES on the device
 * current on the calling thread (the index's device).  The array is loaded
 * with the library and held by each GPU it runs on until the process ends;
 * its address is resolved on the first call on a device.  No hipMalloc,
 * hipFree or other allocating call is made.  Every call on one GPU shares
 * that GPU's array and leaves its contents behind (the retrieval needs none
 * of it initialised), so calls that overlap on one GPU -- on different
 * streams, or from different threads without ordering -- race and must not
 * be issued.  Same arguments, outputs and errors as pariskv_retrieve_topk,
 * plus WORKSPACE when pariskv_retrieve_workspace_bytes(k) for this index
 * exceeds PARISKV_NOALLOC_SCRATCH_BYTES (the 1M-key x 8-head layer at
 * k = 4096 needs about 25 MiB). */
PARISKV_API int32_t pariskv_retrieve_topk_noalloc(const pariskv_index *index,
                                                  const void *Q, int32_t k,
                                                  int32_t *out_idx,
                                                  float *out_est,
                                                  void *stream);

/* Same as pariskv_retrieve_topk, and times each stage's kernel: events
 * holds 2 * PARISKV_RETRIEVE_STAGES caller-created hipEvent_t (timing
 * enabled); events[2s] and events[2s+1] are stamped by the dispatch of stage
 * s itself when that kernel starts and ends (hipExtLaunchKernel), so the
 * pair brackets exactly that kernel.  Stages: query prep, vote scan,
 * threshold, compact + rerank, top-k, top-k second pass.  Top-k is one
 * kernel for up to 16384 candidates per retrieval unit; above that it is
 * a histogram kernel (stage 4) and a select kernel (stage 5).  A stage that
 * a call does not run has its two events recorded back to back.
 * Not for use under stream capture. */
PARISKV_API int32_t pariskv_retrieve_topk_profiled(
    const pariskv_index *index, const void *Q, int32_t k, int32_t *out_idx,
    float *out_est, void *ws, size_t ws_bytes, void *stream, void **events);

/* ---------------------------------------------------------------------- */
/* Retrieval and sparse attention in one call.                             */
/* [TS] Core Algorithmic Innovations 2 (the two-stage retrieval) followed  */
/* by System-Level Innovations 1: only the selected Top-k rows of K and V  */
/* are fetched and attended.  The retrieval kernels, then the split-K      */
/* attention and its merge, queued by one call on one stream.  The results */
/* are those of pariskv_retrieve_topk followed by pariskv_sparse_attn (or  */
/* its per-query-head form) with the same arguments: identical out_idx,    */
/* out_est and attention output.                                           */
/* ---------------------------------------------------------------------- */

/* Bytes of the workspace pariskv_retrieve_attend needs for k. */
PARISKV_API int32_t pariskv_retrieve_attend_workspace_bytes(const pariskv_config *cfg,
                                                            int32_t k, size_t *bytes);

/* Retrieval as pariskv_retrieve_topk (out_idx, optional out_est), then the
 * attention of every query head over its selected rows into `out`.
 *   K, V             device-accessible, key_dtype, [b][H_kv][kv_rows_per_head][d]
 *                    (kv_rows_per_head >= the index size).
 *   scale            softmax scale (normally 1/sqrt(d)), finite.
 *   out              device, key_dtype, [b][H_q][d].
 *   ws               >= pariskv_retrieve_attend_workspace_bytes(k), 256-byte
 *                    aligned; contents need not be initialised.
 * No host synchronisation and no allocation: capturable in a HIP graph.
 * Errors: as pariskv_retrieve_topk, plus INVALID_ARG for null K, V or out, a
 * non-finite scale or kv_rows_per_head below the index size. */
PARISKV_API int32_t pariskv_retrieve_attend(const pariskv_index *index, const void *Q,
                                            const void *K, const void *V,
                                            int64_t kv_rows_per_head, int32_t k,
                                            float scale, int32_t *out_idx,
                                            float *out_est, void *out, void *ws,
                                            size_t ws_bytes, void *stream);

/* Same, timing its kernels: events holds 2 * PARISKV_RETRIEVE_STAGES + 4
 * caller-created events, the retrieval stages as for
 * pariskv_retrieve_topk_profiled, then the attention split and merge.
 * Not for use under stream capture. */
PARISKV_API int32_t pariskv_retrieve_attend_profiled(
    const pariskv_index *index, const void *Q, const void *K, const void *V,
    int64_t kv_rows_per_head, int32_t k, float scale, int32_t *out_idx, float *out_est,
    void *out, void *ws, size_t ws_bytes, void *stream, void **events);

/* Name of retrieval stage s, or NULL. */
PARISKV_API const char *pariskv_stage_name(int32_t stage);

/* How pariskv_retrieve_topk runs on an index: an execution choice for the
 * same [TS] Core Algorithmic Innovations 2 pipeline, not a different method.
 *   PARISKV_PATH_AUTO (the default): the multi-kernel pipeline.
 *   PARISKV_PATH_PIPELINE: the multi-kernel pipeline.
 *   PARISKV_PATH_SINGLE: one kernel, one 1024-thread block per unit running
 *     every stage with block barriers instead of kernel boundaries; it
 *     serves units of one (b, KV head) (shared retrieval) with at most 16,384
 *     candidates, and returns UNSUPPORTED otherwise.  Units of at most 8192
 *     keys and 2048 candidates keep ids, scores and candidates in registers
 *     and LDS.  Measured about 3% faster than the pipeline on a 4K-key unit
 *     and slower on larger ones (one CU per unit), so AUTO does not pick it.
 * The two paths return the same bits and leave the same intermediates in
 * the workspace.  Errors: INVALID_ARG. */
#define PARISKV_PATH_AUTO 0
#define PARISKV_PATH_PIPELINE 1
#define PARISKV_PATH_SINGLE 2
PARISKV_API int32_t pariskv_set_retrieval_path(pariskv_index *index,
                                               int32_t path);

/* The path (PARISKV_PATH_PIPELINE or PARISKV_PATH_SINGLE) a retrieval of
 * k keys would take on the index now, or a negative status
 * (INVALID_ARG, UNSUPPORTED).  With PARISKV_PATH_SINGLE the profiled call
 * stamps the single kernel as stage 1 (vote scan) and records every other
 * stage's events back to back. */
PARISKV_API int32_t pariskv_retrieval_path(const pariskv_index *index,
                                           int32_t k);

/* ---------------------------------------------------------------------- */
/* Sparse attention.                                                       */
/* [TS] Problem Statement (attend to a Top-k subset of past tokens) and    */
/* System-Level Innovations 1 (only the selected Top-k K/V pairs are       */
/* fetched).  out = softmax(scale * q K_idx^T) V_idx per query head, over   */
/* the k rows idx of its KV head; fp32 accumulation, output in `dtype`.    */
/* ---------------------------------------------------------------------- */

/*   Q    device, dtype, [batch][n_q_heads][d].
 *   K, V device-accessible (HBM or mapped pinned host memory), dtype,
 *        element (b, h, i, j) at [((b * n_kv_heads + h) * kv_rows_per_head
 *        + i) * d + j].
 *   idx  device int32 [batch][n_kv_heads][k]; every entry in
 *        [0, kv_rows_per_head) (not checked on the device).
 *   out  device, dtype, [batch][n_q_heads][d].
 *   ws   device, >= pariskv_attn_workspace_bytes.
 * Errors: INVALID_ARG, UNSUPPORTED (head_dim != 128), WORKSPACE, HIP. */
PARISKV_API int32_t pariskv_sparse_attn(const void *Q, const void *K,
                                        const void *V,
                                        int64_t kv_rows_per_head,
                                        const int32_t *idx, int32_t k,
                                        int32_t batch, int32_t n_q_heads,
                                        int32_t n_kv_heads, int32_t head_dim,
                                        int32_t dtype, float scale, void *out,
                                        void *ws, size_t ws_bytes,
                                        void *stream);

/* Same, with events[0..1] stamped around the split-K kernel and
 * events[2..3] around the merge kernel by their own dispatches
 * (caller-created hipEvent_t, timing enabled). */
PARISKV_API int32_t pariskv_sparse_attn_profiled(
    const void *Q, const void *K, const void *V, int64_t kv_rows_per_head,
    const int32_t *idx, int32_t k, int32_t batch, int32_t n_q_heads,
    int32_t n_kv_heads, int32_t head_dim, int32_t dtype, float scale,
    void *out, void *ws, size_t ws_bytes, void *stream, void **events);

/* Attention with an index list per query head (idx [batch][n_q_heads][k],
 * e.g. from a per_query_head retrieval): query head q attends to its own k
 * rows of KV head q / G.  Other arguments and errors as pariskv_sparse_attn;
 * the workspace is pariskv_attn_workspace_bytes(batch, n_q_heads, k, d). */
PARISKV_API int32_t pariskv_sparse_attn_per_query_head(
    const void *Q, const void *K, const void *V, int64_t kv_rows_per_head,
    const int32_t *idx, int32_t k, int32_t batch, int32_t n_q_heads,
    int32_t n_kv_heads, int32_t head_dim, int32_t dtype, float scale,
    void *out, void *ws, size_t ws_bytes, void *stream);

/* Same, timing its two kernels as pariskv_sparse_attn_profiled does. */
PARISKV_API int32_t pariskv_sparse_attn_per_query_head_profiled(
    const void *Q, const void *K, const void *V, int64_t kv_rows_per_head,
    const int32_t *idx, int32_t k, int32_t batch, int32_t n_q_heads,
    int32_t n_kv_heads, int32_t head_dim, int32_t dtype, float scale,
    void *out, void *ws, size_t ws_bytes, void *stream, void **events);

/* ---------------------------------------------------------------------- */
/* Sliding window.                                                         */
/* [TS] System-Level Innovations 2: four regions per (b, h) -- Sink (first */
/* S tokens), Retrieval (indexed; rows may live in host memory), Local     */
/* (the L most recent tokens before the buffer) and an Update Buffer of up */
/* to U new tokens.  When the buffer fills, the U oldest Local tokens move */
/* to Retrieval (rows copied to the far store, keys encoded into the       */
/* index) and the buffer becomes part of Local.  Attention covers the      */
/* sinks, the retrieved top-k and every Local and buffer token.  Host-side */
/* bookkeeping; the caller owns every buffer.                              */
/* ---------------------------------------------------------------------- */

/* Creates a window over `index`, whose keys [0, S + R) are the sinks and the
 * retrieval region (R = index size - S).  Positions: sinks [0, S), retrieval
 * [S, S + R), then the L local tokens [S + R, S + R + L); the buffer is empty.
 *   K_near, V_near  device [b][h][S + L + U][d] (key_dtype): rows [0, S) hold
 *                   the sinks; position p >= S + R lives at row
 *                   S + (p - S) % (L + U).  The caller fills the sinks and
 *                   the L local rows before the first call.
 *   K_far, V_far    device-accessible (HBM or mapped pinned host memory)
 *                   [b][h][far_rows_per_head][d]: position p of the
 *                   retrieval region at row p.  far_rows_per_head >= the
 *                   index capacity.
 *   n_local L, n_update U   U >= 1, L >= U, L a multiple of U.
 * The window keeps the pointers; they must outlive it.
 * Errors: INVALID_ARG, NOMEM. */
PARISKV_API int32_t pariskv_window_create(pariskv_index *index,
                                          int64_t n_local, int64_t n_update,
                                          void *K_near, void *V_near,
                                          void *K_far, void *V_far,
                                          int64_t far_rows_per_head,
                                          pariskv_window **out);

/* Appends one token per (b, h) (rows K_new/V_new[(b * n_kv_heads + h) *
 * new_rows_per_head], device-accessible) to the update buffer; when that
 * fills the buffer, moves the U oldest local tokens to the retrieval region
 * (far-store copies and an index encode, asynchronous on `stream`).  Their
 * ring rows start at S + R % (L + U) and wrap to row S when they pass the
 * ring's end, so R needs no alignment to U.
 * Errors: INVALID_ARG, CAPACITY (the index cannot take U more keys), HIP. */
PARISKV_API int32_t pariskv_window_append(pariskv_window *w, const void *K_new,
                                          const void *V_new,
                                          int64_t new_rows_per_head,
                                          void *stream);

/* Current tokens per (b, h), retrieval-region size R, and the attended
 * tail L + u (local plus buffer).  Any pointer may be NULL. */
PARISKV_API int32_t pariskv_window_state(const pariskv_window *w,
                                         int64_t *n_tokens,
                                         int64_t *n_retrieval,
                                         int64_t *n_tail);

/* Bytes of the workspace pariskv_window_attn needs for k listed rows. */
PARISKV_API int32_t pariskv_window_attn_workspace_bytes(const pariskv_window *w,
                                                        int32_t k,
                                                        size_t *bytes);

/* Attention of every query head over the k positions idx (the output of
 * pariskv_retrieve_topk on the window's index: sinks then retrieved, read
 * from the near store below S and from the far store above) and the tail
 * [S + R, S + R + L + u) read from the near store's ring.  Q, out, idx as for
 * pariskv_sparse_attn; dtype = the index's key_dtype.
 * Errors: INVALID_ARG, UNSUPPORTED, WORKSPACE, HIP. */
PARISKV_API int32_t pariskv_window_attn(const pariskv_window *w, const void *Q,
                                        const int32_t *idx, int32_t k,
                                        float scale, void *out, void *ws,
                                        size_t ws_bytes, void *stream);

/* Same as pariskv_window_attn, and times its two kernels: events holds 4
 * caller-created hipEvent_t, stamped as by pariskv_sparse_attn_profiled.
 * Not for use under stream capture. */
PARISKV_API int32_t pariskv_window_attn_profiled(const pariskv_window *w,
                                                 const void *Q,
                                                 const int32_t *idx, int32_t k,
                                                 float scale, void *out,
                                                 void *ws, size_t ws_bytes,
                                                 void *stream, void **events);

PARISKV_API void pariskv_window_destroy(pariskv_window *w);

/* ---------------------------------------------------------------------- */
/* Self-Indexing retrieval (a second workload on the same machinery).      */
/* [SI] "Self-Indexing KVCache: Predicting Sparse Attention from          */
/* Compressed Keys" (gist.science/paper/2603.14224), Methodology:          */
/*  A.4  keys are centred by their channel means mu (over the indexed      */
/*       prefill keys [S, n_keys) of each (b, h)), y = fp32(k - mu);       */
/*  A.1-2 y splits into 32 sub-vectors of 4 coordinates, each coded by its  */
/*       sign pattern: id_b = sum_j [y_{4b+j} < 0] 2^j, 16 clusters;       */
/*  A.3  the centroid of cluster (b, p) is the mean of its members' y_b    */
/*       (over the same prefill keys; an empty cluster has centroid 0);    */
/*  B    a query's LUT holds lut_b[p] = <qbar_b, c_{b,p}> and a key's score */
/*       is the sum of its LUT entries; the top-k by score is selected;    */
/*  C    the S sink tokens [0, S) are always selected and never scored.    */
/* Decode keys appended later are coded with the prefill means and join    */
/* the same clusters; the codebook is not updated.  qbar is the mean of    */
/* the G query heads of a KV head, as for ParisKV.  Arithmetic (fp32, no   */
/* contraction): lut_b[p] = ((0 + qbar_{4b} c_0) + qbar_{4b+1} c_1) + ...; */
/* score = sum over the key's 16 id bytes s, in order from 0, of           */
/* (lut_{2s}[id_{2s}] + lut_{2s+1}[id_{2s+1}]).  Means and centroids are   */
/* accumulated in fp64 and rounded once to fp32.  Selection order: (score  */
/* desc, position asc).  Attention over the selection: pariskv_sparse_attn. */
/* ---------------------------------------------------------------------- */

/* Shapes of a Self-Indexing index.
 *   head_dim   d (this build: 128).
 *   n_sink     S, keys [0, S) always selected, outside the means/codebook.
 *   batch, n_kv_heads, n_q_heads   as pariskv_config (G in {1, 2, 4, 8}).
 *   key_dtype  PARISKV_DTYPE_BF16 or _FP32 (K and Q).
 *   capacity   keys per (b, h); capacity - S <= 4,194,304. */
typedef struct pariskv_si_config {
    int32_t head_dim;
    int32_t n_sink;
    int32_t batch;
    int32_t n_kv_heads;
    int32_t n_q_heads;
    int32_t key_dtype;
    int64_t capacity;
} pariskv_si_config;

typedef struct pariskv_si_index pariskv_si_index; /* opaque host-side handle */

/* Stages pariskv_si_retrieve_topk_profiled brackets: LUT, scan, threshold,
 * compaction, top-k histogram, top-k select. */
#define PARISKV_SI_STAGES 6

/* Bytes of the device index buffer: per key and (b, h) 16 B of sign ids
 * (byte s: id_{2s} in the low nibble, id_{2s+1} in the high nibble), plus
 * per (b, h) the 128 fp32 means and the 32 x 16 x 4 fp32 centroids.
 * Errors: INVALID_ARG / UNSUPPORTED for a bad config. */
PARISKV_API int32_t pariskv_si_index_bytes(const pariskv_si_config *cfg,
                                           size_t *bytes);

/* Bytes of the device scratch pariskv_si_build_index needs for n_keys keys
 * (per-chunk fp64 partial sums; free after the build has run). */
PARISKV_API int32_t pariskv_si_build_workspace_bytes(
    const pariskv_si_config *cfg, int64_t n_keys, size_t *bytes);

/* Bytes of the device workspace pariskv_si_retrieve_topk needs for any index
 * size up to capacity (scores and candidate lists for up to capacity - S
 * keys per (b, h)). */
PARISKV_API int32_t pariskv_si_retrieve_workspace_bytes(
    const pariskv_si_config *cfg, int32_t k, size_t *bytes);

/* Creates a handle over `index_buf` (device, >= si_index_bytes, 256-byte
 * aligned, must outlive the handle): means and codebook from keys
 * [S, n_keys), sign ids of keys [0, n_keys), asynchronously on `stream`.
 *   K   device-accessible, key_dtype, element (b, h, i, j) at
 *       K[((b * n_kv_heads + h) * k_rows_per_head + i) * d + j].
 *   build_ws   device scratch of >= si_build_workspace_bytes(n_keys) bytes,
 *       in use until the build's kernels have run on `stream`.
 * Errors: INVALID_ARG, UNSUPPORTED, CAPACITY, WORKSPACE, NOMEM, HIP. */
PARISKV_API int32_t pariskv_si_build_index(
    const pariskv_si_config *cfg, void *index_buf, size_t index_bytes,
    const void *K, int64_t k_rows_per_head, int64_t n_keys, void *build_ws,
    size_t build_ws_bytes, void *stream, pariskv_si_index **out);

/* Codes n_new keys per (b, h) (rows K_new[(b * n_kv_heads + h) *
 * new_rows_per_head + r], device-accessible) with the stored means,
 * asynchronously on `stream`.  Errors: INVALID_ARG, CAPACITY, HIP. */
PARISKV_API int32_t pariskv_si_append_keys(pariskv_si_index *index,
                                           const void *K_new,
                                           int64_t new_rows_per_head,
                                           int64_t n_new, void *stream);

/* Current number of keys per (b, h), or -1 for a NULL handle. */
PARISKV_API int64_t pariskv_si_index_size(const pariskv_si_index *index);

/* Frees the host handle (never the caller's buffers). */
PARISKV_API void pariskv_si_index_destroy(pariskv_si_index *index);

/* Top-k of every (b, KV head) by LUT-GEMV score, asynchronously on `stream`.
 *   Q          device [batch][n_q_heads][d], key_dtype.
 *   k          S < k <= N.
 *   out_idx    device int32 [batch * n_kv_heads][k]: the sinks 0..S-1, then
 *              the k - S selected positions in ascending order.
 *   out_score  optional device fp32 [batch * n_kv_heads][k - S]: scores of
 *              out_idx[S..] in the same order.
 *   ws         device workspace of >= si_retrieve_workspace_bytes bytes
 *              (no initialisation needed; one call at a time per ws).
 * Errors: INVALID_ARG, WORKSPACE, HIP. */
PARISKV_API int32_t pariskv_si_retrieve_topk(const pariskv_si_index *index,
                                             const void *Q, int32_t k,
                                             int32_t *out_idx, float *out_score,
                                             void *ws, size_t ws_bytes,
                                             void *stream);

/* Same, with 2 * PARISKV_SI_STAGES caller-created hipEvent_t (start/stop per
 * stage, stamped by the kernels' own dispatches). */
PARISKV_API int32_t pariskv_si_retrieve_topk_profiled(
    const pariskv_si_index *index, const void *Q, int32_t k, int32_t *out_idx,
    float *out_score, void *ws, size_t ws_bytes, void *stream, void **events);

/* Parity-test introspection (synchronous).  ids_host [b][h][hi - lo][32]
 * (one 4-bit id per byte), mean_host [b][h][128], codebook_host
 * [b][h][32][16][4]; any may be NULL. */
PARISKV_API int32_t pariskv_si_debug_export(const pariskv_si_index *index,
                                            int64_t lo, int64_t hi,
                                            uint8_t *ids_host, float *mean_host,
                                            float *codebook_host);

/* Intermediates of the last pariskv_si_retrieve_topk that used `ws`:
 * which = 0: LUT fp32 [b][h][32][16]; 1: scores fp32 [b][h][N - S] (every
 * eligible key's, recomputed by this call from the index and the workspace's
 * byte table with the scan's arithmetic into a region of the workspace that
 * the retrieval leaves unused: the retrieval itself stores bins only);
 * 2: int32 [b][h][4] = (threshold bin T, #bin > T, #bin == T, candidates). */
PARISKV_API int32_t pariskv_si_debug_intermediate(const pariskv_si_index *index,
                                                  int32_t k, const void *ws,
                                                  size_t ws_bytes, int32_t which,
                                                  void *dst, size_t dst_bytes);

/* ---------------------------------------------------------------------- */
/* Introspection for parity tests (synchronous; not for the hot path).     */
/* ---------------------------------------------------------------------- */

/* Copies rows [lo, hi) of every (b, h) to host arrays laid out
 * [b][h][hi - lo][...]: ids_host B bytes, nib_host d/2 bytes (coordinate 2p
 * in the low nibble of byte p), w_host B fp16 bit patterns per key.  Any of
 * the three may be NULL.  Synchronises the index's last stream. */
PARISKV_API int32_t pariskv_debug_export(const pariskv_index *index,
                                         int64_t lo, int64_t hi,
                                         uint8_t *ids_host, uint8_t *nib_host,
                                         uint16_t *w_host);

/* Intermediates of the last pariskv_retrieve_topk that used `ws` (same
 * index, same k), copied to host after a device synchronisation.
 *   which = 0: vote table uint8 [b][h][16][256], the one the scan reads:
 *              row s is indexed by byte s of a key's ids; m = 8: subspace
 *              s's LUT; m = 4: entry v = LUT_{2s}[v & 15] + LUT_{2s+1}[v >> 4]
 *           1: yq         float [b][h][d] (rotated group query)
 *           2: scores     uint8 [b][h][E]  (E = N - S)
 *           3: cand       int32 [b][h][C]  ascending key positions
 *           4: est        float [b][h][C]  aligned with cand
 *           5: threshold  int32 [b][h][4]  (T, #score > T, tie quota, C)
 * Errors: INVALID_ARG (unknown which, dst_bytes too small), HIP. */
PARISKV_API int32_t pariskv_debug_intermediate(const pariskv_index *index,
                                               int32_t k, const void *ws,
                                               size_t ws_bytes, int32_t which,
                                               void *host_dst,
                                               size_t dst_bytes);

/* E and C for the index's current size and this k. */
PARISKV_API int32_t pariskv_retrieve_sizes(const pariskv_index *index,
                                           int32_t k, int64_t *E, int64_t *C);

/* The library's fp32 RSQ-IP codebook for subspace size m (levels L[8],
 * thresholds tau[7]) and its rotation scale fp32(1/sqrt(d)).  Host-only. */
PARISKV_API int32_t pariskv_codebook(int32_t m, float *L, float *tau);
PARISKV_API float pariskv_rot_scale(int32_t head_dim);

/* The rotation's random diagonal D from a 64-bit seed, for callers that
 * keep a seed rather than the signs ([TS] Core Algorithmic Innovations 1:
 * one random rotation, implemented via SRHT, shared by keys and queries):
 * signs[j] = -1 when bit 63 of the j-th output (j = 0 .. head_dim - 1) of
 * SplitMix64 seeded with `seed` is set, else +1 (Steele, Lea and Flood,
 * "Fast Splittable Pseudorandom Number Generators", OOPSLA 2014).  The
 * result can be passed as pariskv_build_index's srht_signs.  Host-only.
 *   signs   host int8 [head_dim], written.
 * Errors: INVALID_ARG (null signs, head_dim < 1 or > 1024). */
PARISKV_API int32_t pariskv_srht_signs_from_seed(uint64_t seed, int32_t head_dim,
                                                 int8_t *signs);

/* Human-readable text for a status code (static storage). */
PARISKV_API const char *pariskv_status_string(int32_t status);

#ifdef __cplusplus
}
#endif
#endif /* PARISKV_H */
