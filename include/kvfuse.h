/*
 * libkvfuse - one transformer layer of RAG KV-cache fusion with selective
 * recomputation, for AMD Instinct MI355X (gfx950).
 *
 * Sources, cited by page title and section / equation:
 *   [QCF] "QCFuse: Query-Aware Cache Fusion via Compressed View for Efficient
 *         RAG Serving": 2.1.1 (Eq. 1, context C and query U), 2.1.2 (Eq. 3-5,
 *         per-chunk caches and their re-positioning), 2.1.3 (Eq. 6-7,
 *         selective recomputation and the fused cache), 2.2.1 (EPIC's
 *         boundary tokens), 3.2.1 (Eq. 9-11, query-to-context attention mass
 *         and TopK), 3.3.1 (Eq. 14, per-chunk anchors, Knorm ranking).
 *   [KVB] "KVBoost: Chunk-Level Key-Value Cache Reuse with Deviation-Guided
 *         Recomputation for Efficient Large Language Model Inference":
 *         3.1 (Eq. 1-2, projections, attention, cache layout), 3.2 (Eq. 3,
 *         RoPE and the rotation correction), 4.1 (attention-sink tokens),
 *         4.5 (Eq. 7, KIVI int8/int4), 4.6.1 (Algorithm 1, seam windows),
 *         4.6.2 (Algorithm 2, key-deviation scoring), 7.3 (memory budget:
 *         an 8-bit cache halves a 16-bit one).
 *
 * One layer, per request:  N context tokens (stitched chunks) then U query
 * tokens, T = N + U.  The path is
 *   kvf_rerotate -> kvf_score -> kvf_select_topk -> kvf_recompute_qkv
 *   -> kvf_scatter_kv -> kvf_sparse_q_attention
 * every call enqueues HIP kernels on the caller's stream and returns; there
 * is no host synchronisation inside the library.  Other selectors feed the
 * same recompute path: kvf_select_static builds a mask of static positions
 * (attention sinks, chunk boundary tokens, seam windows) that kvf_select_topk
 * takes as a forced set, and kvf_select_topk_segmented selects per chunk
 * (e.g. over kvf_score's KVF_SCORE_KEY_NORM scores).  With an int8-resident
 * fused cache (kvf_q8_cache) the calls that touch the cache have _q8 forms:
 *   kvf_rerotate_q8 -> kvf_score_q8 -> kvf_select_topk -> kvf_recompute_qkv
 *   -> kvf_scatter_kv_q8 -> kvf_sparse_q_attention_q8
 * The re-positioning and a score can share one pass over the keys:
 * kvf_rerotate_deviation / kvf_rerotate_q8_deviation (re-positioning plus
 * the deviation score, with the probe keys computed first) and
 * kvf_rerotate_score_attn_mass (keys-only re-positioning inside the
 * attention-mass score's first pass).
 *
 * Conventions for every call:
 *  - Pointers are DEVICE pointers unless the comment says "host".
 *  - All tensors are contiguous row-major.  K/V caches are token-major
 *    [rows, Hkv, d] ([KVB] 3.1).  Q is [rows, Hq, d].  Query head h reads
 *    kv head h / (Hq / Hkv).  Weights are [out, in], the projection is x W^T.
 *  - Element type: kvf_layer_desc.dtype selects fp32 or bf16 for every
 *    float tensor of a call (activations, weights, caches, outputs).
 *    Scores, statistics, LSE and rope tables are always fp32.
 *  - Ownership: the caller allocates every buffer, including workspaces
 *    (sized by the *_workspace_size queries).  The library never allocates or
 *    frees device memory and keeps no pointer after a call returns.
 *  - Streams: `stream` is a hipStream_t passed as void*; NULL is the null
 *    stream.
 *  - Errors: arguments are validated on the host before anything is
 *    enqueued: KVF_ERR_INVALID_ARG for malformed arguments,
 *    KVF_ERR_UNSUPPORTED for shapes the kernels do not implement,
 *    KVF_ERR_WORKSPACE for a too-small workspace.  A failed launch returns
 *    KVF_ERR_HIP.  kvf_last_error() gives a thread-local text of the last
 *    failure.  On error, output contents are undefined.  No C++ exception
 *    crosses this interface and the library never aborts.
 *  - Device-side indices (row maps, positions, chunk tables) are checked
 *    inside the kernels against the sizes passed here; an out-of-range
 *    entry makes the kernel skip that row (its outputs are left unwritten)
 *    instead of reading or writing outside the buffers.
 *  - Thread safety: calls may be made from several host threads; calls that
 *    write the same buffers must be ordered by the caller.
 *  - Debugging: with KVF_SYNC_CHECK=1 in the environment (read once per
 *    process), every call synchronises its stream after enqueueing and
 *    returns KVF_ERR_HIP if one of its kernels failed to launch or run, so a
 *    fault is reported by the call that caused it.  Streams being captured
 *    into a graph are not synchronised.
 */
#ifndef KVFUSE_H
#define KVFUSE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define KVF_ABI_VERSION 11
#define KVF_MAX_REQ 64      /* requests per call (batch metadata is passed by value) */

typedef enum {
  KVF_OK = 0,
  KVF_ERR_INVALID_ARG = 1,
  KVF_ERR_UNSUPPORTED = 2,
  KVF_ERR_WORKSPACE = 3,
  KVF_ERR_HIP = 4
} kvf_status;

typedef enum { KVF_F32 = 0, KVF_BF16 = 1 } kvf_dtype;

typedef enum {
  KVF_SCORE_DEVIATION = 0,   /* [KVB] 4.6.2 Algorithm 2: 1 - mean_h cos(K, K~) */
  KVF_SCORE_ATTN_MASS = 1,   /* [QCF] 3.2.1 Eq. 9-10: query-to-context mass  */
  KVF_SCORE_KEY_NORM = 2,    /* [QCF] 3.3.1 Knorm: L2 norm of the cached key  */
  /* flag OR-ed into the mode: add this layer's score to `scores` instead of
   * overwriting them - I(t) = sum over layers of the per-layer score
   * ([QCF] 3.2.1 Eq. 10 over all layers, 3.4.2 Eq. 20 over a layer set) */
  KVF_SCORE_ACCUMULATE = 0x100
} kvf_score_mode;

enum { KVF_OUT_Q = 1, KVF_OUT_K = 2, KVF_OUT_V = 4 };

/* Layer shape (host struct).  head_dim must be 64 or 128; n_q_heads must be a
 * multiple of n_kv_heads.  RoPE is the rotate-half form (channel j paired
 * with j + d/2), the reading this library takes of [KVB] 3.2 Eq. 3. */
typedef struct {
  int32_t hidden;
  int32_t n_q_heads;
  int32_t n_kv_heads;
  int32_t head_dim;
  int32_t dtype;             /* kvf_dtype */
} kvf_layer_desc;

/* Request batch (host struct, HOST arrays).  Request r owns rows
 * [cu_T[r], cu_T[r+1]) of x and of the fused cache; its first n_ctx[r] rows
 * are the context C, the rest the query U ([QCF] 2.1.1). */
typedef struct {
  int32_t n_req;             /* 1 .. KVF_MAX_REQ */
  const int32_t* cu_T;       /* host [n_req + 1], cu_T[0] = 0, non-decreasing */
  const int32_t* n_ctx;      /* host [n_req], 0 <= n_ctx[r] <= T_r */
} kvf_batch;

/* One stitched chunk (device array element, 32 bytes): `len` cached rows
 * starting at pool row `src_row`, encoded at chunk-local positions 0..len-1,
 * land at fused rows dst_row.. with request positions pos0.. ([QCF] 2.1.2
 * Eq. 4).  pool_chunk indexes per-chunk KIVI key statistics. */
typedef struct {
  int32_t src_row;
  int32_t dst_row;
  int32_t pos0;
  int32_t len;
  int32_t pool_chunk;
  int32_t reserved[3];
} kvf_chunk;

/* KIVI quantised cache ([KVB] 4.5 Eq. 7, b = 8 or 4): value = min + code *
 * scale.  Keys: per (pool chunk, kv head, channel) statistics; values: per
 * (pool row, kv head).  b = 8: one code per byte.  b = 4: two codes per byte,
 * channel 2i in bits 0-3 and channel 2i + 1 in bits 4-7 of byte i of the
 * row, so a [pool_rows, Hkv, d] cache takes [pool_rows, Hkv, d / 2] bytes. */
typedef struct {
  const uint8_t* k_codes;    /* [pool_rows, Hkv, d * bits / 8] */
  const uint8_t* v_codes;    /* [pool_rows, Hkv, d * bits / 8] */
  const float* k_min;        /* [n_pool_chunks, Hkv, d] */
  const float* k_scale;      /* [n_pool_chunks, Hkv, d] */
  const float* v_min;        /* [pool_rows, Hkv] */
  const float* v_scale;      /* [pool_rows, Hkv] */
  int32_t n_pool_chunks;
  int32_t bits;              /* 8 or 4 */
} kvf_kivi;

/* Int8-resident fused cache ([KVB] 4.5 Eq. 7 with b = 8, kept by the fused
 * cache itself instead of expanding it to bf16 - [KVB] 7.3: an 8-bit cache
 * takes half the bytes).  Device arrays.  Every (row, kv head) of K and of V
 * is d one-byte codes plus one float pair (min, scale); value = min + code *
 * scale.  A (row, head) group's statistics come from that row's own d values
 * - one group per token for keys as for values, because fused rows are
 * written one at a time (by re-positioning and by fusion).  Encoding, fp32
 * in this order: range = max - min; scale = range / 255; inv = 255 / range;
 * code = (x - min) * inv rounded half to even, clamped to [0, 255]; a group
 * with range 0 gets scale 0 and codes 0.  Written by kvf_rerotate_q8 and
 * kvf_scatter_kv_q8, read (decoded on load) by kvf_score_q8 and
 * kvf_sparse_q_attention_q8. */
typedef struct {
  uint8_t* k_codes;          /* [rows, Hkv, d] */
  uint8_t* v_codes;          /* [rows, Hkv, d] */
  float* k_stats;            /* [rows, Hkv, 2]: (min, scale) */
  float* v_stats;            /* [rows, Hkv, 2] */
  int64_t rows;
} kvf_q8_cache;

/* Static recompute rules (host struct); every field >= 0, 0 turns a rule off.
 *   sink:     request positions 0 .. sink-1 ([KVB] 4.1, attention-sink
 *             tokens always kept live);
 *   boundary: the first `boundary` positions of every stitched chunk
 *             ([QCF] 2.2.1, EPIC's boundary tokens);
 *   seam:     R of [KVB] 4.6.1 Algorithm 1: positions max(0, p - R) .. p - 1
 *             before every chunk start p > 0.
 * Every range is clipped to the request's context [0, N). */
typedef struct {
  int32_t sink;
  int32_t boundary;
  int32_t seam;
} kvf_static_rules;

/* One selection segment of kvf_select_topk_segmented (device array element,
 * 32 bytes): scores req's context positions pos0 .. pos0+len-1 and keeps k of
 * them; its picks land at slots out_off .. out_off+k-1 of the request's k_r
 * picks ([QCF] 3.3.1 Eq. 14: A_i = TopK(G_i, ceil(r_a |c_i|)) per chunk). */
typedef struct {
  int32_t req;
  int32_t pos0;
  int32_t len;
  int32_t k;
  int32_t out_off;
  int32_t reserved[3];
} kvf_segment;

/* ---------------------------------------------------------------------------
 * kvf_rope_table - cos/sin of the rotation angles p * theta_j for positions
 * p in [0, n_pos) and j in [0, d/2), theta_j = base^(-2j/d) ([KVB] 3.2,
 * Eq. 3).  Angles and cos/sin are evaluated in fp64 on the device and
 * rounded to fp32.  cos_tab, sin_tab: [n_pos, d/2] fp32.  Built once per
 * (base, d); every call that rotates takes these tables.
 */
kvf_status kvf_rope_table(double base, int32_t head_dim, int32_t n_pos,
                          float* cos_tab, float* sin_tab, void* stream);

/* ---------------------------------------------------------------------------
 * kvf_rerotate - S1: re-position and stitch per-chunk caches into the fused
 * cache ([QCF] 2.1.2 Eq. 4; [KVB] 3.2).  For every chunk c and t < len:
 *   fused_k[dst_row + t] = R(pos0) * K_pool[src_row + t]   (delta rotation:
 *                          the cached key already carries R(t), and
 *                          R(pos0) R(t) = R(pos0 + t))
 *   fused_v[dst_row + t] = V_pool[src_row + t]
 * Dense caches: pool_k, pool_v [pool_rows, Hkv, d] in dtype, kivi = NULL.
 * KIVI caches (8 or 4 bits): pool_k = pool_v = NULL and kivi != NULL; codes
 * are decoded (min + code * scale, fp32) before the rotation
 * (dequant-on-load).  Output dtype must be bf16 for KIVI caches.
 * k_only = 1 (dense caches only): keys only - the loader has already
 *   stitched the values into fused_v ([QCF] 2.1.2: values keep their token
 *   order; only keys carry the rotation, [KVB] 3.2 Eq. 3), so pool_v and
 *   fused_v are not read or written (either may be NULL).  pool_k may be
 *   fused_k itself (in place) when every chunk has src_row == dst_row; a
 *   thread reads both channels of each rotation pair before writing them.
 *   Chunks whose rows overlap between source and destination otherwise are
 *   undefined.  k_only = 0 gathers keys and values as above.
 * chunks: device [n_chunks]; max_chunk_len (host) bounds every len.
 * rope tables cover positions [0, rope_n_pos); pos0 >= rope_n_pos skips the
 * chunk.  Fused rows no chunk covers are not written.
 */
kvf_status kvf_rerotate(const kvf_layer_desc* layer, const kvf_chunk* chunks,
                        int32_t n_chunks, int32_t max_chunk_len,
                        const void* pool_k, const void* pool_v,
                        const kvf_kivi* kivi, int64_t pool_rows,
                        const float* rope_cos, const float* rope_sin,
                        int32_t rope_n_pos, void* fused_k, void* fused_v,
                        int64_t fused_rows, int32_t k_only, void* stream);

/* ---------------------------------------------------------------------------
 * kvf_rerotate_deviation - S1 and the deviation score S2b in one pass
 * ([KVB] 4.6.2 Algorithm 2 at one layer: the probe's fresh keys are compared
 * with the re-positioned cached keys; [QCF] 2.1.2 Eq. 4 for the
 * re-positioning).  Does exactly what kvf_rerotate does with the same
 * arguments, and for every fused row a chunk writes that is a context row of
 * `batch` (row cu_T[r] + i with i < n_ctx[r]) it also writes the
 * KVF_SCORE_DEVIATION score of kvf_score to scores[cu_N[r] + i]
 * (cu_N = prefix sums of n_ctx), computed from the key as fused_k stores it
 * (bf16-rounded for bf16 layers), so that the score pass does not read the
 * fused keys back.  eligible ([sum N] uint8 or NULL) and accumulate (0 or
 * 1; 1 = scores[t] += this layer's score) behave as in kvf_score.
 * k_fresh: [fused_rows, Hkv, d] in dtype, the probe's keys (kvf_recompute_qkv
 *   with KVF_OUT_K over the rows), indexed like the fused cache; an
 *   ineligible row's k_fresh is not read.
 * Context rows that no chunk covers get no score (their entries are left
 * as they were): the chunks should tile every request's context, as the
 * loader's stitch does.
 * Errors: those of kvf_rerotate; KVF_ERR_UNSUPPORTED unless Hkv * d / 16 is
 * a power of two of at most 64 (a row's key is reduced within one wave).
 */
kvf_status kvf_rerotate_deviation(const kvf_layer_desc* layer, const kvf_batch* batch,
                                  const kvf_chunk* chunks, int32_t n_chunks, int32_t max_chunk_len,
                                  const void* pool_k, const void* pool_v, const kvf_kivi* kivi,
                                  int64_t pool_rows, const float* rope_cos, const float* rope_sin,
                                  int32_t rope_n_pos, void* fused_k, void* fused_v,
                                  int64_t fused_rows, int32_t k_only, const void* k_fresh,
                                  const uint8_t* eligible, int32_t accumulate, float* scores,
                                  void* stream);

/* ---------------------------------------------------------------------------
 * kvf_rerotate_q8 - S1 into an int8-resident fused cache (kvf_q8_cache):
 * the chunks of kvf_rerotate (k_only = 0), with fused row dst_row + t of
 * every chunk written as
 *   K: R(pos0) * K_pool[src_row + t] - the per-chunk key decoded and
 *      rotated in fp32, then encoded (one group per row and kv head);
 *   V: from an 8-bit KIVI per-chunk cache, the row's codes and (min, scale)
 *      copied unchanged (KIVI values are per-token 8-bit groups already);
 *      from a dense bf16 cache, the value encoded.
 * Per-chunk cache: dense bf16 (pool_k, pool_v; kivi = NULL) or KIVI with
 * bits = 8 (pool_k = pool_v = NULL); a 4-bit KIVI cache gives
 * KVF_ERR_UNSUPPORTED.  layer->dtype must be KVF_BF16.  Fused rows no chunk
 * covers are not written; chunk descriptors are checked as in kvf_rerotate.
 */
kvf_status kvf_rerotate_q8(const kvf_layer_desc* layer, const kvf_chunk* chunks,
                           int32_t n_chunks, int32_t max_chunk_len,
                           const void* pool_k, const void* pool_v,
                           const kvf_kivi* kivi, int64_t pool_rows,
                           const float* rope_cos, const float* rope_sin,
                           int32_t rope_n_pos, const kvf_q8_cache* fused,
                           void* stream);

/* ---------------------------------------------------------------------------
 * kvf_rerotate_q8_deviation - kvf_rerotate_q8 and the deviation score S2b in
 * one pass ([KVB] 4.6.2 Algorithm 2 at one layer), as kvf_rerotate_deviation
 * is for a bf16 cache: every context row a chunk writes also gets the
 * KVF_SCORE_DEVIATION score of kvf_score_q8, from the key as the int8 cache
 * now stores it (min + code * scale of its own codes and statistics), at
 * scores[cu_N[r] + i].  k_fresh: bf16 [fused->rows, Hkv, d].  eligible and
 * accumulate as in kvf_score.  Context rows no chunk covers get no score.
 * Errors: those of kvf_rerotate_q8; KVF_ERR_UNSUPPORTED unless Hkv * d / 8
 * is a power of two of at most 64 and divides 256 (a row's items stay
 * within one wave and one workgroup).
 */
kvf_status kvf_rerotate_q8_deviation(const kvf_layer_desc* layer, const kvf_batch* batch,
                                     const kvf_chunk* chunks, int32_t n_chunks,
                                     int32_t max_chunk_len, const void* pool_k,
                                     const void* pool_v, const kvf_kivi* kivi, int64_t pool_rows,
                                     const float* rope_cos, const float* rope_sin,
                                     int32_t rope_n_pos, const kvf_q8_cache* fused,
                                     const void* k_fresh, const uint8_t* eligible,
                                     int32_t accumulate, float* scores, void* stream);

/* ---------------------------------------------------------------------------
 * kvf_score - S2: one fp32 score per context token; scores [sum_r n_ctx[r]]
 * request-major.  mode: one of the modes below, optionally OR KVF_SCORE_ACCUMULATE
 * (scores[t] += this layer's score; a NaN already there stays NaN).
 * eligible: [sum N] uint8 or NULL.  A position whose byte is 0 is not scored:
 *   its score is set to NaN, which every selection ranks below all numbers -
 *   the candidate set of CacheBlend's layer-by-layer filtering ([QCF] 2.2.1):
 *   only the previous layer's picks stay in play.  Deviation and key norm
 *   skip the ineligible rows' loads (their k_fresh rows need not exist).
 * KVF_SCORE_DEVIATION ([KVB] 4.6.2 Algorithm 2, one layer):
 *   score_t = 1 - (1/Hkv) sum_h cos(fused_k[t, h], k_fresh[t, h]),
 *   cos := 0 when either norm is 0.  fused_k and k_fresh are [sum T, Hkv, d]
 *   indexed by the same rows; only context rows are read.  q_u unused.
 * KVF_SCORE_ATTN_MASS ([QCF] 3.2.1 Eq. 9-10, one layer):
 *   q_u [sum_r U_r, Hq, d] holds the rotated queries of each request's query
 *   tokens (positions N..T-1), request-major.  fused_k must already hold the
 *   query tokens' keys at rows N..T-1.  Query token i attends causally to
 *   keys 0..N+i; each (i, head) softmax is over that whole row, and
 *   score_t = sum over the last n_last_q query tokens (all when <= 0) and all
 *   query heads of the probability at context position t.  Softmax scale is
 *   1/sqrt(d).  Needs a workspace of kvf_score_workspace_size() bytes; its
 *   first 65536 bytes are arrival counters (one per 128-key context tile, so
 *   at most 16384 tiles per call, else KVF_ERR_UNSUPPORTED) that must be
 *   zero before its first use (zero-fill it once when allocating it); every
 *   completed call leaves them zero, so calls of any shape may share one
 *   workspace.  Calls that share a workspace must not overlap.  The scores
 *   are deterministic (fixed summation order).
 * KVF_SCORE_KEY_NORM ([QCF] 3.3.1, the Knorm ranking rule):
 *   score_t = sqrt(sum over heads h and channels j of fused_k[t, h, j]^2),
 *   fp32 accumulation.  The norm is rotation invariant, so the re-positioned
 *   fused cache gives the per-chunk cache's score.  k_fresh and q_u unused.
 *   Rank the negated scores for "smallest norm first".
 */
kvf_status kvf_score(kvf_score_mode mode, const kvf_layer_desc* layer,
                     const kvf_batch* batch, const void* fused_k,
                     const void* k_fresh, const void* q_u, int32_t n_last_q,
                     const uint8_t* eligible, float* scores, void* workspace,
                     size_t ws_bytes, void* stream);
size_t kvf_score_workspace_size(kvf_score_mode mode, const kvf_layer_desc* layer,
                                const kvf_batch* batch, int32_t n_last_q);

/* ---------------------------------------------------------------------------
 * kvf_rerotate_score_attn_mass - keys-only S1 and the attention-mass score
 * S2c in one pass over the keys ([QCF] 2.1.2 Eq. 4 with [KVB] 3.2 Eq. 3 for
 * the re-positioning; [QCF] 3.2.1 Eq. 9-10 for the score).  Equal to
 * kvf_rerotate(k_only = 1) of `chunks` from pool_k into fused_k, followed by
 * kvf_score(KVF_SCORE_ATTN_MASS [| ACCUMULATE when accumulate = 1]) over
 * fused_k: the pass that first reads a tile of context keys reads them from
 * pool_k, turns each by its chunk's R(pos0), scores them and writes them to
 * fused_k, so the fused keys are not written and read back before the score.
 *   chunks, pool_k [pool_rows, Hkv, d] (bf16 layers: bf16), rope tables,
 *     max_chunk_len, fused_rows (>= the batch's rows): as in kvf_rerotate
 *     with k_only = 1 (pool_k may be fused_k when every chunk has
 *     src_row == dst_row); every chunk's fused rows must lie within the
 *     batch's requests (rows outside them are not re-positioned).  Query
 *     rows (N..T-1), which no chunk covers, must already hold the query
 *     tokens' keys (kvf_recompute_qkv of the query rows).
 *   q_u, n_last_q, eligible, scores, workspace (size from
 *     kvf_score_workspace_size(KVF_SCORE_ATTN_MASS, ...)): as in kvf_score.
 * Errors: those of kvf_rerotate and kvf_score.
 */
kvf_status kvf_rerotate_score_attn_mass(const kvf_layer_desc* layer, const kvf_batch* batch,
                                        const kvf_chunk* chunks, int32_t n_chunks,
                                        int32_t max_chunk_len, const void* pool_k, int64_t pool_rows,
                                        const float* rope_cos, const float* rope_sin,
                                        int32_t rope_n_pos, void* fused_k, int64_t fused_rows,
                                        const void* q_u, int32_t n_last_q,
                                        const uint8_t* eligible, int32_t accumulate, float* scores,
                                        void* workspace, size_t ws_bytes, void* stream);

/* kvf_score_q8 - kvf_score over an int8-resident fused cache: modes
 * KVF_SCORE_DEVIATION and KVF_SCORE_KEY_NORM (optionally OR
 * KVF_SCORE_ACCUMULATE), with the same definitions, batch, eligibility and
 * output; every fused key is decoded in fp32 (min + code * scale, one fused
 * multiply-add) before use.  k_fresh (deviation) is bf16 [sum T, Hkv, d].
 * KVF_SCORE_ATTN_MASS gives KVF_ERR_UNSUPPORTED.  No workspace. */
kvf_status kvf_score_q8(kvf_score_mode mode, const kvf_layer_desc* layer,
                        const kvf_batch* batch, const kvf_q8_cache* fused,
                        const void* k_fresh, const uint8_t* eligible, float* scores,
                        void* stream);

/* ---------------------------------------------------------------------------
 * kvf_score_attn_mass_noalloc - kvf_score(KVF_SCORE_ATTN_MASS) for callers
 * that cannot allocate device memory (code being captured into a graph,
 * tight serving loops, harnesses that forbid allocation).  Same arguments
 * and result as kvf_score in attention-mass mode (accumulate: 1 adds to
 * `scores` like KVF_SCORE_ACCUMULATE), but no workspace: the call uses a
 * scratch array of KVF_NOALLOC_SCRATCH_BYTES (48 MiB) inside the library,
 * one per GPU, held from the first use on that GPU until the process ends.
 * Calls whose kvf_score_workspace_size would exceed it get
 * KVF_ERR_UNSUPPORTED.  The call allocates and frees nothing.  Every call on
 * a GPU shares that GPU's array: calls that overlap in time on one GPU (on
 * different streams, or from several host threads) race and give undefined
 * scores; order them.  The device the stream belongs to must be current.
 */
#define KVF_NOALLOC_SCRATCH_BYTES (48u << 20)
kvf_status kvf_score_attn_mass_noalloc(const kvf_layer_desc* layer, const kvf_batch* batch,
                                       const void* fused_k, const void* q_u, int32_t n_last_q,
                                       const uint8_t* eligible, float* scores, int32_t accumulate,
                                       void* stream);

/* ---------------------------------------------------------------------------
 * kvf_select_topk - S3: P_r = TopK(score, k_r) per request ([QCF] 3.2.1
 * Eq. 11).  Order: larger score first; ties to the lower position; -0 == +0;
 * NaN ranks below every number.  k_per_req: HOST [n_req], 0 <= k_r <= N_r.
 * scores: [sum N] request-major, or NULL to rank every position equal.
 * forced: [sum N] uint8 (may be NULL): positions with a nonzero byte rank
 *   above every score, so with f_r forced positions P_r holds all of them
 *   when f_r <= k_r (the rest by score) and the f_r lowest otherwise.  With
 *   scores NULL and k_r = f_r, P_r is exactly the forced set.
 *   out_idx  [sum k_r]: P_r ascending, positions within the request.
 *   out_rows [sum (k_r + U_r)] (may be NULL): flat rows (cu_T[r] + p) of
 *            P_r followed by the request's query rows, i.e. the rows to
 *            recompute, ascending per request.
 *   out_pos  [sum (k_r + U_r)] (may be NULL): the matching positions.
 *   out_mask [sum N] uint8 (may be NULL): 1 at the picks, 0 at every other
 *            context position (the next layer's `eligible` set in
 *            kvf_score).
 * Needs kvf_select_workspace_size() bytes of workspace (0 today; the
 * argument is reserved).
 */
kvf_status kvf_select_topk(const float* scores, const uint8_t* forced,
                           const kvf_batch* batch,
                           const int32_t* k_per_req, int32_t* out_idx,
                           int32_t* out_rows, int32_t* out_pos, uint8_t* out_mask,
                           void* workspace, size_t ws_bytes, void* stream);
size_t kvf_select_workspace_size(const kvf_batch* batch);

/* ---------------------------------------------------------------------------
 * kvf_select_topk_segmented - per-segment TopK ([QCF] 3.3.1 Eq. 14): every
 * segment g keeps the g.k best of its positions by kvf_select_topk's order
 * (and forced rule), written ascending as request positions at
 * out_idx[sum_{r' < g.req} k_r' + g.out_off ..].  k_per_req: HOST [n_req],
 * the number of picks of each request (the sum of its segments' k).
 * out_rows / out_pos (both or neither): as in kvf_select_topk, the picks'
 * flat rows and positions at the same slots of each request's k_r + U_r
 * list, then the U_r query rows.  A request's picks come out ascending when
 * its segments are ascending, disjoint and take consecutive output slots in
 * that order.  segs: device [n_segs].  A segment whose request, range
 * (pos0 + len <= N_req), k (<= len) or slots (out_off + k <= k_req) is out
 * of bounds writes nothing.
 */
kvf_status kvf_select_topk_segmented(const float* scores, const uint8_t* forced,
                                     const kvf_batch* batch, const kvf_segment* segs,
                                     int32_t n_segs, const int32_t* k_per_req,
                                     int32_t* out_idx, int32_t* out_rows,
                                     int32_t* out_pos, void* stream);

/* ---------------------------------------------------------------------------
 * kvf_select_static - mask[cu_N[r] + t] = 1 if a static rule picks context
 * position t of request r, else 0 (kvf_static_rules; [KVB] 4.1, 4.6.1
 * Algorithm 1; [QCF] 2.2.1).  mask: device [sum N] uint8, every byte
 * written.  The chunk starts are read from the chunk table kvf_rerotate
 * takes (device [n_chunks]): chunk c starts at context position
 * dst_row - cu_T[r] of the request r whose context rows hold dst_row;
 * chunks whose dst_row lies in no request's context are ignored.
 */
kvf_status kvf_select_static(const kvf_batch* batch, const kvf_chunk* chunks,
                             int32_t n_chunks, const kvf_static_rules* rules,
                             uint8_t* mask, void* stream);

/* Host-side count of the positions kvf_select_static marks per request, from
 * a HOST copy of the same chunk table: counts HOST [n_req].  Sizes the
 * kvf_select_topk call that turns the mask into a position list. */
kvf_status kvf_static_counts(const kvf_batch* batch, const kvf_chunk* chunks_host,
                             int32_t n_chunks, const kvf_static_rules* rules,
                             int32_t* counts);

/* ---------------------------------------------------------------------------
 * kvf_recompute_qkv - S4: fresh Q/K/V of M rows ([QCF] 2.1.3 KV^New;
 * [KVB] 3.1 Eq. 1 and 3.2 Eq. 3).  For m < M with r = row_src[m] and
 * p = row_pos[m]:
 *   q_out[m] = R(p) x[r] Wq^T   (if out_mask & KVF_OUT_Q)   [M, Hq, d]
 *   k_out[m] = R(p) x[r] Wk^T   (if out_mask & KVF_OUT_K)   [M, Hkv, d]
 *   v_out[m] =      x[r] Wv^T   (if out_mask & KVF_OUT_V)   [M, Hkv, d]
 * x: [x_rows, hidden]; w_qkv: [(Hq + 2 Hkv) d, hidden] = [Wq; Wk; Wv].
 * row_src may be NULL (identity, requires M <= x_rows).  fp32 accumulation.
 * A row whose row_src entry is outside [0, x_rows) or (for Q/K) whose
 * position is outside the rope table is left unwritten.
 * The same call builds per-chunk caches ahead of serving ([QCF] 2.1.2 Eq. 3):
 * pass the cached hidden states with chunk-local positions and mask K|V.
 * kv_out_row (optional, [M]): when given, K/V row m is written to row
 * kv_out_row[m] of k_out / v_out, which then hold kv_out_rows rows - the
 * fresh K/V go straight into the fused cache, which fuses S5's scatter
 * ([QCF] 2.1.3 Eq. 7) into this call.  Entries outside [0, kv_out_rows) are
 * skipped; destination rows must be unique.  Q is always written densely.
 * workspace: kvf_recompute_workspace_size(layer, M, out_mask) bytes of
 * device memory (may be NULL when that is 0).  Calls with few rows split the
 * hidden dimension: the workspace then holds 4096 bytes of per-tile arrival
 * counters, which must be zero before its first use and which every call
 * leaves zero, followed by the slices' partial sums.  Calls of any shape may
 * share one workspace (the counters sit at a fixed offset) but must not
 * overlap in time.
 */
size_t kvf_recompute_workspace_size(const kvf_layer_desc* layer, int32_t M,
                                    uint32_t out_mask);
kvf_status kvf_recompute_qkv(const kvf_layer_desc* layer, const void* x,
                             int64_t x_rows, const int32_t* row_src,
                             const int32_t* row_pos, int32_t M,
                             const void* w_qkv, uint32_t out_mask,
                             const float* rope_cos, const float* rope_sin,
                             int32_t rope_n_pos, void* q_out, void* k_out,
                             void* v_out, const int32_t* kv_out_row,
                             int64_t kv_out_rows, void* workspace,
                             size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * kvf_scatter_kv - S5: KV^Fuse_p = KV^New_p for the recomputed rows
 * ([QCF] 2.1.3 Eq. 7), written in place:
 *   fused_k[dst_row[m]] = k_src[k_src_row ? k_src_row[m] : m]
 *   fused_v[dst_row[m]] = v_src[v_src_row ? v_src_row[m] : m]
 * k_src: [k_src_rows, Hkv, d], v_src: [v_src_rows, Hkv, d]; either side may
 * be NULL to leave that cache untouched.  Destination rows must be unique
 * (duplicates race).
 */
kvf_status kvf_scatter_kv(const kvf_layer_desc* layer, const void* k_src,
                          const int32_t* k_src_row, int64_t k_src_rows,
                          const void* v_src, const int32_t* v_src_row,
                          int64_t v_src_rows, const int32_t* dst_row, int32_t M,
                          void* fused_k, void* fused_v, int64_t fused_rows,
                          void* stream);

/* kvf_scatter_kv_q8 - S5 into an int8-resident fused cache: the rows of
 * kvf_scatter_kv (k_src, v_src bf16 [rows, Hkv, d], either may be NULL),
 * each destination (row, kv head) encoded from its source values.
 * Destination rows must be unique (duplicates race); entries outside
 * [0, fused->rows), and sources outside their row range, are skipped. */
kvf_status kvf_scatter_kv_q8(const kvf_layer_desc* layer, const void* k_src,
                             const int32_t* k_src_row, int64_t k_src_rows,
                             const void* v_src, const int32_t* v_src_row,
                             int64_t v_src_rows, const int32_t* dst_row, int32_t M,
                             const kvf_q8_cache* fused, void* stream);

/* ---------------------------------------------------------------------------
 * kvf_sparse_q_attention - S6: causal attention of the recomputed rows over
 * the fused cache ([QCF] 2.1.3: a recomputed token reads prefix positions
 * j <= p; [KVB] 3.1 Eq. 2).  Request r owns q rows [cu_q[r], cu_q[r+1]) whose
 * positions q_pos (within the request) are ascending; for q head h:
 *   out[m, h] = sum_{j <= q_pos[m]} softmax_j(q[m,h] . K[cu_T[r]+j, h/G] *
 *               sm_scale) V[cu_T[r]+j, h/G]
 *   lse[m, h] = natural log-sum-exp of the scaled scores (lse may be NULL).
 * cu_q: HOST [n_req + 1].  q_pos[m] must be < T_r (else the row is skipped).
 */
kvf_status kvf_sparse_q_attention(const kvf_layer_desc* layer,
                                  const kvf_batch* batch, const void* q,
                                  const int32_t* q_pos, const int32_t* cu_q,
                                  const void* fused_k, const void* fused_v,
                                  float sm_scale, void* out, float* lse,
                                  void* workspace, size_t workspace_bytes,
                                  void* stream);

/* kvf_sparse_q_attention_q8 - kvf_sparse_q_attention over an int8-resident
 * fused cache (same arguments otherwise, layer->dtype KVF_BF16, q bf16).
 * Each K/V tile is decoded once per workgroup (fp32 min + code * scale,
 * rounded to fp16) on its way into on-chip memory, and the products run in
 * fp16 with fp32 accumulation: queries and probabilities are rounded to fp16
 * as well.  Every decoded value and query element must lie within the fp16
 * range (|x| <= 65504); outputs of rows that read one beyond it are
 * undefined.  The workspace is that of kvf_attention_workspace_size (the same
 * layer, batch and cu_q) and follows the same rules. */
kvf_status kvf_sparse_q_attention_q8(const kvf_layer_desc* layer,
                                     const kvf_batch* batch, const void* q,
                                     const int32_t* q_pos, const int32_t* cu_q,
                                     const kvf_q8_cache* fused, float sm_scale,
                                     void* out, float* lse, void* workspace,
                                     size_t workspace_bytes, void* stream);

/* Workspace bytes kvf_sparse_q_attention can use for the same layer, batch
 * and cu_q (HOST).  0 when the call would not use one (fp32, or a grid large
 * enough to balance by itself).  With a workspace, the row tiles of long
 * rows split their keys over several workgroups (2 to 8, more when the grid
 * has fewer row tiles) and merge (same result up to fp32 rounding order);
 * with workspace NULL the call runs unsplit.  The
 * workspace's first 4096 bytes are per-tile arrival counters that must be
 * zero before its first use (zero-fill it once when allocating it); every
 * completed call leaves them zero again, so calls of any shape may share one
 * workspace.  Calls that share a workspace must not overlap.
 * A non-NULL workspace smaller than this size gives KVF_ERR_WORKSPACE. */
size_t kvf_attention_workspace_size(const kvf_layer_desc* layer,
                                    const kvf_batch* batch,
                                    const int32_t* cu_q);

/* ---------------------------------------------------------------------------
 * kvf_kivi_encode - offline encoder of a dense bf16 per-chunk cache into the
 * KIVI form read by kvf_rerotate ([KVB] 4.5 Eq. 7), b = out->bits (8 or 4).
 * Runs ahead of serving, not on the fused-layer path.  With
 * levels = 2^b - 1, fp32 arithmetic in this order: range = max - min;
 * scale = range / levels; inv = levels / range;
 * code = round-half-even((x - min) * inv) clamped to [0, levels]; range 0
 * gives scale 0 and code 0.  Keys: statistics per (pool chunk, head,
 * channel) over the chunk's rows pool_cu[c]..pool_cu[c+1]-1 (pool_cu: device
 * [n_pool_chunks + 1]); values: per (row, head) over the channels.
 * out must point at writable arrays (the const members are written).
 */
kvf_status kvf_kivi_encode(const kvf_layer_desc* layer, const void* pool_k,
                           const void* pool_v, const int32_t* pool_cu,
                           int32_t n_pool_chunks, int64_t pool_rows,
                           int32_t max_chunk_len, const kvf_kivi* out,
                           void* stream);

/* floor(ratio_pct * n_ctx / 100) in integer arithmetic: the recompute budget
 * |P| = floor(rho N) of [QCF] 3.2.1 Eq. 11.  Returns -1 for negative input
 * or ratio_pct > 100. */
int32_t kvf_recompute_budget(int32_t n_ctx, int32_t ratio_pct);

/* ceil(len * ra_num / ra_den) in integer arithmetic: the anchor budget
 * ceil(r_a |c_i|) of [QCF] 3.3.1 Eq. 14 with r_a = ra_num / ra_den.  Returns
 * -1 for len < 0, ra_den <= 0, ra_num < 0 or ra_num > ra_den. */
int32_t kvf_anchor_budget(int32_t len, int32_t ra_num, int32_t ra_den);

const char* kvf_status_string(kvf_status status);
const char* kvf_last_error(void);
int32_t kvf_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* KVFUSE_H */
