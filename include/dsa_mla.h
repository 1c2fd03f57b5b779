/*
 * dsa_mla.h -- C ABI of the MI355X (gfx950) library for one attention read
 * of Mistral Large 4: DeepSeek-Sparse-Attention indexer -> top-2,048
 * selection -> 64-head Multi-head Latent Attention over the selected
 * positions only.
 *
 * The operations are defined on the "Mistral Large 4" concept page
 * (liminalml.com/concepts/mistral-large-4):
 *   - "What to keep": each cached position holds a 512-value latent plus a
 *     64-value rotary key shared by all 64 heads, 576 values per row;
 *   - "Where to look": an indexer with 32 small heads rates every earlier
 *     position and keeps the best 2,048; all 64 heads attend to those only;
 *     the change list adds that a layer may reuse the selection of the most
 *     recent layer that ran its indexer;
 *   - "Sparse attention": the score of every earlier position, the top
 *     2,048, and a softmax normalised over the kept positions alone; its cost
 *     figures (32 x 128 multiply-adds per scored position, 64 x (512 + 64 +
 *     512) per attended one) fix the shapes below.
 *   - the change list: every fourth layer has no rotary encoding (its rows
 *     hold the 512-value latent alone), from layer 39 on those layers read
 *     layer 35's latent, and 28 layers reuse the selection of the most
 *     recent layer that ran its indexer ("Cache" counts the result).
 * The page's display formula for the score was lost; this library computes
 *   I[q][s] = sum_{h<32} w[q][h] * max(0, sum_{d<128} qI[q][h][d] * kI[s][d])
 * and the absorbed-form MLA read, with row width W = 512 + rope_dim
 * (rope_dim = 64, or 0 in a layer without rotary encoding):
 *   l[h][j] = scale * (q[h][0:W] . kv[S_j][0:W]),  p = softmax_j(l) over S,
 *   o[h][:] = sum_j p[h][j] * kv[S_j][0:512],  lse[h] = log sum_j exp(l[h][j]).
 *
 * Conventions shared by every entry point
 *   - Every array argument is a DEVICE pointer owned by the caller, except
 *     the dsa_batch_t struct itself, the layer plans and the per-layer
 *     pointer tables of the multi-layer calls, which are HOST memory read
 *     during the call only.
 *   - The library never allocates, frees or synchronises.  Work is enqueued
 *     on `stream` (a hipStream_t; NULL = the default stream) and the call
 *     returns at once; results are ready when the stream reaches them.
 *   - Return value: DSA_OK (0) or a negative dsa_status_t.  Arguments are
 *     validated on the host before anything is enqueued; a validation error
 *     enqueues nothing.  A failed launch returns DSA_ERR_HIP.  The message of
 *     the last error on the calling thread is in dsa_last_error().
 *   - Dtypes: DSA_BF16 (bf16 storage, fp32 accumulation) or DSA_F32; the
 *     indexer's query and keys may also be DSA_FP8_E4M3.  Indexer weights,
 *     scores and log-sum-exp are always float32.
 *   - Alignment: the arrays read or written as 16-byte vectors -- q_idx,
 *     w_idx, k_idx, q, kv, out, the workspace ws, and every array of
 *     dsa_rope_append -- must be 16-byte aligned; every other array needs
 *     only its element's alignment: 4 bytes for scores, idx, count, lse and
 *     the int32 batch arrays, 8 bytes for seq_row0.  A misaligned pointer is
 *     DSA_ERR_ALIGN.  Row strides are fixed: indexer keys 128 elements, cache
 *     rows 512 + rope_dim (512 latent, then the rotary key if any); the
 *     score row stride ld is free (rows need not start on 16 bytes).
 *   - Entries are re-entrant; calls that share a workspace race unless they
 *     are ordered on one stream.
 */
#ifndef DSA_MLA_H
#define DSA_MLA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define DSA_ABI_VERSION 4

#define DSA_INDEX_HEADS 32  /* indexer heads                          */
#define DSA_INDEX_DIM 128   /* indexer head width                     */
#define DSA_MLA_HEADS 64    /* attention heads                        */
#define DSA_LATENT 512      /* latent width = value width             */
#define DSA_ROPE 64         /* rotary key width                       */
#define DSA_ROW 576         /* cache row = latent + rotary key        */
#define DSA_TOPK_MAX 2048   /* largest supported k (the pages' 2,048) */
#define DSA_MAX_LAYERS 16   /* largest n_layers of the fused call     */
#define DSA_ML4_LAYERS 72   /* decoder layers of Mistral Large 4      */
#define DSA_MAX_LEN 3728270 /* longest sequence: its 1,152-byte bf16
                               cache rows are addressed with 32 bits   */

typedef enum {
  DSA_OK = 0,
  DSA_ERR_NULL = -1,        /* a required pointer is NULL                         */
  DSA_ERR_SHAPE = -2,       /* a size is out of range                             */
  DSA_ERR_DTYPE = -3,       /* unknown dtype                                      */
  DSA_ERR_ALIGN = -4,       /* a pointer lacks the alignment its array needs      */
  DSA_ERR_WORKSPACE = -5,   /* workspace NULL or smaller than the size query says */
  DSA_ERR_UNSUPPORTED = -6, /* valid but not supported (k > 2,048, too many layers) */
  DSA_ERR_HIP = -7          /* the HIP runtime reported an error                  */
} dsa_status_t;

/*
 * Element types.  DSA_FP8_E4M3 is for the indexer's inputs only (q_idx and
 * k_idx; w_idx stays float32): the concept page's 1M-token serving
 * scenario keeps the indexer keys in FP8.  It is the OCP 8-bit E4M3 encoding (sign,
 * 4 exponent bits with bias 7, 3 mantissa bits; 0x7F/0xFF are NaN, no
 * infinities, largest finite 448) with no scale factor: the caller stores
 * values already scaled.  Products are exact in float32 and summed in float32.
 */
typedef enum { DSA_F32 = 0, DSA_BF16 = 1, DSA_FP8_E4M3 = 2 } dsa_dtype_t;

/*
 * A batch of queries over one or more sequences.
 *   nq, nseq, max_len : host integers.  nq >= 0 (0 is a no-op), nseq >= 1,
 *                       1 <= max_len <= DSA_MAX_LEN bounds every sequence
 *                       length and sizes the launch grids (larger:
 *                       DSA_ERR_UNSUPPORTED).
 *   q_seq  [nq]   (device) sequence of each query, in [0, nseq).
 *   q_pos  [nq]   (device) absolute position of each query.
 *   seq_len[nseq] (device) cached positions of each sequence, <= max_len.
 *   seq_row0[nseq](device) first row of the sequence in every cache array
 *                  (indexer keys and each layer's cache rows), so sequences
 *                  may be packed, padded or ragged.
 * The candidates of query q are positions s in [0, n_cand(q)) with
 *   n_cand(q) = min(q_pos[q] + 1, seq_len[q_seq[q]], max_len)
 * (its own position and every earlier one; "Sparse attention" section).
 * Decode is nq = nseq with q_pos = seq_len - 1; a prefill chunk is many
 * queries of a sequence at increasing positions (causal), and a prefill
 * batch may hold chunks of several sequences.
 * Out-of-range device values are clamped so that no access leaves
 * [seq_row0, seq_row0 + n_cand); the results are then undefined.
 */
typedef struct dsa_batch {
  int32_t nq;
  int32_t nseq;
  int32_t max_len;
  const int32_t* q_seq;
  const int32_t* q_pos;
  const int32_t* seq_len;
  const int64_t* seq_row0;
} dsa_batch_t;

/* DSA_ABI_VERSION of the built library. */
int32_t dsa_abi_version(void);
/* Static text for a status code. */
const char* dsa_status_string(int32_t status);
/* Detail of the last failing call on this thread ("" if none). */
const char* dsa_last_error(void);

/*
 * Checks of a debug build (for callers chasing a wrong result, not a
 * contract of the method).  A library built with -DDSA_DEBUG checks, inside
 * its kernels, what the release build only guards or assumes, and records
 * each failed check as a bit instead of trapping:
 *   DSA_DEBUG_IDX_RANGE     an MLA selection entry outside [-1, n_cand)
 *                           (skipped by both builds, flagged by this one)
 *   DSA_DEBUG_TOPK_SLOT     a top-k output or candidate slot past its bound
 *   DSA_DEBUG_LIST          the split top-k's chunk lists disagree with its
 *                           histogram
 *   DSA_DEBUG_SCORE_COL     an indexer score column at or past ld
 *   DSA_DEBUG_HIST_RECOUNT  a workspace's precounted top-k histogram failed
 *                           its check and was recounted (expected on a
 *                           workspace's first use, not after)
 *   DSA_DEBUG_GATHER_ROW    an MLA gather row below -1
 * dsa_debug_flags waits for the device (hipDeviceSynchronize), stores the
 * union of the bits set since the last reset in *flags and, with reset != 0,
 * clears them.  flags: host pointer.  Release builds return
 * DSA_ERR_UNSUPPORTED and leave *flags untouched; a NULL flags is
 * DSA_ERR_NULL; a HIP failure is DSA_ERR_HIP.
 */
#define DSA_DEBUG_IDX_RANGE 1u
#define DSA_DEBUG_TOPK_SLOT 2u
#define DSA_DEBUG_LIST 4u
#define DSA_DEBUG_SCORE_COL 8u
#define DSA_DEBUG_HIST_RECOUNT 16u
#define DSA_DEBUG_GATHER_ROW 32u
int32_t dsa_debug_flags(uint32_t* flags, int32_t reset);

/*
 * Indexer scores ("Where to look" / "Sparse attention"; formula above).
 *   dtype  DSA_F32, DSA_BF16 or DSA_FP8_E4M3 (q_idx and k_idx)
 *   q_idx  [nq][32][128] dtype      w_idx [nq][32] float32
 *   k_idx  [rows][128]   dtype      (row seq_row0[s] + p is position p)
 *   scores [nq][ld]      float32    column s < n_cand(q) receives I[q][s];
 *                                   columns >= n_cand(q) are left untouched.
 *   ld >= max_len.
 * Decode batches stream the keys once per query; batches with many queries
 * per sequence (prefill; on average at least 32) run as a blocked matrix
 * product that shares each key tile across the queries of a 32-query block
 * that belong to its sequence, so a sequence's queries are best contiguous.
 */
int32_t dsa_index_score(const dsa_batch_t* batch, int32_t dtype, const void* q_idx,
                        const float* w_idx, const void* k_idx, float* scores, int64_t ld,
                        void* stream);

/*
 * Top-k selection ("Where to look": keep the best 2,048).  For each query,
 * S_q = the first min(k, n_cand(q)) positions under the total order
 * (score descending, position ascending); ties therefore go to the lower
 * position and S_q is unique.  Score -0.0 equals +0.0; NaN is undefined.
 *   scores [nq][ld] float32 (columns < n_cand(q) are read)
 *   idx    [nq][k]  int32   S_q in ascending position order, then -1 padding
 *   count  [nq]     int32   |S_q| (may be NULL)
 *   1 <= k <= 2,048.  ws: dsa_topk_workspace_size(nq, max_len, k) bytes
 *   (may be 0, then ws may be NULL).
 */
size_t dsa_topk_workspace_size(int32_t nq, int32_t max_len, int32_t k);
int32_t dsa_topk(const dsa_batch_t* batch, const float* scores, int64_t ld, int32_t k,
                 int32_t* idx, int32_t* count, void* ws, size_t ws_bytes, void* stream);

/*
 * Sparse MLA read of one layer ("What to keep", "Sparse attention").
 *   dtype, out_dtype  DSA_F32 or DSA_BF16
 *   rope_dim   DSA_ROPE (64), or 0 for a layer without rotary encoding;
 *              W = 512 + rope_dim (other values: DSA_ERR_SHAPE)
 *   q   [nq][64][W]   dtype    absorbed query: 512 latent-space (+ 64 rotary)
 *   kv  [rows][W]     dtype    cache rows (512 latent (+ 64 rotary key))
 *   idx [nq][k]       int32    selected positions; entries outside
 *                              [0, n_cand(q)) (e.g. the -1 padding) are skipped
 *   scale                      logit scale (the harness uses 1/sqrt(192))
 *   out [nq][64][512] out_dtype  softmax over the selected entries only
 *   lse [nq][64]      float32  natural log-sum-exp of the scaled logits
 *                              (may be NULL); a query with no valid entry
 *                              gets out = 0 and lse = -inf.
 *   1 <= k <= 2,048.  ws: mla_sparse_attend_workspace_size(nq, k, 1) bytes.
 */
size_t mla_sparse_attend_workspace_size(int32_t nq, int32_t k, int32_t n_layers);
int32_t mla_sparse_attend(const dsa_batch_t* batch, int32_t dtype, int32_t rope_dim, const void* q, const void* kv,
                          const int32_t* idx, int32_t k, float scale, void* out,
                          int32_t out_dtype, float* lse, void* ws, size_t ws_bytes,
                          void* stream);

/*
 * Fused decode read with selection sharing (change list on the concept
 * page: 28 layers reuse the selection of the most recent layer that ran its
 * indexer).  Runs the indexer and the top-k once, then the sparse MLA read
 * of n_layers layers, each with its own query and cache, over that one
 * selection.  Arguments as in the three calls above; index_dtype is the
 * indexer's dtype (q_idx, k_idx), dtype and rope_dim those of every layer's
 * query and cache rows.  Per-layer arrays come as HOST tables of n_layers
 * device pointers (two layers may name the same cache):
 *   q_l[l]   [nq][64][W] dtype      kv_l[l] [rows][W] dtype
 *   out_l[l] [nq][64][512] out_dtype  lse_l[l] [nq][64] float32 (lse_l or
 *   any entry may be NULL)
 *   idx_out  [nq][k] int32 (may be NULL): the shared selection.
 *   1 <= n_layers <= 16.  ws: dsa_mla_decode_fused_workspace_size(...) bytes.
 */
size_t dsa_mla_decode_fused_workspace_size(int32_t nq, int32_t max_len, int32_t k,
                                           int32_t n_layers);
int32_t dsa_mla_decode_fused(const dsa_batch_t* batch, int32_t index_dtype, const void* q_idx,
                             const float* w_idx, const void* k_idx, int32_t k, int32_t n_layers,
                             int32_t dtype, int32_t rope_dim, const void* const* q_l,
                             const void* const* kv_l, void* const* out_l, float* const* lse_l,
                             int32_t out_dtype, float scale, int32_t* idx_out, void* ws,
                             size_t ws_bytes, void* stream);

/*
 * Allocation-free fused decode read, for callers that cannot allocate device
 * memory or pass a workspace (code under graph capture, tight serving loops,
 * harnesses that forbid allocation).  Same arguments, results and errors as
 * dsa_mla_decode_fused without ws and ws_bytes: its scratch is a library-
 * owned array of DSA_NOALLOC_SCRATCH_BYTES (128 MiB) in device memory, one
 * per GPU the library runs on, held until the process ends.  The first call
 * on a device is its set-up: it looks the array's address up, and the HIP
 * runtime materialises the array on that device then; later calls allocate
 * and free nothing.  The call uses the array of the calling thread's current
 * device, which must be the device of `stream`.  A batch whose dsa_mla_decode_fused_workspace_size exceeds
 * DSA_NOALLOC_SCRATCH_BYTES is rejected with DSA_ERR_WORKSPACE before
 * anything is enqueued.  The array keeps the last call's contents and every
 * call clears what it relies on; calls that overlap on one GPU (different
 * streams or threads without ordering) share the array and race.
 */
#define DSA_NOALLOC_SCRATCH_BYTES (128u << 20)
int32_t dsa_mla_decode_fused_noalloc(const dsa_batch_t* batch, int32_t index_dtype, const void* q_idx,
                                     const float* w_idx, const void* k_idx, int32_t k, int32_t n_layers,
                                     int32_t dtype, int32_t rope_dim, const void* const* q_l,
                                     const void* const* kv_l, void* const* out_l, float* const* lse_l,
                                     int32_t out_dtype, float scale, int32_t* idx_out, void* stream);

/*
 * Layer schedule (concept page, change list and layer map).  For each layer:
 *   runs_indexer  1: the layer scores and selects with its own indexer;
 *                 0: it reuses the selection of the most recent layer that
 *                 ran its indexer (layer 0 must run one);
 *   rope_dim      DSA_ROPE, or 0 for a layer without rotary encoding;
 *   kv_source     the layer whose cache it reads: itself, or an earlier
 *                 layer that owns its cache and has the same rope_dim
 *                 (a layer never reads a cache built with another
 *                 positional scheme).
 * dsa_ml4_layer_plan fills plan[0 .. n_layers) with Mistral Large 4's
 * schedule (1 <= n_layers <= DSA_ML4_LAYERS; fewer layers take the first
 * ones): no rotary encoding in layers l with (l + 1) % 4 == 0; from layer 39
 * those layers read layer 35's cache; from layer 16, in every group of four
 * layers the middle two reuse the selection of the group's first layer
 * (this reading of the pages gives the 44 indexer layers, 28 reusing layers
 * and 35,712 cached values per position that the concept page prints).
 * plan is HOST memory.
 */
typedef struct dsa_layer_plan {
  int32_t runs_indexer;
  int32_t rope_dim;
  int32_t kv_source;
} dsa_layer_plan_t;

int32_t dsa_ml4_layer_plan(int32_t n_layers, dsa_layer_plan_t* plan);

/*
 * Decode read over a stack of layers under a schedule: for each layer in
 * order, run the indexer and the top-k if the plan says so, then the sparse
 * MLA read over the current selection, reading the cache of the layer's
 * kv_source.  Consecutive layers that share a selection and a rope_dim run
 * as one MLA launch (up to DSA_MAX_LAYERS layers).  HOST tables of n_layers
 * device pointers:
 *   q_idx_l[l] [nq][32][128] index_dtype, w_idx_l[l] [nq][32] float32,
 *   k_idx_l[l] [rows][128] index_dtype    read for indexer layers only
 *                                          (other entries may be NULL);
 *   q_l[l]     [nq][64][W_l] dtype         W_l = 512 + plan[l].rope_dim;
 *   kv_l[l]    [rows][W_l] dtype           read for layers that own their
 *                                          cache (kv_source == l); layer l
 *                                          reads kv_l[plan[l].kv_source];
 *   out_l[l]   [nq][64][512] out_dtype;   lse_l (or an entry) may be NULL;
 *   idx_l      may be NULL; idx_l[l] (may be NULL) [nq][k] int32 receives
 *              the selection made at indexer layer l.
 *   1 <= n_layers <= DSA_ML4_LAYERS.
 *   ws: dsa_mla_decode_layers_workspace_size(nq, max_len, k, n_layers, plan).
 * An invalid plan (first layer not an indexer layer, rope_dim not 0 or 64,
 * kv_source after the layer, not owning its cache or with another rope_dim)
 * is DSA_ERR_SHAPE; the size query then returns 0.
 */
size_t dsa_mla_decode_layers_workspace_size(int32_t nq, int32_t max_len, int32_t k, int32_t n_layers,
                                            const dsa_layer_plan_t* plan);
int32_t dsa_mla_decode_layers(const dsa_batch_t* batch, int32_t n_layers, const dsa_layer_plan_t* plan,
                              int32_t index_dtype, const void* const* q_idx_l,
                              const float* const* w_idx_l, const void* const* k_idx_l, int32_t k,
                              int32_t dtype, const void* const* q_l, const void* const* kv_l,
                              void* const* out_l, float* const* lse_l, int32_t out_dtype, float scale,
                              int32_t* const* idx_l, void* ws, size_t ws_bytes, void* stream);

/*
 * The step just upstream of the read (concept page, "Positions" and "Query
 * scaling"; the YaRN wavelength function of its example).
 *
 * dsa_rope_frequencies: HOST.  freq[i] (radians per position, i < 32) for
 * pair i of the 64-value rotary part: omega_i = 10000^(-2i/64); YaRN with
 * original window 512 and factor 2,048 keeps the pairs that complete at
 * least 32 turns within the window, divides by 2,048 those that complete
 * less than one, and blends linearly in the pair index in between (from the
 * rounded-down index of 32 turns to the rounded-up index of one turn);
 * LeRoPE then multiplies frequency i by e^{alpha[i]} (alpha: HOST [32], or
 * NULL for zeros).  Computed in double precision.
 *
 * dsa_rope_append: for each query q of the batch (one new token at 0-based
 * position t = q_pos[q] of sequence q_seq[q]; t must be < seq_len, else the
 * token is skipped), with W = 512 + rope_dim:
 *   kv[seq_row0 + t][0:512]  = latent[q]                        (rounded to dtype)
 *   kv[seq_row0 + t][512:W]  = rope_key[q] rotated by t          (rope_dim = 64)
 *   q_attn[q][h][:]          = m_h(t) * q_attn[q][h][:], then its values
 *                              [512, W) rotated by t             (in place; may be NULL)
 * where pair i = values (2i, 2i+1) turns by the angle t * freq[i] (formed in
 * double precision), and m_h(t) = ssmax_s[h] * ln(t + 1) + ssmax_b[h] when
 * both per-head arrays are given, else 1 (the page's query-scaling formula
 * was lost; this affine function of the log of the number of visible
 * positions is the reading taken).
 *   dtype      DSA_F32 or DSA_BF16 (kv and q_attn)
 *   rope_dim   DSA_ROPE, or 0 (a layer without rotary encoding: only the
 *              latent is written and the query only scaled; freq and
 *              rope_key may be NULL)
 *   freq       [32] double (device)      latent [nq][512] float32
 *   rope_key   [nq][64] float32          kv [rows][W] dtype
 *   q_attn     [nq][64][W] dtype or NULL ssmax_s, ssmax_b [64] float32, both or neither
 */
int32_t dsa_rope_frequencies(const float* alpha, double* freq);
int32_t dsa_rope_append(const dsa_batch_t* batch, int32_t dtype, int32_t rope_dim, const double* freq,
                        const float* latent, const float* rope_key, void* kv, void* q_attn,
                        const float* ssmax_s, const float* ssmax_b, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* DSA_MLA_H */
