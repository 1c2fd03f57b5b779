/*
 * dsa_oracle.c -- plain, slow CPU oracle for the attention read of
 * Mistral Large 4: DSA indexer -> top-2,048 -> sparse MLA.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  The product path
 * (the HIP library under sparse_attention_12_amd/) shares no code with it.
 *
 * Source pages (cited by title and section, never by line):
 *   [ML4-concepts]  "Mistral Large 4" concept page (liminalml.com), sections
 *                   "What to keep" / "Where to look" (MLA cache of a 512-value
 *                   latent plus a 64-value rotary key; DSA indexer with 32
 *                   small heads keeping the best 2,048), "Cache", and
 *                   "Sparse attention" (the indexer scores every earlier
 *                   position, the top 2,048 are kept, attention normalises
 *                   over those alone; 32 x 128 multiply-adds per scored
 *                   position against 64 x (512 + 64 + 512) per attended one).
 *   [ML4-summary]   "Mistral Large 4" illustrated summary (avisoori1x), the
 *                   DeepSeek Sparse Attention adoption paragraph (a
 *                   lightweight indexer picks the top 2,048 keys per query).
 *
 * Readings taken where the pages are silent or garbled (the display formula
 * of the "Sparse attention" section was lost in extraction):
 *   - indexer score  I[s] = sum_h w[h] * max(0, q_h . k_s)   (32 heads x 128);
 *     the 32 x 128 cost figure rules out a purely linear head sum, which
 *     would collapse to a single 128-wide dot product;
 *   - "earlier" positions include the query's own position;
 *   - ties in the top-k are broken by the lower position index, which makes
 *     the selected set unique;
 *   - the MLA read is in absorbed form: the 576-wide query is dotted with the
 *     576-wide cache row (512 latent + 64 rotary), the value is the 512-wide
 *     latent, the logit is scaled by tau, and the softmax runs over the
 *     selected positions only;
 *   - a layer without rotary encoding (every fourth layer, [ML4-concepts]
 *     list of changes and "Cache": such a layer keeps the 512-value latent
 *     alone) reads 512-wide rows, and its logit is the 512-wide dot product.
 *
 * All arithmetic is in IEEE double.  Inputs arrive as float (bf16 inputs are
 * widened exactly by the caller).  No blocking, fusion or reordering beyond
 * the definitions: every loop below is the sum in the formula it cites.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_HI 32   /* indexer heads                       */
#define ORC_DI 128  /* indexer head width                  */
#define ORC_H 64    /* MLA heads                           */
#define ORC_DC 512  /* latent width (also the value width) */
#define ORC_DR 64   /* rotary key width                    */
#define ORC_D 576   /* cache row: latent then rotary       */

int oracle_dims(int32_t* out6) {
  out6[0] = ORC_HI;
  out6[1] = ORC_DI;
  out6[2] = ORC_H;
  out6[3] = ORC_DC;
  out6[4] = ORC_DR;
  out6[5] = ORC_D;
  return 6;
}

/*
 * Indexer score of one query against positions 0..n-1 ([ML4-concepts],
 * "Where to look" and "Sparse attention"; reading above):
 *   out[s] = sum_{h<32} w[h] * max(0, sum_{d<128} qI[h][d] * kI[s][d]).
 * qI: [32][128], w: [32], kI: [n][128] (row s is position s), out: [n].
 * Parallel over positions for timing only; each out[s] is computed alone.
 */
void oracle_index_score(const float* qI, const float* w, const float* kI,
                        int64_t n, double* out) {
  int64_t s;
#pragma omp parallel for schedule(static)
  for (s = 0; s < n; ++s) {
    const float* ks = kI + s * ORC_DI;
    double total = 0.0;
    for (int h = 0; h < ORC_HI; ++h) {
      const float* qh = qI + h * ORC_DI;
      double dot = 0.0;
      for (int d = 0; d < ORC_DI; ++d) dot += (double)qh[d] * (double)ks[d];
      double relu = dot > 0.0 ? dot : 0.0;
      total += (double)w[h] * relu;
    }
    out[s] = total;
  }
}

typedef struct {
  double score;
  int64_t pos;
} orc_item;

/* Total order of the selection: higher score first, lower position on ties. */
static int orc_by_score_desc_pos_asc(const void* a, const void* b) {
  const orc_item* x = (const orc_item*)a;
  const orc_item* y = (const orc_item*)b;
  if (x->score > y->score) return -1;
  if (x->score < y->score) return 1;
  return (x->pos < y->pos) ? -1 : (x->pos > y->pos ? 1 : 0);
}

static int orc_int_asc(const void* a, const void* b) {
  int32_t x = *(const int32_t*)a, y = *(const int32_t*)b;
  return (x < y) ? -1 : (x > y ? 1 : 0);
}

/*
 * Top-k selection ([ML4-concepts] "Where to look": keep the best 2,048;
 * [ML4-summary] DSA paragraph).  Sorts all n candidates by (score desc,
 * position asc), keeps the first min(k, n), and writes them in ascending
 * position order to idx_out[0..m), padding idx_out[m..k) with -1.
 * Returns m, or -1 if a score is not finite or an argument is invalid.
 */
int64_t oracle_topk(const double* scores, int64_t n, int64_t k, int32_t* idx_out) {
  if (n < 0 || k < 0) return -1;
  for (int64_t s = 0; s < n; ++s)
    if (!isfinite(scores[s])) return -1;
  orc_item* items = (orc_item*)malloc((size_t)(n > 0 ? n : 1) * sizeof(orc_item));
  if (!items) return -1;
  for (int64_t s = 0; s < n; ++s) {
    items[s].score = scores[s];
    items[s].pos = s;
  }
  qsort(items, (size_t)n, sizeof(orc_item), orc_by_score_desc_pos_asc);
  int64_t m = n < k ? n : k;
  for (int64_t j = 0; j < m; ++j) idx_out[j] = (int32_t)items[j].pos;
  free(items);
  qsort(idx_out, (size_t)m, sizeof(int32_t), orc_int_asc);
  for (int64_t j = m; j < k; ++j) idx_out[j] = -1;
  return m;
}

/*
 * Sparse MLA read of one query over a selected set ([ML4-concepts] "What to
 * keep", "Where to look", "Sparse attention"; absorbed form, reading above),
 * with rotary width R = 64 (R = 0 for a layer without rotary encoding) and
 * row width W = 512 + R:
 *   l[h][j] = tau * ( sum_{d<512} q[h][d]     * kv[sel_j][d]
 *                   + sum_{d<R}   q[h][512+d] * kv[sel_j][512+d] )
 *   M_h = max_j l[h][j];  Z_h = sum_j exp(l[h][j] - M_h)
 *   o[h][e] = sum_j exp(l[h][j] - M_h) / Z_h * kv[sel_j][e]    (e < 512)
 *   lse[h] = M_h + ln Z_h
 * q: [64][W]; kv: cache rows of the sequence, row p = position p, [.][W];
 * sel: m positions (any order; entries < 0 are skipped); o: [64][512];
 * lse: [64].  With no selected position, o = 0 and lse = -inf.
 * Parallel over heads for timing only.
 */
void oracle_mla_attend(const float* q, const float* kv, const int32_t* sel, int64_t m,
                       int32_t rope, double tau, double* o, double* lse) {
  const int64_t W = ORC_DC + rope;
  int h;
#pragma omp parallel for schedule(static)
  for (h = 0; h < ORC_H; ++h) {
    const float* qh = q + (int64_t)h * W;
    double* oh = o + (int64_t)h * ORC_DC;
    double* logit = (double*)malloc((size_t)(m > 0 ? m : 1) * sizeof(double));
    for (int e = 0; e < ORC_DC; ++e) oh[e] = 0.0;
    double mx = -INFINITY;
    int64_t used = 0;
    for (int64_t j = 0; j < m; ++j) {
      if (sel[j] < 0) continue;
      const float* row = kv + (int64_t)sel[j] * W;
      double latent = 0.0, rot = 0.0;
      for (int d = 0; d < ORC_DC; ++d) latent += (double)qh[d] * (double)row[d];
      for (int d = 0; d < rope; ++d) rot += (double)qh[ORC_DC + d] * (double)row[ORC_DC + d];
      logit[j] = tau * (latent + rot);
      if (logit[j] > mx) mx = logit[j];
      ++used;
    }
    if (used == 0) {
      lse[h] = -INFINITY;
      free(logit);
      continue;
    }
    double z = 0.0;
    for (int64_t j = 0; j < m; ++j)
      if (sel[j] >= 0) z += exp(logit[j] - mx);
    for (int64_t j = 0; j < m; ++j) {
      if (sel[j] < 0) continue;
      const float* row = kv + (int64_t)sel[j] * W;
      double p = exp(logit[j] - mx) / z;
      for (int e = 0; e < ORC_DC; ++e) oh[e] += p * (double)row[e];
    }
    lse[h] = mx + log(z);
    free(logit);
  }
}

/* Threads OpenMP would use (1 when built without OpenMP). */
int oracle_max_threads(void) {
#ifdef _OPENMP
  extern int omp_get_max_threads(void);
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/* Threads for the following calls (timing only; results do not depend on it). */
void oracle_set_threads(int n) {
#ifdef _OPENMP
  extern void omp_set_num_threads(int);
  omp_set_num_threads(n > 0 ? n : 1);
#else
  (void)n;
#endif
}
