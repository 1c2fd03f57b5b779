/*
 * Host-path driver for the sanitized build (AddressSanitizer and
 * UndefinedBehaviorSanitizer) of the library's C ABI layer and of the CPU
 * oracle.  The kernel launchers are stand-ins (launch_stubs.cpp), so every
 * entry point can be called with stand-in device addresses that are never
 * dereferenced: each error path, each valid call down to its launches, the
 * size queries over small and very large shapes, the layer plan, the
 * frequencies; then the oracle's functions on tiny inputs.  Exit status 0
 * when every expectation holds (the sanitizers abort on the first report).
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "../../include/dsa_mla.h"

int stub_calls(int which);
void stub_reset(void);

/* oracle (oracle/dsa_oracle.c) */
void oracle_index_score(const float* qI, const float* w, const float* kI, int64_t n, double* out);
int64_t oracle_topk(const double* scores, int64_t n, int64_t k, int32_t* idx_out);
void oracle_mla_attend(const float* q, const float* kv, const int32_t* sel, int64_t m, int32_t rope, double tau,
                       double* o, double* lse);

static int failures;
#define EXPECT(cond)                                                          \
  do {                                                                        \
    if (!(cond)) {                                                            \
      fprintf(stderr, "%s:%d: expectation failed: %s (%s)\n", __FILE__, __LINE__, #cond, dsa_last_error()); \
      ++failures;                                                             \
    }                                                                         \
  } while (0)

/* stand-in device addresses (never dereferenced) */
#define P(x) ((void*)(uintptr_t)(x))
static const uintptr_t A = 0x100000, A4 = 0x100004, A8 = 0x100008;

static dsa_batch_t batch(int nq, int nseq, int max_len) {
  dsa_batch_t b;
  b.nq = nq;
  b.nseq = nseq;
  b.max_len = max_len;
  b.q_seq = (const int32_t*)P(A);
  b.q_pos = (const int32_t*)P(A);
  b.seq_len = (const int32_t*)P(A);
  b.seq_row0 = (const int64_t*)P(A);
  return b;
}

static void check_index_score(void) {
  dsa_batch_t b = batch(64, 64, 32768);
  EXPECT(dsa_index_score(NULL, DSA_BF16, P(A), P(A), P(A), P(A), 32768, NULL) == DSA_ERR_NULL);
  EXPECT(dsa_index_score(&b, 9, P(A), P(A), P(A), P(A), 32768, NULL) == DSA_ERR_DTYPE);
  EXPECT(dsa_index_score(&b, DSA_BF16, P(A4), P(A), P(A), P(A), 32768, NULL) == DSA_ERR_ALIGN);
  EXPECT(dsa_index_score(&b, DSA_BF16, P(A), P(A), P(A), P(A), 100, NULL) == DSA_ERR_SHAPE);
  dsa_batch_t bad = b;
  bad.seq_row0 = (const int64_t*)P(A4);
  EXPECT(dsa_index_score(&bad, DSA_BF16, P(A), P(A), P(A), P(A), 32768, NULL) == DSA_ERR_ALIGN);
  bad = b;
  bad.max_len = DSA_MAX_LEN + 1;
  EXPECT(dsa_index_score(&bad, DSA_BF16, P(A), P(A), P(A), P(A), DSA_MAX_LEN + 1, NULL) == DSA_ERR_UNSUPPORTED);
  stub_reset();
  for (int dt = 0; dt <= 2; ++dt)
    EXPECT(dsa_index_score(&b, dt, P(A), P(A), P(A), P(A4), 32768, NULL) == DSA_OK);
  dsa_batch_t pf = batch(2048, 1, 65536); /* prefill-shaped */
  EXPECT(dsa_index_score(&pf, DSA_BF16, P(A), P(A), P(A), P(A), 65536, NULL) == DSA_OK);
  dsa_batch_t many = batch(3000, 3000, 1500); /* more than the balanced kernel's queries */
  EXPECT(dsa_index_score(&many, DSA_FP8_E4M3, P(A), P(A), P(A), P(A), 1500, NULL) == DSA_OK);
  EXPECT(stub_calls(0) == 5 && stub_calls(5) == 0);
}

static void check_topk(void) {
  const int lens[] = {1, 2048, 49152, 49153, 131072, 1 << 20, DSA_MAX_LEN};
  for (size_t i = 0; i < sizeof(lens) / sizeof(lens[0]); ++i)
    for (int nq = 1; nq <= 4096; nq *= 8) {
      const size_t need = dsa_topk_workspace_size(nq, lens[i], 2048);
      dsa_batch_t b = batch(nq, nq, lens[i]);
      stub_reset();
      EXPECT(dsa_topk(&b, (const float*)P(A4), lens[i], 2048, (int32_t*)P(A4), (int32_t*)P(A4),
                      need ? P(A) : NULL, need, NULL) == DSA_OK);
      EXPECT(stub_calls(1) == 1 && stub_calls(5) == 0);
      if (need) EXPECT(dsa_topk(&b, (const float*)P(A), lens[i], 2048, (int32_t*)P(A), NULL, P(A), need - 1, NULL) ==
                       DSA_ERR_WORKSPACE);
    }
  dsa_batch_t b = batch(2, 2, 100);
  EXPECT(dsa_topk(&b, (const float*)P(A), 100, 0, (int32_t*)P(A), NULL, NULL, 0, NULL) == DSA_ERR_SHAPE);
  EXPECT(dsa_topk(&b, (const float*)P(A), 100, 2049, (int32_t*)P(A), NULL, NULL, 0, NULL) == DSA_ERR_UNSUPPORTED);
  EXPECT(dsa_topk(&b, (const float*)P(A + 2), 100, 8, (int32_t*)P(A), NULL, NULL, 0, NULL) == DSA_ERR_ALIGN);
}

static void check_mla(void) {
  for (int nq = 1; nq <= 4096; nq *= 4)
    for (int k = 1; k <= 2048; k = k * 3 + 1) {
      dsa_batch_t b = batch(nq, nq, 5000);
      for (int dt = 0; dt <= 1; ++dt)
        for (int rope = 0; rope <= 64; rope += 64) {
          const size_t need = mla_sparse_attend_workspace_size(nq, k, 1);
          stub_reset();
          EXPECT(mla_sparse_attend(&b, dt, rope, P(A), P(A), (const int32_t*)P(A4), k, 0.07f, P(A), dt,
                                   (float*)P(A4), need ? P(A) : NULL, need, NULL) == DSA_OK);
          EXPECT(stub_calls(2) == 1 && stub_calls(5) == 0);
        }
    }
  dsa_batch_t b = batch(2, 2, 100);
  EXPECT(mla_sparse_attend(&b, DSA_BF16, 32, P(A), P(A), (const int32_t*)P(A), 2048, 0.07f, P(A), 0, NULL, P(A),
                           (size_t)1 << 40, NULL) == DSA_ERR_SHAPE);
  EXPECT(mla_sparse_attend(&b, DSA_BF16, 64, P(A), P(A8), (const int32_t*)P(A), 2048, 0.07f, P(A), 0, NULL, P(A),
                           (size_t)1 << 40, NULL) == DSA_ERR_ALIGN);
}

static void check_fused(void) {
  const void* tab[DSA_MAX_LAYERS];
  void* otab[DSA_MAX_LAYERS];
  float* ltab[DSA_MAX_LAYERS];
  for (int l = 0; l < DSA_MAX_LAYERS; ++l) {
    tab[l] = P(A);
    otab[l] = P(A);
    ltab[l] = (float*)P(A4);
  }
  const int shapes[][2] = {{1, 4096}, {16, 131072}, {64, 32768}, {4, 1 << 20}, {1100, 1500}, {300, 70000}};
  for (size_t i = 0; i < sizeof(shapes) / sizeof(shapes[0]); ++i)
    for (int n_layers = 1; n_layers <= DSA_MAX_LAYERS; n_layers += 5)
      for (int idt = 0; idt <= 2; ++idt) {
        dsa_batch_t b = batch(shapes[i][0], shapes[i][0], shapes[i][1]);
        const size_t need = dsa_mla_decode_fused_workspace_size(b.nq, b.max_len, 2048, n_layers);
        const int dt = idt == 0 ? DSA_F32 : DSA_BF16;
        stub_reset();
        EXPECT(dsa_mla_decode_fused(&b, idt, P(A), (const float*)P(A), P(A), 2048, n_layers, dt, 64, tab, tab, otab,
                                    ltab, 0, 0.07f, (int32_t*)P(A4), P(A), need, NULL) == DSA_OK);
        EXPECT(stub_calls(0) == 1 && stub_calls(1) == 1 && stub_calls(2) == 1 && stub_calls(5) == 0);
        EXPECT(dsa_mla_decode_fused(&b, idt, P(A), (const float*)P(A), P(A), 2048, n_layers, dt, 64, tab, tab, otab,
                                    ltab, 0, 0.07f, NULL, P(A), need - 1, NULL) == DSA_ERR_WORKSPACE);
      }
  /* very large shapes: the size queries must not overflow */
  EXPECT(dsa_mla_decode_fused_workspace_size(1024, DSA_MAX_LEN, 2048, 16) > (size_t)1024 * DSA_MAX_LEN * 4);
  EXPECT(dsa_topk_workspace_size(255, 8 << 20, 2048) > 0);
}

static void check_layers(void) {
  dsa_layer_plan_t plan[DSA_ML4_LAYERS];
  EXPECT(dsa_ml4_layer_plan(DSA_ML4_LAYERS, plan) == DSA_OK);
  int indexers = 0;
  for (int l = 0; l < DSA_ML4_LAYERS; ++l) indexers += plan[l].runs_indexer;
  EXPECT(indexers == 44);
  const void* tab[DSA_ML4_LAYERS];
  void* otab[DSA_ML4_LAYERS];
  const float* wtab[DSA_ML4_LAYERS];
  int32_t* itab[DSA_ML4_LAYERS];
  for (int l = 0; l < DSA_ML4_LAYERS; ++l) {
    tab[l] = P(A);
    otab[l] = P(A);
    wtab[l] = (const float*)P(A);
    itab[l] = (int32_t*)P(A4);
  }
  dsa_batch_t b = batch(64, 64, 32768);
  const size_t need = dsa_mla_decode_layers_workspace_size(b.nq, b.max_len, 2048, DSA_ML4_LAYERS, plan);
  EXPECT(need > 0);
  stub_reset();
  EXPECT(dsa_mla_decode_layers(&b, DSA_ML4_LAYERS, plan, DSA_BF16, tab, wtab, tab, 2048, DSA_BF16, tab, tab, otab,
                               NULL, 0, 0.07f, itab, P(A), need, NULL) == DSA_OK);
  EXPECT(stub_calls(0) == 44 && stub_calls(1) == 44 && stub_calls(5) == 0);
  /* one MLA launch per run of layers sharing a selection and a rotary width:
     every indexer layer opens a run, and from layer 16 its two reusers join it */
  EXPECT(stub_calls(2) == 44);
  plan[10].kv_source = 11;
  EXPECT(dsa_mla_decode_layers(&b, DSA_ML4_LAYERS, plan, DSA_BF16, tab, wtab, tab, 2048, DSA_BF16, tab, tab, otab,
                               NULL, 0, 0.07f, NULL, P(A), need, NULL) == DSA_ERR_SHAPE);
}

static void check_rope(void) {
  double f[32];
  float alpha[32];
  for (int i = 0; i < 32; ++i) alpha[i] = 0.01f * (float)i;
  EXPECT(dsa_rope_frequencies(NULL, f) == DSA_OK);
  EXPECT(f[0] == 1.0 && f[31] > 0.0 && f[31] < f[16]);
  EXPECT(dsa_rope_frequencies(alpha, f) == DSA_OK);
  EXPECT(dsa_rope_frequencies(NULL, NULL) == DSA_ERR_NULL);
  dsa_batch_t b = batch(300, 1, 5000);
  stub_reset();
  EXPECT(dsa_rope_append(&b, DSA_BF16, 64, (const double*)P(A), (const float*)P(A), (const float*)P(A), P(A), P(A),
                         (const float*)P(A), (const float*)P(A), NULL) == DSA_OK);
  EXPECT(dsa_rope_append(&b, DSA_F32, 0, NULL, (const float*)P(A), NULL, P(A), NULL, NULL, NULL, NULL) == DSA_OK);
  EXPECT(stub_calls(3) == 2 && stub_calls(5) == 0);
  EXPECT(dsa_rope_append(&b, DSA_BF16, 64, (const double*)P(A8), (const float*)P(A), (const float*)P(A), P(A), NULL,
                         NULL, NULL, NULL) == DSA_ERR_ALIGN);
}

static void check_strings(void) {
  for (int st = -8; st <= 1; ++st) EXPECT(dsa_status_string(st) != NULL && strlen(dsa_status_string(st)) > 0);
  EXPECT(dsa_abi_version() == DSA_ABI_VERSION);
}

static void check_oracle(void) {
  enum { n = 40, HI = 32, DI = 128, H = 64, W = 576 };
  float* qI = calloc(HI * DI, sizeof(float));
  float* w = calloc(HI, sizeof(float));
  float* kI = calloc(n * DI, sizeof(float));
  double* sc = calloc(n, sizeof(double));
  int32_t idx[64];
  for (int i = 0; i < HI * DI; ++i) qI[i] = (float)((i * 7) % 7 - 3);
  for (int i = 0; i < HI; ++i) w[i] = (float)(1 + i % 4);
  for (int i = 0; i < n * DI; ++i) kI[i] = (float)((i * 5) % 7 - 3);
  oracle_index_score(qI, w, kI, n, sc);
  oracle_index_score(qI, w, kI, 0, sc);
  EXPECT(oracle_topk(sc, n, 8, idx) == 8);
  EXPECT(oracle_topk(sc, n, 64, idx) == n && idx[n] == -1 && idx[63] == -1);
  EXPECT(oracle_topk(sc, 0, 4, idx) == 0 && idx[0] == -1);
  for (int i = 1; i < 8; ++i) EXPECT(oracle_topk(sc, n, 8, idx) == 8 && idx[i] > idx[i - 1]);
  sc[3] = INFINITY;
  EXPECT(oracle_topk(sc, n, 8, idx) == -1);
  float* q = calloc(H * W, sizeof(float));
  float* kv = calloc(n * W, sizeof(float));
  double* o = calloc(H * 512, sizeof(double));
  double lse[H];
  for (int i = 0; i < H * W; ++i) q[i] = 0.01f * (float)(i % 13);
  for (int i = 0; i < n * W; ++i) kv[i] = 0.02f * (float)(i % 17) - 0.1f;
  const int32_t sel[6] = {0, 5, -1, 39, 12, 7};
  oracle_mla_attend(q, kv, sel, 6, 64, 0.07, o, lse);
  EXPECT(isfinite(lse[0]) && isfinite(o[0]));
  oracle_mla_attend(q, kv, sel, 6, 0, 0.07, o, lse);
  const int32_t none[2] = {-1, -1};
  oracle_mla_attend(q, kv, none, 2, 64, 0.07, o, lse);
  EXPECT(isinf(lse[0]) && lse[0] < 0 && o[5] == 0.0);
  oracle_mla_attend(q, kv, none, 0, 64, 0.07, o, lse);
  free(qI);
  free(w);
  free(kI);
  free(sc);
  free(q);
  free(kv);
  free(o);
}

int main(void) {
  check_index_score();
  check_topk();
  check_mla();
  check_fused();
  check_layers();
  check_rope();
  check_strings();
  check_oracle();
  if (stub_calls(5) != 0) ++failures;
  if (failures) {
    fprintf(stderr, "%d expectation(s) failed\n", failures);
    return 1;
  }
  printf("host paths and oracle clean under the sanitizers\n");
  return 0;
}
