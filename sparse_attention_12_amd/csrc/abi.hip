// C ABI of the library (declared in include/dsa_mla.h): host-side argument
// validation, workspace accounting and kernel dispatch.  Nothing here
// allocates, frees or synchronises (except the debug build's
// dsa_debug_flags, which waits for the device); every launch goes to the
// caller's stream.
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include "../../include/dsa_mla.h"
#include "abi_internal.h"
#include "dsa_common.h"
#include "kernels.h"

namespace {

thread_local char g_err[512] = "";

int vfail(int status, const char* fmt, va_list ap) {
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  return status;
}

int fail(int status, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vfail(status, fmt, ap);
  va_end(ap);
  return status;
}

int hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return DSA_OK;
  return fail(DSA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }
bool aligned16(const void* p) { return aligned(p, 16); }

// A required array read or written as 16-byte vectors.
#define REQUIRE_PTR(p)                                        \
  do {                                                        \
    if ((p) == nullptr) return fail(DSA_ERR_NULL, "%s is NULL", #p); \
    if (!aligned16(p)) return fail(DSA_ERR_ALIGN, "%s is not 16-byte aligned", #p); \
  } while (0)

// A required array of 4-byte elements (int32 or float32), accessed one
// element at a time.
#define REQUIRE_PTR4(p)                                       \
  do {                                                        \
    if ((p) == nullptr) return fail(DSA_ERR_NULL, "%s is NULL", #p); \
    if (!aligned((p), 4)) return fail(DSA_ERR_ALIGN, "%s is not 4-byte aligned", #p); \
  } while (0)

// An optional array (NULL allowed) of 4-byte elements.
#define OPTIONAL_PTR4(p)                                      \
  do {                                                        \
    if ((p) != nullptr && !aligned((p), 4)) return fail(DSA_ERR_ALIGN, "%s is not 4-byte aligned", #p); \
  } while (0)

int check_batch(const dsa_batch_t* b, dsa::BatchDev* out) {
  if (b == nullptr) return fail(DSA_ERR_NULL, "batch is NULL");
  if (b->nq < 0) return fail(DSA_ERR_SHAPE, "nq = %d < 0", b->nq);
  if (b->nseq < 1) return fail(DSA_ERR_SHAPE, "nseq = %d < 1", b->nseq);
  if (b->max_len < 1) return fail(DSA_ERR_SHAPE, "max_len = %d < 1", b->max_len);
  if (b->max_len > DSA_MAX_LEN)
    return fail(DSA_ERR_UNSUPPORTED, "max_len = %d > %d", b->max_len, DSA_MAX_LEN);
  if (b->nq > 0) {
    if (!b->q_seq || !b->q_pos || !b->seq_len || !b->seq_row0)
      return fail(DSA_ERR_NULL, "a batch index array is NULL");
    if (!aligned(b->q_seq, 4) || !aligned(b->q_pos, 4) || !aligned(b->seq_len, 4))
      return fail(DSA_ERR_ALIGN, "a batch int32 array is not 4-byte aligned");
    if (!aligned(b->seq_row0, 8)) return fail(DSA_ERR_ALIGN, "batch seq_row0 is not 8-byte aligned");
  }
  out->nq = b->nq;
  out->nseq = b->nseq;
  out->max_len = b->max_len;
  out->q_seq = b->q_seq;
  out->q_pos = b->q_pos;
  out->seq_len = b->seq_len;
  out->seq_row0 = b->seq_row0;
  return DSA_OK;
}

int check_dtype(int32_t dt, const char* what) {
  if (dt != DSA_F32 && dt != DSA_BF16) return fail(DSA_ERR_DTYPE, "%s = %d is not DSA_F32 or DSA_BF16", what, dt);
  return DSA_OK;
}

// The indexer also takes FP8 E4M3 inputs.
int check_index_dtype(int32_t dt, const char* what) {
  if (dt != DSA_F32 && dt != DSA_BF16 && dt != DSA_FP8_E4M3)
    return fail(DSA_ERR_DTYPE, "%s = %d is not DSA_F32, DSA_BF16 or DSA_FP8_E4M3", what, dt);
  return DSA_OK;
}

int check_rope(int32_t rope_dim) {
  if (rope_dim != 0 && rope_dim != DSA_ROPE)
    return fail(DSA_ERR_SHAPE, "rope_dim = %d is neither 0 nor %d", rope_dim, DSA_ROPE);
  return DSA_OK;
}

int check_k(int32_t k) {
  if (k < 1) return fail(DSA_ERR_SHAPE, "k = %d < 1", k);
  if (k > DSA_TOPK_MAX) return fail(DSA_ERR_UNSUPPORTED, "k = %d > %d", k, DSA_TOPK_MAX);
  return DSA_OK;
}

hipStream_t as_stream(void* s) { return (hipStream_t)s; }

}  // namespace

namespace dsa {
int abi_fail(int status, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vfail(status, fmt, ap);
  va_end(ap);
  return status;
}
int abi_hip_status(hipError_t e, const char* what) { return hip_status(e, what); }
}  // namespace dsa

extern "C" {

int32_t dsa_abi_version(void) { return DSA_ABI_VERSION; }

int32_t dsa_debug_flags(uint32_t* flags, int32_t reset) {
  if (flags == nullptr) return fail(DSA_ERR_NULL, "flags is NULL");
#ifdef DSA_DEBUG
  static_assert(DSA_DEBUG_IDX_RANGE == dsa::DBG_IDX_RANGE && DSA_DEBUG_TOPK_SLOT == dsa::DBG_TOPK_SLOT &&
                    DSA_DEBUG_LIST == dsa::DBG_LIST && DSA_DEBUG_SCORE_COL == dsa::DBG_SCORE_COL &&
                    DSA_DEBUG_HIST_RECOUNT == dsa::DBG_HIST_RECOUNT && DSA_DEBUG_GATHER_ROW == dsa::DBG_GATHER_ROW,
                "header bits match the kernels' bits");
  int st;
  if ((st = hip_status(hipDeviceSynchronize(), "device synchronize"))) return st;
  const uint32_t parts[3] = {dsa::debug_flags_indexer(reset != 0), dsa::debug_flags_topk(reset != 0),
                             dsa::debug_flags_mla(reset != 0)};
  uint32_t v = 0;
  for (uint32_t x : parts) {
    if (x == 0xffffffffu) return fail(DSA_ERR_HIP, "reading the debug flags failed");
    v |= x;
  }
  *flags = v;
  return DSA_OK;
#else
  (void)reset;
  return fail(DSA_ERR_UNSUPPORTED, "a release build has no debug checks (build with DSA_DEBUG)");
#endif
}

const char* dsa_status_string(int32_t st) {
  switch (st) {
    case DSA_OK: return "DSA_OK";
    case DSA_ERR_NULL: return "DSA_ERR_NULL: a required pointer is NULL";
    case DSA_ERR_SHAPE: return "DSA_ERR_SHAPE: a size is out of range";
    case DSA_ERR_DTYPE: return "DSA_ERR_DTYPE: unknown dtype";
    case DSA_ERR_ALIGN: return "DSA_ERR_ALIGN: a pointer lacks the alignment its array needs";
    case DSA_ERR_WORKSPACE: return "DSA_ERR_WORKSPACE: workspace missing or too small";
    case DSA_ERR_UNSUPPORTED: return "DSA_ERR_UNSUPPORTED: valid but unsupported arguments";
    case DSA_ERR_HIP: return "DSA_ERR_HIP: the HIP runtime reported an error";
    default: return "unknown status";
  }
}

const char* dsa_last_error(void) { return g_err; }

int32_t dsa_index_score(const dsa_batch_t* batch, int32_t dtype, const void* q_idx, const float* w_idx,
                        const void* k_idx, float* scores, int64_t ld, void* stream) {
  dsa::BatchDev b;
  int st = check_batch(batch, &b);
  if (st) return st;
  if ((st = check_index_dtype(dtype, "dtype"))) return st;
  if (b.nq == 0) return DSA_OK;
  REQUIRE_PTR(q_idx);
  REQUIRE_PTR(w_idx);
  REQUIRE_PTR(k_idx);
  REQUIRE_PTR4(scores);
  if (ld < b.max_len) return fail(DSA_ERR_SHAPE, "ld = %lld < max_len = %d", (long long)ld, b.max_len);
  return hip_status(dsa::launch_index_score(b, dtype, q_idx, w_idx, k_idx, scores, ld, as_stream(stream)),
                    "dsa_index_score launch");
}

size_t dsa_topk_workspace_size(int32_t nq, int32_t max_len, int32_t k) {
  if (nq <= 0 || max_len <= 0 || k <= 0) return 0;
  return dsa::topk_workspace_bytes(nq, max_len, k);
}


int32_t dsa_topk(const dsa_batch_t* batch, const float* scores, int64_t ld, int32_t k, int32_t* idx,
                 int32_t* count, void* ws, size_t ws_bytes, void* stream) {
  dsa::BatchDev b;
  int st = check_batch(batch, &b);
  if (st) return st;
  if ((st = check_k(k))) return st;
  if (b.nq == 0) return DSA_OK;
  REQUIRE_PTR4(scores);
  REQUIRE_PTR4(idx);
  OPTIONAL_PTR4(count);
  if (ld < b.max_len) return fail(DSA_ERR_SHAPE, "ld = %lld < max_len = %d", (long long)ld, b.max_len);
  const size_t need = dsa::topk_workspace_bytes(b.nq, b.max_len, k);
  if (need > 0 && (ws == nullptr || ws_bytes < need))
    return fail(DSA_ERR_WORKSPACE, "top-k workspace: %zu bytes given, %zu needed", ws_bytes, need);
  if (need > 0 && !aligned16(ws)) return fail(DSA_ERR_ALIGN, "ws is not 16-byte aligned");
  return hip_status(dsa::launch_topk(b, scores, ld, k, idx, count, ws, ws_bytes, as_stream(stream)),
                    "dsa_topk launch");
}

size_t mla_sparse_attend_workspace_size(int32_t nq, int32_t k, int32_t n_layers) {
  if (nq <= 0 || k <= 0 || n_layers <= 0) return 0;
  // sized for the larger of the two dtypes' split plans
  size_t a = dsa::mla_workspace_bytes(0, nq, k, n_layers);
  size_t c = dsa::mla_workspace_bytes(1, nq, k, n_layers);
  return a > c ? a : c;
}

static int check_mla_layer(const void* q, const void* kv, const void* out) {
  REQUIRE_PTR(q);
  REQUIRE_PTR(kv);
  REQUIRE_PTR(out);
  return DSA_OK;
}

int32_t mla_sparse_attend(const dsa_batch_t* batch, int32_t dtype, int32_t rope_dim, const void* q, const void* kv,
                          const int32_t* idx, int32_t k, float scale, void* out, int32_t out_dtype,
                          float* lse, void* ws, size_t ws_bytes, void* stream) {
  dsa::BatchDev b;
  int st = check_batch(batch, &b);
  if (st) return st;
  if ((st = check_dtype(dtype, "dtype"))) return st;
  if ((st = check_rope(rope_dim))) return st;
  if ((st = check_dtype(out_dtype, "out_dtype"))) return st;
  if ((st = check_k(k))) return st;
  if (b.nq == 0) return DSA_OK;
  if ((st = check_mla_layer(q, kv, out))) return st;
  REQUIRE_PTR4(idx);
  OPTIONAL_PTR4(lse);
  const size_t need = dsa::mla_workspace_bytes(dtype, b.nq, k, 1);
  if (need > 0 && (ws == nullptr || ws_bytes < need))
    return fail(DSA_ERR_WORKSPACE, "MLA workspace: %zu bytes given, %zu needed", ws_bytes, need);
  if (ws && !aligned16(ws)) return fail(DSA_ERR_ALIGN, "ws is not 16-byte aligned");
  dsa::MlaLayers L;
  memset(&L, 0, sizeof(L));
  L.q[0] = q;
  L.kv[0] = kv;
  L.out[0] = out;
  L.lse[0] = lse;
  return hip_status(dsa::launch_mla(b, dtype, rope_dim, L, 1, idx, k, scale, out_dtype, ws, ws_bytes,
                                    as_stream(stream)),
                    "mla_sparse_attend launch");
}

size_t dsa_mla_decode_fused_workspace_size(int32_t nq, int32_t max_len, int32_t k, int32_t n_layers) {
  if (nq <= 0 || max_len <= 0 || k <= 0 || n_layers <= 0) return 0;
  return dsa::fused_layout(nq, max_len, k, n_layers).bytes;
}

// Indexer scores, then top-k into idx, in the scores, histogram and top-k
// parts of a fused-layout workspace.  The indexer counts the top-k's
// first-level histograms into the histogram part, which each call leaves
// zero (the top-k checks it and clears it after use), so the workspace
// needs no clearing by the caller.
static int run_selection(const dsa::BatchDev& b, int32_t index_dtype, const void* q_idx, const float* w_idx,
                         const void* k_idx, int32_t k, int32_t* idx, char* base, const dsa::FusedLayout& f,
                         hipStream_t s) {
  int st;
  float* scores = (float*)(base + f.scores);
  uint32_t* hist = (uint32_t*)(base + f.hist);
  bool counted = false;
  if ((st = hip_status(
           dsa::launch_index_score(b, index_dtype, q_idx, w_idx, k_idx, scores, f.score_ld, s, hist, &counted),
           "index score launch")))
    return st;
  return hip_status(dsa::launch_topk(b, scores, f.score_ld, k, idx, nullptr, base + f.topk, f.mla - f.topk, s,
                                     counted ? hist : nullptr),
                    "top-k launch");
}

int32_t dsa_mla_decode_fused(const dsa_batch_t* batch, int32_t index_dtype, const void* q_idx,
                             const float* w_idx, const void* k_idx, int32_t k, int32_t n_layers,
                             int32_t dtype, int32_t rope_dim, const void* const* q_l, const void* const* kv_l,
                             void* const* out_l, float* const* lse_l, int32_t out_dtype, float scale,
                             int32_t* idx_out, void* ws, size_t ws_bytes, void* stream) {
  return dsa::fused_read(batch, index_dtype, q_idx, w_idx, k_idx, k, n_layers, dtype, rope_dim, q_l, kv_l, out_l,
                         lse_l, out_dtype, scale, idx_out, ws, ws_bytes, nullptr, stream);
}

int32_t dsa_ml4_layer_plan(int32_t n_layers, dsa_layer_plan_t* plan) {
  if (plan == nullptr) return fail(DSA_ERR_NULL, "plan is NULL");
  if (n_layers < 1 || n_layers > DSA_ML4_LAYERS)
    return fail(DSA_ERR_SHAPE, "n_layers = %d outside [1, %d]", n_layers, DSA_ML4_LAYERS);
  for (int l = 0; l < n_layers; ++l) {
    const bool nope = (l & 3) == 3;                     // layers 3, 7, 11, ...: no rotary encoding
    plan[l].rope_dim = nope ? 0 : DSA_ROPE;
    plan[l].kv_source = (nope && l > 35) ? 35 : l;      // later rotary-free layers read layer 35's latent
    plan[l].runs_indexer = (l < 16 || (l & 3) == 0 || nope) ? 1 : 0;  // from 16, the middle two of a group reuse
  }
  return DSA_OK;
}

// Validates a plan; on success *max_group is the largest number of layers
// one MLA launch covers (consecutive layers with one selection and one
// rope_dim, at most DSA_MAX_LAYERS).
static int check_plan(int32_t n_layers, const dsa_layer_plan_t* plan, int* max_group) {
  if (plan == nullptr) return fail(DSA_ERR_NULL, "plan is NULL");
  if (n_layers < 1 || n_layers > DSA_ML4_LAYERS)
    return fail(DSA_ERR_SHAPE, "n_layers = %d outside [1, %d]", n_layers, DSA_ML4_LAYERS);
  if (!plan[0].runs_indexer) return fail(DSA_ERR_SHAPE, "layer 0 does not run its indexer");
  int group = 0, best = 0;
  for (int l = 0; l < n_layers; ++l) {
    const dsa_layer_plan_t& p = plan[l];
    if (p.rope_dim != 0 && p.rope_dim != DSA_ROPE)
      return fail(DSA_ERR_SHAPE, "layer %d: rope_dim = %d is neither 0 nor %d", l, p.rope_dim, DSA_ROPE);
    if (p.kv_source < 0 || p.kv_source > l)
      return fail(DSA_ERR_SHAPE, "layer %d: kv_source = %d is not an earlier layer", l, p.kv_source);
    const dsa_layer_plan_t& src = plan[p.kv_source];
    if (src.kv_source != p.kv_source)
      return fail(DSA_ERR_SHAPE, "layer %d: its kv_source %d does not own its cache", l, p.kv_source);
    if (src.rope_dim != p.rope_dim)
      return fail(DSA_ERR_SHAPE, "layer %d: kv_source %d has another rope_dim", l, p.kv_source);
    const bool joins = l > 0 && !p.runs_indexer && p.rope_dim == plan[l - 1].rope_dim && group < DSA_MAX_LAYERS;
    group = joins ? group + 1 : 1;
    best = group > best ? group : best;
  }
  *max_group = best;
  return DSA_OK;
}

size_t dsa_mla_decode_layers_workspace_size(int32_t nq, int32_t max_len, int32_t k, int32_t n_layers,
                                            const dsa_layer_plan_t* plan) {
  int group = 0;
  if (nq <= 0 || max_len <= 0 || k <= 0 || check_plan(n_layers, plan, &group)) return 0;
  return dsa::fused_layout(nq, max_len, k, group).bytes;
}

int32_t dsa_mla_decode_layers(const dsa_batch_t* batch, int32_t n_layers, const dsa_layer_plan_t* plan,
                              int32_t index_dtype, const void* const* q_idx_l, const float* const* w_idx_l,
                              const void* const* k_idx_l, int32_t k, int32_t dtype, const void* const* q_l,
                              const void* const* kv_l, void* const* out_l, float* const* lse_l, int32_t out_dtype,
                              float scale, int32_t* const* idx_l, void* ws, size_t ws_bytes, void* stream) {
  dsa::BatchDev b;
  int st = check_batch(batch, &b);
  if (st) return st;
  int max_group = 0;
  if ((st = check_plan(n_layers, plan, &max_group))) return st;
  if ((st = check_index_dtype(index_dtype, "index_dtype"))) return st;
  if ((st = check_dtype(dtype, "dtype"))) return st;
  if ((st = check_dtype(out_dtype, "out_dtype"))) return st;
  if ((st = check_k(k))) return st;
  if (b.nq == 0) return DSA_OK;
  if (!q_idx_l || !w_idx_l || !k_idx_l || !q_l || !kv_l || !out_l)
    return fail(DSA_ERR_NULL, "a per-layer pointer table is NULL");
  for (int l = 0; l < n_layers; ++l) {
    if (plan[l].runs_indexer) {
      const void* q_idx = q_idx_l[l];
      const void* w_idx = w_idx_l[l];
      const void* k_idx = k_idx_l[l];
      REQUIRE_PTR(q_idx);
      REQUIRE_PTR(w_idx);
      REQUIRE_PTR(k_idx);
      if (idx_l && idx_l[l] && !aligned(idx_l[l], 4)) return fail(DSA_ERR_ALIGN, "idx_l[%d] is not 4-byte aligned", l);
    }
    if ((st = check_mla_layer(q_l[l], kv_l[plan[l].kv_source], out_l[l]))) return st;
    if (lse_l && lse_l[l] && !aligned(lse_l[l], 4)) return fail(DSA_ERR_ALIGN, "lse_l[%d] is not 4-byte aligned", l);
  }
  const dsa::FusedLayout f = dsa::fused_layout(b.nq, b.max_len, k, max_group);
  const size_t need = f.bytes;
  if (ws == nullptr || ws_bytes < need)
    return fail(DSA_ERR_WORKSPACE, "layers workspace: %zu bytes given, %zu needed", ws_bytes, need);
  if (!aligned16(ws)) return fail(DSA_ERR_ALIGN, "ws is not 16-byte aligned");
  char* base = (char*)ws;
  hipStream_t s = as_stream(stream);
  int32_t* idx = nullptr;
  for (int l = 0; l < n_layers;) {
    if (plan[l].runs_indexer) {
      idx = (idx_l && idx_l[l]) ? idx_l[l] : (int32_t*)(base + f.idx);
      if ((st = run_selection(b, index_dtype, q_idx_l[l], w_idx_l[l], k_idx_l[l], k, idx, base, f, s))) return st;
    }
    // this layer and the following ones that reuse the same selection with
    // the same rotary width: one MLA launch
    int n = 1;
    while (l + n < n_layers && n < DSA_MAX_LAYERS && !plan[l + n].runs_indexer &&
           plan[l + n].rope_dim == plan[l].rope_dim)
      ++n;
    dsa::MlaLayers L;
    memset(&L, 0, sizeof(L));
    for (int j = 0; j < n; ++j) {
      L.q[j] = q_l[l + j];
      L.kv[j] = kv_l[plan[l + j].kv_source];
      L.out[j] = out_l[l + j];
      L.lse[j] = lse_l ? lse_l[l + j] : nullptr;
    }
    if ((st = hip_status(dsa::launch_mla(b, dtype, plan[l].rope_dim, L, n, idx, k, scale, out_dtype,
                                         base + f.mla, need - f.mla, s),
                         "layers: MLA launch")))
      return st;
    l += n;
  }
  return DSA_OK;
}

int32_t dsa_rope_frequencies(const float* alpha, double* freq) {
  if (freq == nullptr) return fail(DSA_ERR_NULL, "freq is NULL");
  dsa::rope_frequencies(alpha, freq);
  return DSA_OK;
}

int32_t dsa_rope_append(const dsa_batch_t* batch, int32_t dtype, int32_t rope_dim, const double* freq,
                        const float* latent, const float* rope_key, void* kv, void* q_attn, const float* ssmax_s,
                        const float* ssmax_b, void* stream) {
  dsa::BatchDev b;
  int st = check_batch(batch, &b);
  if (st) return st;
  if ((st = check_dtype(dtype, "dtype"))) return st;
  if ((st = check_rope(rope_dim))) return st;
  if ((ssmax_s == nullptr) != (ssmax_b == nullptr))
    return fail(DSA_ERR_NULL, "ssmax_s and ssmax_b must be given together");
  if (b.nq == 0) return DSA_OK;
  REQUIRE_PTR(latent);
  REQUIRE_PTR(kv);
  if (rope_dim) {
    REQUIRE_PTR(freq);
    REQUIRE_PTR(rope_key);
  }
  if (q_attn && !aligned16(q_attn)) return fail(DSA_ERR_ALIGN, "q_attn is not 16-byte aligned");
  if (ssmax_s && (!aligned16(ssmax_s) || !aligned16(ssmax_b)))
    return fail(DSA_ERR_ALIGN, "ssmax arrays are not 16-byte aligned");
  return hip_status(dsa::launch_rope_append(b, dtype, rope_dim, freq, latent, rope_key, kv, q_attn, ssmax_s, ssmax_b,
                                            as_stream(stream)),
                    "dsa_rope_append launch");
}

}  // extern "C"

namespace dsa {

int fused_read(const dsa_batch_t* batch, int32_t index_dtype, const void* q_idx, const float* w_idx,
               const void* k_idx, int32_t k, int32_t n_layers, int32_t dtype, int32_t rope_dim,
               const void* const* q_l, const void* const* kv_l, void* const* out_l, float* const* lse_l,
               int32_t out_dtype, float scale, int32_t* idx_out, void* ws, size_t ws_bytes, ScratchFn scratch,
               void* stream) {
  dsa::BatchDev b;
  int st = check_batch(batch, &b);
  if (st) return st;
  if ((st = check_index_dtype(index_dtype, "index_dtype"))) return st;
  if ((st = check_dtype(dtype, "dtype"))) return st;
  if ((st = check_rope(rope_dim))) return st;
  if ((st = check_dtype(out_dtype, "out_dtype"))) return st;
  if ((st = check_k(k))) return st;
  if (n_layers < 1) return fail(DSA_ERR_SHAPE, "n_layers = %d < 1", n_layers);
  if (n_layers > DSA_MAX_LAYERS) return fail(DSA_ERR_UNSUPPORTED, "n_layers = %d > %d", n_layers, DSA_MAX_LAYERS);
  if (b.nq == 0) return DSA_OK;
  REQUIRE_PTR(q_idx);
  REQUIRE_PTR(w_idx);
  REQUIRE_PTR(k_idx);
  if (!q_l || !kv_l || !out_l) return fail(DSA_ERR_NULL, "a per-layer pointer table is NULL");
  dsa::MlaLayers L;
  memset(&L, 0, sizeof(L));
  for (int l = 0; l < n_layers; ++l) {
    if ((st = check_mla_layer(q_l[l], kv_l[l], out_l[l]))) return st;
    if (lse_l && lse_l[l] && !aligned(lse_l[l], 4)) return fail(DSA_ERR_ALIGN, "lse_l[%d] is not 4-byte aligned", l);
    L.q[l] = q_l[l];
    L.kv[l] = kv_l[l];
    L.out[l] = out_l[l];
    L.lse[l] = lse_l ? lse_l[l] : nullptr;
  }
  OPTIONAL_PTR4(idx_out);
  const dsa::FusedLayout f = dsa::fused_layout(b.nq, b.max_len, k, n_layers);
  const size_t need = f.bytes;
  if (scratch != nullptr && (st = scratch(need, &ws, &ws_bytes))) return st;
  if (ws == nullptr || ws_bytes < need)
    return fail(DSA_ERR_WORKSPACE, "fused workspace: %zu bytes given, %zu needed", ws_bytes, need);
  if (!aligned16(ws)) return fail(DSA_ERR_ALIGN, "ws is not 16-byte aligned");
  char* base = (char*)ws;
  int32_t* idx = idx_out ? idx_out : (int32_t*)(base + f.idx);
  hipStream_t s = as_stream(stream);
  if ((st = run_selection(b, index_dtype, q_idx, w_idx, k_idx, k, idx, base, f, s))) return st;
  return hip_status(dsa::launch_mla(b, dtype, rope_dim, L, n_layers, idx, k, scale, out_dtype, base + f.mla,
                                    need - f.mla, s),
                    "fused: MLA launch");
}

}  // namespace dsa
