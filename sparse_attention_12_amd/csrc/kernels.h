// Host-side launchers of the gfx950 kernels, called by the C ABI layer.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "dsa_common.h"

namespace dsa {

constexpr int MLA_MAX_LAYERS = 16;

// Per-query blocks of 32-bit words that must be zero before a later kernel
// runs: query q owns words [q*stride, q*stride + count) of `base`.
struct ZeroSpan {
  uint32_t* base;
  int stride;
  int count;
};
struct ZeroSpans {
  ZeroSpan s[2];
};

// Zeroes every span (one workgroup per query).
hipError_t launch_zero(const ZeroSpans& z, int nq, hipStream_t st);

// Indexer scores of every query over its candidates (indexer.hip).  With
// hist (may be NULL) and a decode batch of at most IDX_BAL_MAXQ queries, the
// launch also adds each query's scores to hist[q][0, TK_BINS1) by their top
// TK_BITS1 key bits (the top-k's first radix level).  The top-k uses such a
// histogram only if its bins sum to the row's length (true exactly when it
// started from zero) and clears it after use; *hist_done (may be NULL) says
// whether the launch counted.
hipError_t launch_index_score(const BatchDev& b, int dtype, const void* qI, const float* w,
                              const void* kI, float* scores, int64_t ld, hipStream_t st,
                              uint32_t* hist = nullptr, bool* hist_done = nullptr);

// Top-k selection (topk.hip).  ws may be NULL when topk_workspace_bytes() ==
// 0.  hist_pre (may be NULL): the indexer's first-level histograms
// [nq][TK_BINS1]; each query's is checked (its bins must sum to the query's
// candidate count, which holds exactly when it started from zero), used in
// place of a counting pass when it checks out, and cleared for the next call
// either way.
hipError_t launch_topk(const BatchDev& b, const float* scores, int64_t ld, int k, int32_t* idx,
                       int32_t* count, void* ws, size_t ws_bytes, hipStream_t st, uint32_t* hist_pre = nullptr);

#ifdef DSA_DEBUG
// Flag words of the debug checks, one per kernel source (DBG_* bits in
// dsa_common.h); each read is synchronous, reset clears the word.
uint32_t debug_flags_indexer(bool reset);
uint32_t debug_flags_topk(bool reset);
uint32_t debug_flags_mla(bool reset);
#endif

// Sparse MLA over a shared selection for n_layers layers (mla.hip).
struct MlaLayers {
  const void* q[MLA_MAX_LAYERS];
  const void* kv[MLA_MAX_LAYERS];
  void* out[MLA_MAX_LAYERS];
  float* lse[MLA_MAX_LAYERS];
};
// rope: rotary width of every layer's rows (DR, or 0 without rotary encoding).
hipError_t launch_mla(const BatchDev& b, int dtype, int rope, const MlaLayers& layers, int n_layers,
                      const int32_t* idx, int k, float scale, int out_dtype, void* ws,
                      size_t ws_bytes, hipStream_t st);

// The rotary / cache-append step (rope.hip).
hipError_t launch_rope_append(const BatchDev& b, int dtype, int rope, const double* freq, const float* latent,
                              const float* rope_key, void* kv, void* q, const float* ss, const float* sb,
                              hipStream_t st);

}  // namespace dsa
