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

// Indexer scores of every query over its candidates (indexer.hip).  The
// first workgroup of each query also zeroes that query's words of `z`
// (nobody else touches them during the launch).
hipError_t launch_index_score(const BatchDev& b, int dtype, const void* qI, const float* w,
                              const void* kI, float* scores, int64_t ld, hipStream_t st,
                              const ZeroSpans* z = nullptr);

// Top-k selection (topk.hip).  ws may be NULL when topk_workspace_bytes() == 0.
// With ws_zeroed, the words topk_zero_span() describes are already zero.
size_t topk_workspace_bytes(int nq, int max_len, int k);
ZeroSpan topk_zero_span(void* ws, int nq, int max_len);
hipError_t launch_topk(const BatchDev& b, const float* scores, int64_t ld, int k, int32_t* idx,
                       int32_t* count, void* ws, size_t ws_bytes, hipStream_t st, bool ws_zeroed = false);

// Sparse MLA over a shared selection for n_layers layers (mla.hip).
struct MlaLayers {
  const void* q[MLA_MAX_LAYERS];
  const void* kv[MLA_MAX_LAYERS];
  void* out[MLA_MAX_LAYERS];
  float* lse[MLA_MAX_LAYERS];
};
int mla_num_splits(int dtype, int nq, int k, int n_layers);
size_t mla_workspace_bytes(int dtype, int nq, int k, int n_layers);
// rope: rotary width of every layer's rows (DR, or 0 without rotary encoding).
hipError_t launch_mla(const BatchDev& b, int dtype, int rope, const MlaLayers& layers, int n_layers,
                      const int32_t* idx, int k, float scale, int out_dtype, void* ws,
                      size_t ws_bytes, hipStream_t st);

// Rotary frequencies (host) and the rotary / cache-append step (rope.hip).
void rope_frequencies(const float* alpha, double* out);
hipError_t launch_rope_append(const BatchDev& b, int dtype, int rope, const double* freq, const float* latent,
                              const float* rope_key, void* kv, void* q, const float* ss, const float* sb,
                              hipStream_t st);

}  // namespace dsa
