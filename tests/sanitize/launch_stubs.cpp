// Stand-ins for the kernel launchers of the library, for a host-only build
// of its C ABI layer under AddressSanitizer and UndefinedBehaviorSanitizer:
// each records the call and checks the arguments it can check without a
// GPU (non-null device pointers where the launch needs them, sizes in
// range), so that a sanitized run covers every host path of the entry
// points, including the ones that would launch.
#include <stdio.h>
#include <stdlib.h>

#include "../../sparse_attention_12_amd/csrc/kernels.h"

namespace {
int n_index, n_topk, n_mla, n_rope, n_zero, n_bad;
void expect(bool ok, const char* what) {
  if (!ok) {
    fprintf(stderr, "launch stub: %s\n", what);
    ++n_bad;
  }
}
}  // namespace

extern "C" int stub_calls(int which) {
  switch (which) {
    case 0: return n_index;
    case 1: return n_topk;
    case 2: return n_mla;
    case 3: return n_rope;
    case 4: return n_zero;
    default: return n_bad;
  }
}

extern "C" void stub_reset(void) { n_index = n_topk = n_mla = n_rope = n_zero = n_bad = 0; }

const char* hipGetErrorString(hipError_t) { return "stubbed HIP runtime"; }

namespace dsa {

hipError_t launch_zero(const ZeroSpans&, int nq, hipStream_t) {
  ++n_zero;
  expect(nq >= 0, "launch_zero: nq < 0");
  return hipSuccess;
}

hipError_t launch_index_score(const BatchDev& b, int dtype, const void* qI, const float* w, const void* kI,
                              float* scores, int64_t ld, hipStream_t, uint32_t* hist, bool* hist_done) {
  ++n_index;
  expect(b.nq > 0 && qI && w && kI && scores, "launch_index_score: empty batch or NULL array");
  expect(ld >= b.max_len, "launch_index_score: ld < max_len");
  expect(dtype >= 0 && dtype <= 2, "launch_index_score: dtype");
  const bool bal = index_kernel(dtype, b.nq, b.nseq) == IndexKernel::Balanced;
  if (hist_done) *hist_done = bal && hist != nullptr;
  return hipSuccess;
}

hipError_t launch_topk(const BatchDev& b, const float* scores, int64_t ld, int k, int32_t* idx, int32_t*, void* ws,
                       size_t ws_bytes, hipStream_t, uint32_t*) {
  ++n_topk;
  expect(b.nq > 0 && scores && idx, "launch_topk: empty batch or NULL array");
  expect(k >= 1 && k <= KMAX && ld >= b.max_len, "launch_topk: k or ld");
  const size_t need = topk_workspace_bytes(b.nq, b.max_len, k);
  expect(need == 0 || (ws && ws_bytes >= need), "launch_topk: workspace smaller than its layout");
  return hipSuccess;
}

hipError_t launch_mla(const BatchDev& b, int dtype, int rope, const MlaLayers& L, int n_layers, const int32_t* idx,
                      int k, float, int out_dtype, void* ws, size_t ws_bytes, hipStream_t) {
  ++n_mla;
  expect(b.nq > 0 && idx && n_layers >= 1 && n_layers <= MLA_MAX_LAYERS, "launch_mla: batch, idx or layers");
  expect(rope == 0 || rope == DR, "launch_mla: rope width");
  expect((dtype == 0 || dtype == 1) && (out_dtype == 0 || out_dtype == 1), "launch_mla: dtype");
  for (int l = 0; l < n_layers; ++l) expect(L.q[l] && L.kv[l] && L.out[l], "launch_mla: NULL layer array");
  const size_t need = mla_workspace_bytes(dtype, b.nq, k, n_layers);
  expect(need == 0 || (ws && ws_bytes >= need), "launch_mla: workspace smaller than the split partials");
  return hipSuccess;
}

hipError_t launch_rope_append(const BatchDev& b, int dtype, int rope, const double* freq, const float* latent,
                              const float* rope_key, void* kv, void*, const float* ss, const float* sb,
                              hipStream_t) {
  ++n_rope;
  expect(b.nq > 0 && latent && kv && (dtype == 0 || dtype == 1), "launch_rope_append: arrays or dtype");
  expect(rope == 0 || (freq && rope_key), "launch_rope_append: rotary arrays");
  expect((ss == nullptr) == (sb == nullptr), "launch_rope_append: scaling arrays");
  return hipSuccess;
}

}  // namespace dsa
