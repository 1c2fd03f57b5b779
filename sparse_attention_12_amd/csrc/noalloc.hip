// The allocation-free fused decode read (dsa_mla_decode_fused_noalloc in
// include/dsa_mla.h): the fused read of abi.hip over a scratch array the
// library owns, one per GPU, for callers that cannot allocate.
#include <mutex>

#include "../../include/dsa_mla.h"
#include "abi_internal.h"

// One copy of this array per GPU, held until the process ends.  Host code
// never uses the array's name as an address: each device's copy is found
// once with hipGetSymbolAddress (with that device current) and its address
// kept in scratch_dev.
static __device__ __align__(256) unsigned char scratch[DSA_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int SCRATCH_MAX_DEVICES = 64;
std::mutex scratch_mu;
void* scratch_dev[SCRATCH_MAX_DEVICES];

// The current device's scratch array (its address looked up on the first
// call on that device) for a batch that needs `need` bytes.
int scratch_for(size_t need, void** ws, size_t* ws_bytes) {
  if (need > (size_t)DSA_NOALLOC_SCRATCH_BYTES)
    return dsa::abi_fail(DSA_ERR_WORKSPACE,
                         "this batch needs %zu bytes of scratch; the allocation-free entry holds %zu (use "
                         "dsa_mla_decode_fused with a workspace)",
                         need, (size_t)DSA_NOALLOC_SCRATCH_BYTES);
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return dsa::abi_hip_status(e, "hipGetDevice");
  if (dev < 0 || dev >= SCRATCH_MAX_DEVICES)
    return dsa::abi_fail(DSA_ERR_UNSUPPORTED, "device %d: the allocation-free entry supports devices 0..%d", dev,
                         SCRATCH_MAX_DEVICES - 1);
  std::lock_guard<std::mutex> lock(scratch_mu);
  if (scratch_dev[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return dsa::abi_hip_status(e, "hipGetSymbolAddress(scratch)");
    if (p == nullptr || ((uintptr_t)p & 255u) != 0)
      return dsa::abi_fail(DSA_ERR_HIP, "the scratch array of device %d has no usable address", dev);
    scratch_dev[dev] = p;
  }
  *ws = scratch_dev[dev];
  *ws_bytes = (size_t)DSA_NOALLOC_SCRATCH_BYTES;
  return DSA_OK;
}

}  // namespace

extern "C" int32_t dsa_mla_decode_fused_noalloc(const dsa_batch_t* batch, int32_t index_dtype, const void* q_idx,
                                                const float* w_idx, const void* k_idx, int32_t k, int32_t n_layers,
                                                int32_t dtype, int32_t rope_dim, const void* const* q_l,
                                                const void* const* kv_l, void* const* out_l, float* const* lse_l,
                                                int32_t out_dtype, float scale, int32_t* idx_out, void* stream) {
  return dsa::fused_read(batch, index_dtype, q_idx, w_idx, k_idx, k, n_layers, dtype, rope_dim, q_l, kv_l, out_l,
                         lse_l, out_dtype, scale, idx_out, nullptr, 0, scratch_for, stream);
}
