// Internal interface between the C ABI layer (abi.hip) and the
// allocation-free entry (noalloc.hip).
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/dsa_mla.h"

namespace dsa {

// Records the message of a failing call (dsa_last_error) and returns status.
int abi_fail(int status, const char* fmt, ...);
// DSA_OK, or DSA_ERR_HIP with the runtime's message.
int abi_hip_status(hipError_t e, const char* what);

// Provides the workspace of a fused read that brings none: given the bytes
// the batch needs, sets *ws and *ws_bytes, or returns an error status.
typedef int (*ScratchFn)(size_t need, void** ws, size_t* ws_bytes);

// The fused decode read (dsa_mla_decode_fused), its workspace either given
// (ws, ws_bytes) or, with scratch, obtained after the arguments are checked.
int fused_read(const dsa_batch_t* batch, int32_t index_dtype, const void* q_idx, const float* w_idx,
               const void* k_idx, int32_t k, int32_t n_layers, int32_t dtype, int32_t rope_dim,
               const void* const* q_l, const void* const* kv_l, void* const* out_l, float* const* lse_l,
               int32_t out_dtype, float scale, int32_t* idx_out, void* ws, size_t ws_bytes, ScratchFn scratch,
               void* stream);

}  // namespace dsa
