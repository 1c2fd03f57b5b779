// Shared device helpers of the gfx950 kernels: fixed shapes, bf16 handling,
// MFMA operand types, per-query candidate ranges and the order-preserving
// score key used by the selection.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "plan.h"

namespace dsa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));  // 32 fp8 operand bytes

// Device copy of the host batch descriptor (passed by value to kernels).
struct BatchDev {
  int nq, nseq, max_len;
  const int32_t* q_seq;
  const int32_t* q_pos;
  const int32_t* seq_len;
  const int64_t* seq_row0;
};

struct QueryRange {
  int n;        // candidates: positions [0, n)
  int64_t row0; // first row of the query's sequence in the caches
};

// Checks of a debug build (-DDSA_DEBUG): a failed check sets its bit in the
// translation unit's flag word, read and cleared from the host through
// dsa_debug_flags; nothing traps.  Release builds compile the checks away.
constexpr uint32_t DBG_IDX_RANGE = 1u;     // an MLA selection entry outside [-1, n) (skipped)
constexpr uint32_t DBG_TOPK_SLOT = 2u;     // a top-k output or candidate slot past its bound
constexpr uint32_t DBG_LIST = 4u;          // the split path's chunk lists disagree with the histogram
constexpr uint32_t DBG_SCORE_COL = 8u;     // an indexer score column at or past the row stride
constexpr uint32_t DBG_HIST_RECOUNT = 16u; // a precounted histogram failed its check and was recounted
constexpr uint32_t DBG_GATHER_ROW = 32u;   // an MLA gather row past its sequence
#ifdef DSA_DEBUG
static __device__ uint32_t dbg_flags;
#define DSA_CHECK(cond, bit)                 \
  do {                                       \
    if (!(cond)) atomicOr(&dbg_flags, (bit)); \
  } while (0)
// Reads (and, with reset, clears) this translation unit's flag word
// (synchronous; defined once per unit by DSA_DEBUG_READER).
#define DSA_DEBUG_READER(fn)                                                          \
  uint32_t fn(bool reset) {                                                           \
    uint32_t v = 0;                                                                   \
    if (hipMemcpyFromSymbol(&v, HIP_SYMBOL(dbg_flags), sizeof(v), 0, hipMemcpyDeviceToHost) != hipSuccess) \
      return 0xffffffffu;                                                             \
    if (reset) {                                                                      \
      const uint32_t z = 0;                                                           \
      if (hipMemcpyToSymbol(HIP_SYMBOL(dbg_flags), &z, sizeof(z), 0, hipMemcpyHostToDevice) != hipSuccess) \
        return 0xffffffffu;                                                           \
    }                                                                                 \
    return v;                                                                         \
  }
#else
#define DSA_CHECK(cond, bit) \
  do {                       \
  } while (0)
#endif

// Candidates of query q: its own position and every earlier one, clamped to
// the sequence length and to max_len (so no access leaves the sequence).
__device__ inline QueryRange query_range(const BatchDev& b, int q) {
  QueryRange r;
  int s = b.q_seq[q];
  if (s < 0 || s >= b.nseq) {
    r.n = 0;
    r.row0 = 0;
    return r;
  }
  int64_t n = (int64_t)b.q_pos[q] + 1;
  int64_t L = b.seq_len[s];
  if (L < n) n = L;
  if (b.max_len < n) n = b.max_len;
  if (n < 0) n = 0;
  r.n = (int)n;
  r.row0 = b.seq_row0[s];
  return r;
}

__device__ inline float bf16_to_f32(uint16_t x) { return __uint_as_float((uint32_t)x << 16); }

// Reductions over lanes l, l^16, l^32, l^48 (the four 16-lane rows of a
// wave) with gfx950's row swaps (v_permlane16_swap / v_permlane32_swap):
// pure VALU, no LDS round trip.  Each swap of x with itself leaves, in every
// lane, the values of the two rows being paired, so the pair's max or sum
// needs no lane select.
// max(x, 0) in one integer instruction: a float with the sign bit set is a
// negative integer, and non-negative floats order as their bit patterns, so
// the signed-integer max with 0 is max(x, +0) for every non-NaN x (fmaxf
// costs a second instruction that quiets NaNs first).
__device__ inline float relu(float x) { return __int_as_float(max(__float_as_int(x), 0)); }

__device__ inline float rows4_max(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

// Sum over lanes l and l^32 (the two halves of a wave).
__device__ inline float halves_sum(float x) {
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

__device__ inline float rows4_sum(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// Two floats -> packed bf16 pair (low half = a), rounded to nearest even by
// the gfx950 conversion instruction (v_cvt_pk_bf16_f32).
typedef __bf16 hw_bf16x2 __attribute__((ext_vector_type(2)));
__device__ inline uint32_t pack_bf16x2(float a, float b) {
  const f32x2 v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, hw_bf16x2));
}

// Unsigned key whose order is the order of the float scores; -0.0 and +0.0
// map to the same key.
__device__ inline uint32_t score_key(float s) {
  uint32_t u = __float_as_uint(s == 0.0f ? 0.0f : s);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// 64-bit key that is unique per position: higher score first, then lower
// position first.
__device__ inline uint64_t select_key(uint32_t skey, int pos) {
  return ((uint64_t)skey << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)pos);
}

__device__ inline u32x4 load16_nt(const void* p) {
  return __builtin_nontemporal_load((const u32x4*)p);
}

__device__ inline u32x4 load16(const void* p) { return *(const u32x4*)p; }

__device__ inline bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

}  // namespace dsa
