// Rotary encoding and cache append on gfx950: the step just upstream of the
// attention read (concept page "Mistral Large 4", sections "Positions" and
// "Query scaling").
//
// The frequencies (host, double precision) come from rope_frequencies in
// plan.cpp: YaRN with an original window of 512 and a stretch of 2,048,
// then LeRoPE's learned multipliers.
// Per new token at 0-based position t (pair i = values 2i, 2i+1 of the
// rotary part, turned by the angle t * omega_i):
//   cache row  = [latent (512) | rotated rotary key (64, rotary layers only)]
//   query h    = m_h(t) * q[h], its rotary part rotated;  m_h(t) =
//                s_h ln(t + 1) + b_h when per-head (s, b) are given (the
//                section's displayed formula was lost; its Scalable-Softmax
//                argument gives the c ln(visible positions) form, and the
//                learned offset b_h is a reading).
// Angles are formed in double precision (t * omega reaches 10^6 radians at
// the end of the 2^20-position range), then applied in float.
#include <math.h>

#include "dsa_common.h"
#include "kernels.h"

namespace dsa {

constexpr int ROPE_THREADS = 256;
constexpr int ROPE_HGROUPS = 8;   // workgroups per token in small batches, each over 8 query heads

template <typename T>
struct Elem;
template <>
struct Elem<float> {
  static __device__ inline void put2(float* p, int i, float a, float b) { *(f32x2*)(p + i) = f32x2{a, b}; }
  static __device__ inline f32x2 get2(const float* p, int i) { return *(const f32x2*)(p + i); }
};
template <>
struct Elem<uint16_t> {
  static __device__ inline f32x2 get2(const uint16_t* p, int i) {
    const uint32_t v = *(const uint32_t*)(p + i);
    return f32x2{__uint_as_float(v << 16), __uint_as_float(v & 0xFFFF0000u)};
  }
  static __device__ inline void put2(uint16_t* p, int i, float a, float b) { *(uint32_t*)(p + i) = pack_bf16x2(a, b); }
};

// gridDim.y workgroups per new token (blockIdx.y: a group of 64/gridDim.y
// query heads; the first group also writes the cache row): small batches
// spread a token over ROPE_HGROUPS workgroups, large ones take one each.
// Pair work is spread over the threads; each pair is two adjacent values, so
// every access is a 4- or 8-byte vector.
template <typename T>
__global__ __launch_bounds__(ROPE_THREADS) void rope_append_kernel(BatchDev b, int rope, const double* __restrict__ freq,
                                                                  const float* __restrict__ latent,
                                                                  const float* __restrict__ rope_key, T* __restrict__ kv,
                                                                  T* __restrict__ q, const float* __restrict__ ss,
                                                                  const float* __restrict__ sb) {
  __shared__ float cs[DR / 2], sn[DR / 2], msc[H];
  const int qi = blockIdx.x;
  const int tid = threadIdx.x;
  const int t = b.q_pos[qi];
  const QueryRange r = query_range(b, qi);
  // the token's own row must lie in its sequence (position t < seq_len)
  if (t < 0 || r.n != t + 1) return;
  if (rope && tid < DR / 2) {
    double sv, cv;
    sincos((double)t * freq[tid], &sv, &cv);
    cs[tid] = (float)cv;
    sn[tid] = (float)sv;
  }
  if (tid < H) msc[tid] = ss ? (float)((double)ss[tid] * log((double)t + 1.0) + (double)sb[tid]) : 1.0f;
  __syncthreads();
  const int W = DC + rope;
  // cache row
  T* row = kv + (r.row0 + t) * (int64_t)W;
  for (int e = tid; e < (blockIdx.y == 0 ? W / 2 : 0); e += ROPE_THREADS) {
    if (2 * e < DC) {
      const f32x2 v = *(const f32x2*)(latent + (int64_t)qi * DC + 2 * e);
      Elem<T>::put2(row, 2 * e, v[0], v[1]);
    } else {
      const int i = e - DC / 2;
      const f32x2 v = *(const f32x2*)(rope_key + (int64_t)qi * DR + 2 * i);
      Elem<T>::put2(row, 2 * e, v[0] * cs[i] - v[1] * sn[i], v[0] * sn[i] + v[1] * cs[i]);
    }
  }
  if (q == nullptr) return;
  // query, in place: scaled per head, rotary pairs rotated
  const int HG = H / (int)gridDim.y;
  T* qq = q + (int64_t)qi * H * W;
  for (int e = tid; e < HG * W / 2; e += ROPE_THREADS) {
    const int hl = e / (W / 2);
    const int h = blockIdx.y * HG + hl;
    const int c = 2 * (e - hl * (W / 2));
    const f32x2 v = Elem<T>::get2(qq, h * W + c);
    const float x = v[0] * msc[h], y = v[1] * msc[h];
    if (c < DC) {
      Elem<T>::put2(qq, h * W + c, x, y);
    } else {
      const int i = (c - DC) / 2;
      Elem<T>::put2(qq, h * W + c, x * cs[i] - y * sn[i], x * sn[i] + y * cs[i]);
    }
  }
}

hipError_t launch_rope_append(const BatchDev& b, int dtype, int rope, const double* freq, const float* latent,
                              const float* rope_key, void* kv, void* q, const float* ss, const float* sb,
                              hipStream_t st) {
  if (b.nq == 0) return hipSuccess;
  const dim3 grid(b.nq, b.nq < 256 ? ROPE_HGROUPS : 1);
  if (dtype == 0)
    hipLaunchKernelGGL(rope_append_kernel<float>, grid, dim3(ROPE_THREADS), 0, st, b, rope, freq, latent,
                       rope_key, (float*)kv, (float*)q, ss, sb);
  else
    hipLaunchKernelGGL(rope_append_kernel<uint16_t>, grid, dim3(ROPE_THREADS), 0, st, b, rope, freq, latent,
                       rope_key, (uint16_t*)kv, (uint16_t*)q, ss, sb);
  return hipGetLastError();
}

}  // namespace dsa
