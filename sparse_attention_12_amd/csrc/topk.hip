// Top-k selection on gfx950 (concept page "Mistral Large 4", section "Where
// to look": the indexer keeps the best 2,048 positions per query).
//
// The kept set is the first min(k, n) positions under (score descending,
// position ascending).  Each position gets a unique 64-bit key
//   key = orderable(score) << 32 | (2^32 - 1 - position)
// so the selection is "the k largest keys" and a radix select needs no
// separate tie handling.  One 1024-thread workgroup per query:
//   1. LDS histogram of the top 12 bits of every candidate's key,
//   2. find the bucket holding the k-th key; positions in higher buckets are
//      kept outright, positions in that bucket become candidates in LDS,
//   3. radix levels of 11 bits over the candidates' remaining 52 key bits
//      until the threshold key is fixed (usually two levels),
//   4. the kept positions are sorted ascending in LDS and written out.
// If the threshold bucket holds more candidates than LDS takes (e.g. many
// equal scores), step 3 runs over the score row itself and step 4 becomes
// an ordered compaction of the row.
#include "dsa_common.h"
#include "kernels.h"

namespace dsa {

constexpr int TK_THREADS = 1024;
constexpr int TK_WAVES = TK_THREADS / 64;
constexpr int TK_BITS1 = 12;
constexpr int TK_BINS1 = 1 << TK_BITS1;
constexpr int TK_LEVEL_BITS = 11;
constexpr int TK_CAP = 8192;  // threshold-bucket candidates held in LDS

struct TopkShared {
  uint32_t hist[TK_BINS1];
  uint32_t ckey[TK_CAP];
  int32_t cpos[TK_CAP];
  int32_t sel[KMAX];
  uint32_t wsum[TK_WAVES];
  uint32_t nsel;
  uint32_t ncand;
  int digit;
  uint32_t above;
};

// Exclusive prefix sum over the 1024 threads (thread order); *total gets
// the sum.  Contains barriers: every thread of the block must call it.
__device__ uint32_t block_exclusive_scan(uint32_t v, uint32_t* wsum, uint32_t* total) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  uint32_t x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    uint32_t y = __shfl_up(x, o);
    if (lane >= o) x += y;
  }
  if (lane == 63) wsum[wave] = x;
  __syncthreads();
  if (wave == 0) {
    uint32_t s = lane < TK_WAVES ? wsum[lane] : 0u;
    uint32_t t = s;
#pragma unroll
    for (int o = 1; o < TK_WAVES; o <<= 1) {
      uint32_t y = __shfl_up(t, o);
      if (lane >= o) t += y;
    }
    if (lane < TK_WAVES) wsum[lane] = t - s;  // exclusive wave offsets
    if (lane == TK_WAVES - 1) wsum[TK_WAVES - 1] = t - s, *total = t;
  }
  __syncthreads();
  const uint32_t res = wsum[wave] + x - v;
  __syncthreads();
  return res;
}

// Finds the bucket d such that fewer than `need` entries lie in buckets
// above d and at least `need` lie in d or above.  Thread 0 covers the
// highest buckets.  Result in sm.digit / sm.above (count strictly above).
__device__ void find_bucket(TopkShared& sm, int nbins, uint32_t need) {
  const int per = (nbins + TK_THREADS - 1) / TK_THREADS;
  const int hi = nbins - (int)threadIdx.x * per;
  const int lo = max(hi - per, 0);
  uint32_t local = 0;
  for (int b = lo; b < hi; ++b) local += sm.hist[b];
  uint32_t total;
  __shared__ uint32_t scan_total;
  uint32_t run = block_exclusive_scan(local, sm.wsum, &scan_total);
  for (int b = hi - 1; b >= lo; --b) {
    const uint32_t c = sm.hist[b];
    if (run < need && run + c >= need) {
      sm.digit = b;
      sm.above = run;
    }
    run += c;
  }
  (void)total;
  __syncthreads();
}

__device__ inline uint64_t row_key(const float* row, int s) {
  return select_key(score_key(row[s]), s);
}

__global__ __launch_bounds__(TK_THREADS) void topk_row_kernel(BatchDev b, const float* __restrict__ scores,
                                                              int64_t ld, int k, int32_t* __restrict__ idx,
                                                              int32_t* __restrict__ count) {
  __shared__ TopkShared sm;
  const int q = blockIdx.x;
  const int tid = threadIdx.x;
  const QueryRange r = query_range(b, q);
  const int n = r.n;
  int32_t* out = idx + (int64_t)q * k;
  if (n <= k) {
    for (int j = tid; j < k; j += TK_THREADS) out[j] = j < n ? j : -1;
    if (tid == 0 && count) count[q] = n;
    return;
  }
  const float* row = scores + (int64_t)q * ld;

  // 1. histogram of the top 12 key bits
  for (int i = tid; i < TK_BINS1; i += TK_THREADS) sm.hist[i] = 0;
  if (tid == 0) {
    sm.nsel = 0;
    sm.ncand = 0;
  }
  __syncthreads();
  for (int s = tid; s < n; s += TK_THREADS) atomicAdd(&sm.hist[score_key(row[s]) >> (32 - TK_BITS1)], 1u);
  __syncthreads();
  find_bucket(sm, TK_BINS1, (uint32_t)k);
  const uint32_t d1 = (uint32_t)sm.digit;
  uint32_t need = (uint32_t)k - sm.above;
  const uint32_t m = sm.hist[d1];
  const bool fits = m <= (uint32_t)TK_CAP;

  // 2. keep the higher buckets, collect the threshold bucket
  for (int s = tid; s < n; s += TK_THREADS) {
    const uint32_t u = score_key(row[s]);
    const uint32_t d = u >> (32 - TK_BITS1);
    if (d > d1) {
      const uint32_t slot = atomicAdd(&sm.nsel, 1u);
      if (slot < (uint32_t)KMAX) sm.sel[slot] = s;
    } else if (d == d1 && fits) {
      const uint32_t c = atomicAdd(&sm.ncand, 1u);
      if (c < (uint32_t)TK_CAP) {
        sm.ckey[c] = u;
        sm.cpos[c] = s;
      }
    }
  }
  __syncthreads();

  // 3. radix levels over the remaining key bits of the threshold bucket
  uint64_t prefix = d1;
  int plen = TK_BITS1;
  while (plen < 64) {
    const int bits = min(TK_LEVEL_BITS, 64 - plen);
    const int shift = 64 - plen - bits;
    const int nb = 1 << bits;
    for (int i = tid; i < nb; i += TK_THREADS) sm.hist[i] = 0;
    __syncthreads();
    if (fits) {
      for (int c = tid; c < (int)m; c += TK_THREADS) {
        const uint64_t key = select_key(sm.ckey[c], sm.cpos[c]);
        if ((key >> (64 - plen)) == prefix) atomicAdd(&sm.hist[(key >> shift) & (uint64_t)(nb - 1)], 1u);
      }
    } else {
      for (int s = tid; s < n; s += TK_THREADS) {
        const uint64_t key = row_key(row, s);
        if ((key >> (64 - plen)) == prefix) atomicAdd(&sm.hist[(key >> shift) & (uint64_t)(nb - 1)], 1u);
      }
    }
    __syncthreads();
    find_bucket(sm, nb, need);
    const uint32_t d = (uint32_t)sm.digit;
    need -= sm.above;
    const uint32_t cnt = sm.hist[d];
    prefix = (prefix << bits) | d;
    plen += bits;
    __syncthreads();
    if (cnt == need) break;
  }
  const uint64_t thresh = plen >= 64 ? prefix : (prefix << (64 - plen));

  if (fits) {
    // 4. add the kept candidates, sort ascending, write
    for (int c = tid; c < (int)m; c += TK_THREADS) {
      if (select_key(sm.ckey[c], sm.cpos[c]) >= thresh) {
        const uint32_t slot = atomicAdd(&sm.nsel, 1u);
        if (slot < (uint32_t)KMAX) sm.sel[slot] = sm.cpos[c];
      }
    }
    int P = 1;
    while (P < k) P <<= 1;
    __syncthreads();
    for (int j = k + tid; j < P; j += TK_THREADS) sm.sel[j] = 0x7FFFFFFF;
    __syncthreads();
    for (int size = 2; size <= P; size <<= 1) {
      for (int stride = size >> 1; stride > 0; stride >>= 1) {
        for (int i = tid; i < (P >> 1); i += TK_THREADS) {
          const int lo = 2 * i - (i & (stride - 1));
          const int hi = lo + stride;
          const bool up = (lo & size) == 0;
          const int x = sm.sel[lo], y = sm.sel[hi];
          if ((x > y) == up) {
            sm.sel[lo] = y;
            sm.sel[hi] = x;
          }
        }
        __syncthreads();
      }
    }
    for (int j = tid; j < k; j += TK_THREADS) out[j] = sm.sel[j];
  } else {
    // 4'. ordered compaction of the row: keep every key >= threshold
    uint32_t base = 0;
    __shared__ uint32_t tile_total;
    for (int t0 = 0; t0 < n; t0 += TK_THREADS) {
      const int s = t0 + tid;
      const uint32_t f = (s < n && row_key(row, s) >= thresh) ? 1u : 0u;
      const uint32_t pos = block_exclusive_scan(f, sm.wsum, &tile_total);
      if (f && base + pos < (uint32_t)k) out[base + pos] = s;
      base += tile_total;
      __syncthreads();
    }
  }
  if (tid == 0 && count) count[q] = k;
}

size_t topk_workspace_bytes(int nq, int max_len, int k) {
  (void)nq;
  (void)max_len;
  (void)k;
  return 0;
}

hipError_t launch_topk(const BatchDev& b, const float* scores, int64_t ld, int k, int32_t* idx,
                       int32_t* count, void* ws, size_t ws_bytes, hipStream_t st) {
  (void)ws;
  (void)ws_bytes;
  if (b.nq == 0) return hipSuccess;
  hipLaunchKernelGGL(topk_row_kernel, dim3(b.nq), dim3(TK_THREADS), 0, st, b, scores, ld, k, idx, count);
  return hipGetLastError();
}

}  // namespace dsa
