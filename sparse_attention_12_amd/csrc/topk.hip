// Top-k selection on gfx950 (concept page "Mistral Large 4", section "Where
// to look": the indexer keeps the best 2,048 positions per query).
//
// The kept set is the first min(k, n) positions under (score descending,
// position ascending), emitted in ascending position order.  Scores are
// mapped to unsigned keys u whose order is the score order (-0.0 = +0.0).
//
// Radix select, ordered throughout so that no sort is ever needed:
//   1. histogram of the top 12 bits of u  ->  bucket d1 holding the k-th key;
//   2. every position whose top 12 bits are >= d1 is copied, in position
//      order, into a candidate list (ordered compaction with block scans);
//   3. two more levels of 10 bits over the candidates of bucket d1 fix the
//      k-th key T exactly; with `need` positions still to take at T,
//   4. one ordered pass keeps u > T, and u == T while fewer than `need`
//      earlier positions with u == T were kept (lower position wins ties).
// Long rows with few queries (decode) split steps 1-2 over many workgroups
// (per-chunk lists, concatenated in chunk order); many rows (prefill) run
// one workgroup per row, which keeps up to 49,152 of a row's scores in
// registers between steps 1 and 2.  If the candidate list would not fit in LDS (for
// instance every score equal), a row-streaming fallback selects with
// 64-bit (u, position) keys and compacts the row itself.
// In the fused decode read, the indexer has already counted step 1's
// histogram while making the scores; it is taken from there after a check
// that its bins sum to the row's length (bins never go negative, so the sum
// is right exactly when the histogram started from zero), and cleared for
// the next call; a histogram that fails the check is recounted here.
#include "dsa_common.h"
#include "kernels.h"

namespace dsa {

constexpr int TK_WAVES = TK_THREADS / 64;
constexpr int TK_FCAP = 12288;          // candidate entries held in LDS
constexpr int TK_LEVEL_BITS = 11;       // fallback levels over 64-bit keys
// First-level histograms are kept in TK_HCOPIES interleaved copies (bin b,
// copy c at word TK_HCOPIES*b + c; lane l adds to copy l % TK_HCOPIES), so
// lanes whose scores share a bin -- the scores crowd into few bins -- mostly
// add to different words.
constexpr int TK_HCOPIES = 4;

// ---------------------------------------------------------------------------
// block-wide helpers (1024 threads; every thread must call them)
// ---------------------------------------------------------------------------
// Inclusive prefix sum over the 64 lanes of a wave with data-parallel
// primitives (DPP lane moves, no LDS round trips): shifts of 1, 2, 4 and 8
// within each row of 16 lanes, then each row adds the total of the rows
// before it (row broadcasts of lanes 15 and 31).  Lanes with no source lane
// receive 0.
__device__ inline uint32_t wave_inclusive_scan(uint32_t x) {
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x111, 0xF, 0xF, false);  // row_shr:1
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x112, 0xF, 0xF, false);  // row_shr:2
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x114, 0xF, 0xF, false);  // row_shr:4
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x118, 0xF, 0xF, false);  // row_shr:8
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x142, 0xA, 0xF, false);  // row_bcast:15 -> rows 1, 3
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x143, 0xC, 0xF, false);  // row_bcast:31 -> rows 2, 3
  return x;
}

__device__ uint32_t block_exclusive_scan(uint32_t v, uint32_t* wsum, uint32_t* total) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const uint32_t x = wave_inclusive_scan(v);
  if (lane == 63) wsum[wave] = x;
  __syncthreads();
  if (wave == 0) {
    const uint32_t s = lane < TK_WAVES ? wsum[lane] : 0u;
    const uint32_t t = wave_inclusive_scan(s);
    if (lane < TK_WAVES) wsum[lane] = t - s;
    if (lane == TK_WAVES - 1) *total = t;
  }
  __syncthreads();
  const uint32_t res = wsum[wave] + x - v;
  __syncthreads();
  return res;
}

struct ScanShared {
  uint32_t wsum[TK_WAVES];
  uint32_t total;
  int digit;
  uint32_t above;
  uint64_t red[TK_WAVES];
};

// Bucket d of hist[0, nbins) with fewer than `need` entries above it and at
// least `need` in d or above (thread 0 covers the highest buckets).
__device__ void find_bucket(const uint32_t* hist, int nbins, uint32_t need, ScanShared& ss, int* digit,
                            uint32_t* above) {
  if (threadIdx.x == 0) {
    ss.digit = 0;
    ss.above = 0;
  }
  const int per = (nbins + TK_THREADS - 1) / TK_THREADS;
  const int hi = nbins - (int)threadIdx.x * per;
  const int lo = max(hi - per, 0);
  uint32_t local = 0;
  for (int b = lo; b < hi; ++b) local += hist[b];
  uint32_t run = block_exclusive_scan(local, ss.wsum, &ss.total);
  for (int b = hi - 1; b >= lo; --b) {
    const uint32_t c = hist[b];
    if (run < need && run + c >= need) {
      ss.digit = b;
      ss.above = run;
    }
    run += c;
  }
  __syncthreads();
  *digit = ss.digit;
  *above = ss.above;
  __syncthreads();
}

// Adds the top-12-bit digits of row[c0, c1) to an LDS histogram.  The
// 16-byte aligned body is read as float4, four per thread in flight, so a
// pass is bandwidth- rather than latency-bound; the unaligned head and tail
// (at most three values each) are read one by one.
__device__ void hist_range(const float* row, int c0, int c1, uint32_t* hist) {
  const int tid = threadIdx.x;
  const uint32_t copy = (uint32_t)tid & (TK_HCOPIES - 1);
  const int mis = (int)(((uintptr_t)(row + c0) >> 2) & 3);
  const int a0 = min(c1, c0 + ((4 - mis) & 3));
  const int nv = (c1 - a0) >> 2;
  const int t0 = a0 + 4 * nv;
  auto add = [&](float x) { atomicAdd(&hist[(score_key(x) >> TK_SHIFT1) * TK_HCOPIES + copy], 1u); };
  if (tid < a0 - c0) add(row[c0 + tid]);
  if (tid < c1 - t0) add(row[t0 + tid]);
  const float4* v = (const float4*)(row + a0);
  for (int i0 = 0; i0 < nv; i0 += 4 * TK_THREADS) {
    float4 x[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int i = i0 + u * TK_THREADS + tid;
      if (i < nv) x[u] = v[i];
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      if (i0 + u * TK_THREADS + tid < nv) {
        add(x[u].x);
        add(x[u].y);
        add(x[u].z);
        add(x[u].w);
      }
    }
  }
}

// 64-bit sum over the workgroup (every thread calls; the result in every
// thread).  red: TK_WAVES words of LDS.
__device__ inline uint64_t block_sum64(uint64_t v, uint64_t* red) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  uint64_t t = 0;
#pragma unroll
  for (int w = 0; w < TK_WAVES; ++w) t += red[w];
  __syncthreads();
  return t;
}

// Takes the indexer's first-level histogram of a row: copies it to hist
// (LDS), clears it in global memory for the next call, and returns whether
// it is the row's histogram (its bins sum to n).  Thread t owns bins
// [4t, 4t + 4).
static_assert(TK_BINS1 == 4 * TK_THREADS, "one uint4 of bins per thread");
__device__ inline bool take_precounted(uint32_t* gh, uint32_t* hist, int n, uint64_t* red) {
  uint4* g4 = (uint4*)gh;
  const uint4 v = g4[threadIdx.x];
  g4[threadIdx.x] = make_uint4(0u, 0u, 0u, 0u);
  *(uint4*)(hist + 4 * threadIdx.x) = v;
  const uint64_t mine = (uint64_t)v.x + v.y + v.z + v.w;
  return block_sum64(mine, red) == (uint64_t)n;
}

// Clears a row's precounted histogram in global memory.
__device__ inline void clear_precounted(uint32_t* gh) {
  ((uint4*)gh)[threadIdx.x] = make_uint4(0u, 0u, 0u, 0u);
}

__device__ inline void hist_copies_zero(uint32_t* hc) {
  for (int i = threadIdx.x; i < TK_BINS1 * TK_HCOPIES; i += TK_THREADS) hc[i] = 0;
}

// hist[b] = sum of the copies of bin b
static_assert(TK_HCOPIES == 4, "the folds below read the copies of a bin as one uint4");
__device__ inline void hist_copies_fold(const uint32_t* hc, uint32_t* hist) {
  for (int b = threadIdx.x; b < TK_BINS1; b += TK_THREADS) {
    const uint4 v = *(const uint4*)(hc + b * TK_HCOPIES);
    hist[b] = v.x + v.y + v.z + v.w;
  }
}

// ---------------------------------------------------------------------------
// finalize from an ordered candidate list held in LDS
// ---------------------------------------------------------------------------
struct ListShared {
  union {
    struct {
      uint32_t ukey[TK_FCAP];
      int32_t pos[TK_FCAP];
    };
    uint32_t hcopies[TK_BINS1 * TK_HCOPIES];  // first-level histogram copies, before the list exists
  };
  uint32_t hist[1 << 10];
  uint32_t lo_min[1 << 10];  // per bin of the first 10-bit level: least and greatest key bits below it
  uint32_t lo_max[1 << 10];
  ScanShared ss;
};
static_assert(2 * TK_FCAP >= TK_BINS1 * TK_HCOPIES, "the histogram copies fit in the list area");
static_assert(TK_FCAP < (1 << 16), "list counts fit the 16-bit fields of a packed scan");

// The list holds, in ascending position order, every position whose top 12
// key bits are >= d1 (`total` entries, `need` of bucket d1 still to take).
// Writes the kept positions in order to out[0, k).
// Two 10-bit levels fix the k-th key T.  The first also records each bin's
// range of the 10 key bits below it: when the bin holding T has one key
// value (tied scores, as integer or FP8 indexer inputs make), T is known
// and the second level is skipped.  The kept entries are those above T and
// the first `need` equal to T: one block scan of the packed per-thread
// counts (above T, equal to T) gives each thread both its tie rank r and
// its first output slot (entries above T before it, plus min(r, need)).
__device__ void finalize_list(ListShared& sm, int total, uint32_t d1, uint32_t need, int k, int32_t* out) {
  const int tid = threadIdx.x;
  uint32_t prefix = d1;
  int plen = TK_BITS1;
  while (plen < 32) {
    const int bits = 10;
    const int shift = 32 - plen - bits;
    const bool range = shift > 0;
    const uint32_t low = (1u << shift) - 1u;
    for (int i = tid; i < (1 << bits); i += TK_THREADS) {
      sm.hist[i] = 0;
      if (range) {
        sm.lo_min[i] = 0xffffffffu;
        sm.lo_max[i] = 0u;
      }
    }
    __syncthreads();
    for (int e = tid; e < total; e += TK_THREADS) {
      const uint32_t u = sm.ukey[e];
      if ((u >> (32 - plen)) == prefix) {
        const uint32_t bin = (u >> shift) & ((1u << bits) - 1);
        atomicAdd(&sm.hist[bin], 1u);
        if (range) {
          atomicMin(&sm.lo_min[bin], u & low);
          atomicMax(&sm.lo_max[bin], u & low);
        }
      }
    }
    __syncthreads();
    int d;
    uint32_t above;
    find_bucket(sm.hist, 1 << bits, need, sm.ss, &d, &above);
    need -= above;
    const uint32_t cnt = sm.hist[d];
    prefix = (prefix << bits) | (uint32_t)d;
    plen += bits;
    if (range && sm.lo_min[d] == sm.lo_max[d]) {
      prefix = (prefix << shift) | sm.lo_min[d];
      plen = 32;
    }
    __syncthreads();
    if (cnt == need) break;
  }
  const int s = 32 - plen;
  // thread t owns the contiguous entries [t*per, (t+1)*per)
  const int per = (total + TK_THREADS - 1) / TK_THREADS;
  const int e0 = min(tid * per, total);
  const int e1 = min(e0 + per, total);
  uint32_t gt = 0, ties = 0;
  for (int e = e0; e < e1; ++e) {
    const uint32_t v = sm.ukey[e] >> s;
    gt += v > prefix ? 1u : 0u;
    ties += v == prefix ? 1u : 0u;
  }
  const uint32_t pre = block_exclusive_scan(gt | (ties << 16), sm.ss.wsum, &sm.ss.total);
  uint32_t tie_rank = pre >> 16;
  uint32_t slot = (pre & 0xffffu) + min(tie_rank, need);
  for (int e = e0; e < e1; ++e) {
    const uint32_t v = sm.ukey[e] >> s;
    bool keep = v > prefix;
    if (v == prefix) keep = tie_rank++ < need;
    if (keep) {
      DSA_CHECK(slot < (uint32_t)k, DBG_TOPK_SLOT);
      if (slot < (uint32_t)k) out[slot] = sm.pos[e];
      ++slot;
    }
  }
}

// ---------------------------------------------------------------------------
// row-streaming fallback (candidate bucket too large for LDS)
// ---------------------------------------------------------------------------
__device__ inline uint64_t row_key(const float* row, int s) { return select_key(score_key(row[s]), s); }

__device__ void select_row_streaming(const float* row, int n, int k, uint32_t d1, uint32_t need, uint32_t* hist,
                                     ScanShared& ss, int32_t* out) {
  const int tid = threadIdx.x;
  uint64_t prefix = d1;
  int plen = TK_BITS1;
  while (plen < 64) {
    const int bits = min(TK_LEVEL_BITS, 64 - plen);
    const int shift = 64 - plen - bits;
    const int nb = 1 << bits;
    for (int i = tid; i < nb; i += TK_THREADS) hist[i] = 0;
    __syncthreads();
    for (int s = tid; s < n; s += TK_THREADS) {
      const uint64_t key = row_key(row, s);
      if ((key >> (64 - plen)) == prefix) atomicAdd(&hist[(key >> shift) & (uint64_t)(nb - 1)], 1u);
    }
    __syncthreads();
    int d;
    uint32_t above;
    find_bucket(hist, nb, need, ss, &d, &above);
    need -= above;
    const uint32_t cnt = hist[d];
    prefix = (prefix << bits) | (uint32_t)d;
    plen += bits;
    __syncthreads();
    if (cnt == need) break;
  }
  const uint64_t thresh = plen >= 64 ? prefix : (prefix << (64 - plen));
  uint32_t base = 0;
  for (int t0 = 0; t0 < n; t0 += TK_THREADS) {
    const int s = t0 + tid;
    const uint32_t f = (s < n && row_key(row, s) >= thresh) ? 1u : 0u;
    const uint32_t p = block_exclusive_scan(f, ss.wsum, &ss.total);
    DSA_CHECK(!f || base + p < (uint32_t)k, DBG_TOPK_SLOT);
    if (f && base + p < (uint32_t)k) out[base + p] = s;
    base += ss.total;
    __syncthreads();
  }
}

// Ordered compaction of row[c0, c1): entries with top-12 key bits >= d1 go
// to (dst_key, dst_pos) in position order.  Returns the count (all threads).
// Thread t takes the 16 consecutive values [16t, 16t + 16) of each
// 16,384-value stretch (four float4 loads when row + c0 is 16-byte
// aligned), so one block scan orders a whole stretch.
constexpr int TK_RUN = 16;
constexpr int TK_STRETCH = TK_RUN * TK_THREADS;

__device__ uint32_t compact_chunk(const float* row, int c0, int c1, uint32_t d1, uint32_t* dst_key,
                                  int32_t* dst_pos, uint32_t cap, ScanShared& ss) {
  const int tid = threadIdx.x;
  const bool vec = (((uintptr_t)(row + c0)) & 15) == 0;
  uint32_t base = 0;
  for (int t0 = c0; t0 < c1; t0 += TK_STRETCH) {
    const int s0 = t0 + tid * TK_RUN;
    uint32_t u[TK_RUN];
    if (vec && s0 + TK_RUN <= c1) {
#pragma unroll
      for (int i = 0; i < TK_RUN / 4; ++i) {
        const float4 x = *(const float4*)(row + s0 + 4 * i);
        u[4 * i + 0] = score_key(x.x);
        u[4 * i + 1] = score_key(x.y);
        u[4 * i + 2] = score_key(x.z);
        u[4 * i + 3] = score_key(x.w);
      }
    } else {
#pragma unroll
      for (int j = 0; j < TK_RUN; ++j) u[j] = s0 + j < c1 ? score_key(row[s0 + j]) : 0u;
    }
    uint32_t f = 0;
#pragma unroll
    for (int j = 0; j < TK_RUN; ++j)
      if (s0 + j < c1 && (u[j] >> TK_SHIFT1) >= d1) f |= 1u << j;
    uint32_t p = block_exclusive_scan(__builtin_popcount(f), ss.wsum, &ss.total);
#pragma unroll
    for (int j = 0; j < TK_RUN; ++j) {
      if (f & (1u << j)) {
        const uint32_t slot = base + p++;
        if (slot < cap) {
          dst_key[slot] = u[j];
          dst_pos[slot] = s0 + j;
        }
      }
    }
    base += ss.total;
    __syncthreads();
  }
  return base;
}

// ---------------------------------------------------------------------------
// one workgroup per row
// ---------------------------------------------------------------------------
struct RowShared {
  uint32_t hist1[TK_BINS1];
  ListShared list;
};

// Rows of n <= k keep every position.
__device__ inline void keep_all(int n, int k, int32_t* out) {
  for (int j = threadIdx.x; j < k; j += TK_THREADS) out[j] = j < n ? j : -1;
}

// One workgroup per row, its first NST * 16,384 scores held in registers:
// thread t loads the runs [16t, 16t + 16) of each such 16,384-score stretch
// once, as keys, and the histogram and the ordered compaction both read
// them there, so that part of the row crosses HBM once.  The rest of a
// longer row (beyond what 128 registers per thread hold) is read twice,
// as in the two-pass path.
// With hist_pre, the row's first-level histogram comes precounted (and is
// cleared for the next call).
template <int NST>
__global__ __launch_bounds__(TK_THREADS) void topk_row_reg_kernel(BatchDev b, const float* __restrict__ scores,
                                                                 int64_t ld, int k, int32_t* __restrict__ idx,
                                                                 int32_t* __restrict__ count,
                                                                 uint32_t* __restrict__ hist_pre) {
  __shared__ __attribute__((aligned(16))) RowShared sm;
  const int q = blockIdx.x;
  const int tid = threadIdx.x;
  const QueryRange r = query_range(b, q);
  const int n = r.n;
  int32_t* out = idx + (int64_t)q * k;
  const float* row = scores + (int64_t)q * ld;
  uint32_t* gh = hist_pre ? hist_pre + (int64_t)q * TK_BINS1 : nullptr;
  if (n <= k) {
    keep_all(n, k, out);
    if (gh) clear_precounted(gh);
  } else {
    constexpr int REG = NST * TK_STRETCH;
    uint32_t* hc = sm.list.hcopies;
    const bool counted = gh && take_precounted(gh, sm.hist1, n, sm.list.ss.red);
    DSA_CHECK(!gh || counted, DBG_HIST_RECOUNT);
    if (!counted) hist_copies_zero(hc);
    // keys of this thread's runs (positions at or past n are never counted)
    uint32_t u[NST][TK_RUN];
    const bool vec = (((uintptr_t)row) & 15) == 0;
#pragma unroll
    for (int st = 0; st < NST; ++st) {
      const int s0 = st * TK_STRETCH + tid * TK_RUN;
      if (vec && s0 + TK_RUN <= n) {
#pragma unroll
        for (int i = 0; i < TK_RUN / 4; ++i) {
          const float4 x = *(const float4*)(row + s0 + 4 * i);
          u[st][4 * i + 0] = score_key(x.x);
          u[st][4 * i + 1] = score_key(x.y);
          u[st][4 * i + 2] = score_key(x.z);
          u[st][4 * i + 3] = score_key(x.w);
        }
      } else {
#pragma unroll
        for (int j = 0; j < TK_RUN; ++j) u[st][j] = s0 + j < n ? score_key(row[s0 + j]) : 0u;
      }
    }
    __syncthreads();  // copies cleared (or the precounted histogram in place)
    if (!counted) {
      const uint32_t copy = (uint32_t)tid & (TK_HCOPIES - 1);
#pragma unroll
      for (int st = 0; st < NST; ++st) {
        const int s0 = st * TK_STRETCH + tid * TK_RUN;
#pragma unroll
        for (int j = 0; j < TK_RUN; ++j)
          if (s0 + j < n) atomicAdd(&hc[(u[st][j] >> TK_SHIFT1) * TK_HCOPIES + copy], 1u);
      }
      if (n > REG) hist_range(row, REG, n, hc);
      __syncthreads();
      hist_copies_fold(hc, sm.hist1);
      __syncthreads();
    }
    int d1;
    uint32_t above;
    find_bucket(sm.hist1, TK_BINS1, (uint32_t)k, sm.list.ss, &d1, &above);
    const uint32_t need = (uint32_t)k - above;
    const uint32_t total = above + sm.hist1[d1];
    if (total <= (uint32_t)TK_FCAP) {
      // ordered compaction of the keys with top 12 bits >= d1: every
      // stretch's per-thread count (at most 16; at most 16,384 per stretch)
      // in a 16-bit field, two stretches to a word, so one block scan
      // orders two stretches
      constexpr int NW = (NST + 1) / 2;
      uint32_t f[NST], cw[NW], pw[NW], tw[NW];
#pragma unroll
      for (int w = 0; w < NW; ++w) cw[w] = 0;
#pragma unroll
      for (int st = 0; st < NST; ++st) {
        const int s0 = st * TK_STRETCH + tid * TK_RUN;
        f[st] = 0;
#pragma unroll
        for (int j = 0; j < TK_RUN; ++j)
          if (s0 + j < n && (u[st][j] >> TK_SHIFT1) >= (uint32_t)d1) f[st] |= 1u << j;
        cw[st >> 1] |= (uint32_t)__builtin_popcount(f[st]) << (16 * (st & 1));
      }
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        pw[w] = block_exclusive_scan(cw[w], sm.list.ss.wsum, &sm.list.ss.total);
        tw[w] = sm.list.ss.total;
      }
      uint32_t base = 0;
#pragma unroll
      for (int st = 0; st < NST; ++st) {
        const int s0 = st * TK_STRETCH + tid * TK_RUN;
        const int sh = 16 * (st & 1);
        uint32_t slot = base + ((pw[st >> 1] >> sh) & 0xffffu);
#pragma unroll
        for (int j = 0; j < TK_RUN; ++j) {
          if (f[st] & (1u << j)) {
            DSA_CHECK(slot < (uint32_t)TK_FCAP, DBG_TOPK_SLOT);
            if (slot < (uint32_t)TK_FCAP) {
              sm.list.ukey[slot] = u[st][j];
              sm.list.pos[slot] = s0 + j;
            }
            ++slot;
          }
        }
        base += (tw[st >> 1] >> sh) & 0xffffu;
      }
      __syncthreads();
      if (n > REG) {
        compact_chunk(row, REG, n, (uint32_t)d1, sm.list.ukey + base, sm.list.pos + base, TK_FCAP - base, sm.list.ss);
        __syncthreads();
      }
      finalize_list(sm.list, (int)total, (uint32_t)d1, need, k, out);
    } else {
      select_row_streaming(row, n, k, (uint32_t)d1, need, sm.hist1, sm.list.ss, out);
    }
  }
  if (tid == 0 && count) count[q] = min(n, k);
}

// ---------------------------------------------------------------------------
// split path: hist -> per-chunk ordered lists -> finalize
// ---------------------------------------------------------------------------
struct SplitWs {
  uint32_t* hist;     // [nq][4096]
  uint32_t* bucket;   // [nq][4]: threshold bucket d1, entries above it, entries in it
  uint32_t* cnt;      // [nq][nchunk]
  uint32_t* lkey;     // [nq][nchunk * TK_CHUNK]
  int32_t* lpos;      // [nq][nchunk * TK_CHUNK]
  int nchunk;
};

__global__ __launch_bounds__(TK_THREADS) void topk_hist_kernel(BatchDev b, const float* __restrict__ scores,
                                                               int64_t ld, int k, SplitWs ws) {
  __shared__ __attribute__((aligned(16))) uint32_t hist[TK_BINS1 * TK_HCOPIES];
  const int q = blockIdx.y;
  const QueryRange r = query_range(b, q);
  const int c0 = blockIdx.x * TK_CHUNK;
  if (r.n <= k || c0 >= r.n) return;
  const int c1 = min(c0 + TK_CHUNK, r.n);
  const int tid = threadIdx.x;
  hist_copies_zero(hist);
  __syncthreads();
  const float* row = scores + (int64_t)q * ld;
  hist_range(row, c0, c1, hist);
  __syncthreads();
  uint32_t* gh = ws.hist + (int64_t)q * TK_BINS1;
  for (int i = tid; i < TK_BINS1; i += TK_THREADS) {
    const uint4 v = *(const uint4*)(hist + i * TK_HCOPIES);
    const uint32_t s = v.x + v.y + v.z + v.w;
    if (s) atomicAdd(&gh[i], s);
  }
}

__global__ __launch_bounds__(TK_THREADS) void topk_gather_kernel(BatchDev b, const float* __restrict__ scores,
                                                                 int64_t ld, int k, SplitWs ws) {
  __shared__ __attribute__((aligned(16))) uint32_t hist[TK_BINS1];
  __shared__ ScanShared ss;
  const int q = blockIdx.y;
  const int c = blockIdx.x;
  const QueryRange r = query_range(b, q);
  const int c0 = c * TK_CHUNK;
  if (r.n <= k || c0 >= r.n) return;
  const int c1 = min(c0 + TK_CHUNK, r.n);
  const int tid = threadIdx.x;
  // this thread's GR consecutive scores, read before the histogram so the
  // two round trips overlap
  constexpr int GR = TK_CHUNK / TK_THREADS;
  static_assert(GR % 4 == 0, "whole float4 runs");
  const float* row = scores + (int64_t)q * ld;
  const int s0 = c0 + tid * GR;
  uint32_t u[GR];
  if ((((uintptr_t)(row + s0)) & 15) == 0 && s0 + GR <= c1) {
#pragma unroll
    for (int i = 0; i < GR / 4; ++i) {
      const float4 x = *(const float4*)(row + s0 + 4 * i);
      u[4 * i + 0] = score_key(x.x);
      u[4 * i + 1] = score_key(x.y);
      u[4 * i + 2] = score_key(x.z);
      u[4 * i + 3] = score_key(x.w);
    }
  } else {
#pragma unroll
    for (int j = 0; j < GR; ++j) u[j] = s0 + j < c1 ? score_key(row[s0 + j]) : 0u;
  }
  // the row's histogram (counted by the indexer or by topk_hist_kernel);
  // one that does not sum to the row's length did not start from zero: the
  // row is recounted here (only after a call that left it uncleared)
  const uint32_t* gh = ws.hist + (int64_t)q * TK_BINS1;
  const uint4 hv = ((const uint4*)gh)[tid];
  *(uint4*)(hist + 4 * tid) = hv;
  if (block_sum64((uint64_t)hv.x + hv.y + hv.z + hv.w, ss.red) != (uint64_t)r.n) {
    DSA_CHECK(false, DBG_HIST_RECOUNT);
    *(uint4*)(hist + 4 * tid) = make_uint4(0u, 0u, 0u, 0u);
    __syncthreads();
    for (int i = tid; i < r.n; i += TK_THREADS) atomicAdd(&hist[score_key(row[i]) >> TK_SHIFT1], 1u);
  }
  __syncthreads();
  int d1;
  uint32_t above;
  find_bucket(hist, TK_BINS1, (uint32_t)k, ss, &d1, &above);
  // ordered compaction of the chunk: one block scan
  uint32_t f = 0;
#pragma unroll
  for (int j = 0; j < GR; ++j)
    if (s0 + j < c1 && (u[j] >> TK_SHIFT1) >= (uint32_t)d1) f |= 1u << j;
  uint32_t slot = block_exclusive_scan(__builtin_popcount(f), ss.wsum, &ss.total);
  // every chunk finds the same bucket; the first publishes it for the final pass
  if (c == 0 && tid == 0) {
    ws.bucket[q * 4 + 0] = (uint32_t)d1;
    ws.bucket[q * 4 + 1] = above;
    ws.bucket[q * 4 + 2] = hist[d1];
  }
  const int64_t lbase = ((int64_t)q * ws.nchunk + c) * TK_CHUNK;
#pragma unroll
  for (int j = 0; j < GR; ++j) {
    if (f & (1u << j)) {
      DSA_CHECK(slot < (uint32_t)TK_CHUNK, DBG_LIST);
      ws.lkey[lbase + slot] = u[j];
      ws.lpos[lbase + slot] = s0 + j;
      ++slot;
    }
  }
  if (tid == 0) ws.cnt[(int64_t)q * ws.nchunk + c] = ss.total;
}

struct FinalShared {
  uint32_t hist1[TK_BINS1];
  uint32_t off[TK_THREADS];
  ListShared list;
};

// Copies the concatenated chunk lists (offsets in off[0..nch), total
// entries) into the LDS list.  Entry e = tid + i * TK_THREADS for i < PER,
// so PER * TK_THREADS must cover total; the caller takes an instance with
// half the rounds when it does, so short lists issue fewer loads and
// searches without a branch per round.
template <int PER>
__device__ __forceinline__ void copy_lists(ListShared& lst, const uint32_t* off, int nch, uint32_t total,
                                           const SplitWs& ws, int64_t lq) {
  const int tid = threadIdx.x;
  // entry e = tid + i * TK_THREADS: the lanes of a wave copy consecutive
  // entries, so each of its loads reads one or two cache lines, and every
  // load of a thread is issued before the first is waited for.  An entry's
  // chunk (the last chunk whose offset is <= e) comes from a binary search
  // over the offsets; a thread's searches step together, and the lanes of a
  // wave, holding neighbouring entries, mostly read the same offsets.
  // Entries past the total load entry 0 of chunk 0 and are not stored.
  int lo[PER], hi[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    lo[i] = 0;
    hi[i] = nch - 1;
  }
  // (branch-free: with lo == hi the step reads off[lo] <= e and keeps lo,
  // so every search takes ceil(log2(nch)) steps and each step's reads go
  // out together)
  for (int it = 0; (1 << it) < nch; ++it) {
    uint32_t v[PER];
    int mid[PER];
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      mid[i] = (lo[i] + hi[i] + 1) >> 1;
      v[i] = off[mid[i]];
    }
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const bool le = v[i] <= (uint32_t)(tid + i * TK_THREADS);
      lo[i] = le ? mid[i] : lo[i];
      hi[i] = le ? hi[i] : mid[i] - 1;
    }
  }
  uint32_t oc[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) oc[i] = off[lo[i]];
  uint32_t kv[PER];
  int32_t pv[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const uint32_t e = (uint32_t)(tid + i * TK_THREADS);
    const int64_t src = e < total ? lq + (int64_t)lo[i] * TK_CHUNK + (e - oc[i]) : lq;
    kv[i] = ws.lkey[src];
    pv[i] = ws.lpos[src];
  }
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const uint32_t e = (uint32_t)(tid + i * TK_THREADS);
    if (e < total) {
      lst.ukey[e] = kv[i];
      lst.pos[e] = pv[i];
    }
  }
}

__global__ __launch_bounds__(TK_THREADS) void topk_final_kernel(BatchDev b, const float* __restrict__ scores,
                                                                int64_t ld, int k, int32_t* __restrict__ idx,
                                                                int32_t* __restrict__ count, SplitWs ws) {
  __shared__ FinalShared sm;
  const int q = blockIdx.x;
  const int tid = threadIdx.x;
  const QueryRange r = query_range(b, q);
  const int n = r.n;
  int32_t* out = idx + (int64_t)q * k;
  // every gather workgroup of this row is done with its histogram: clear
  // it for the next call
  clear_precounted(ws.hist + (int64_t)q * TK_BINS1);
  if (n <= k) {
    for (int j = tid; j < k; j += TK_THREADS) out[j] = j < n ? j : -1;
    if (tid == 0 && count) count[q] = n;
    return;
  }
  // the threshold bucket (found by the gather pass) and the per-chunk list
  // lengths are read together
  const int nch = (n + TK_CHUNK - 1) / TK_CHUNK;
  const uint32_t mine = tid < nch ? ws.cnt[(int64_t)q * ws.nchunk + tid] : 0u;
  const int d1 = (int)ws.bucket[q * 4 + 0];
  const uint32_t above = ws.bucket[q * 4 + 1];
  const uint32_t need = (uint32_t)k - above;
  const uint32_t total = above + ws.bucket[q * 4 + 2];
  if (total <= (uint32_t)TK_FCAP) {
    // concatenate the per-chunk lists in chunk (= position) order: offsets
    // by a block scan, then every entry copied in one parallel pass with all
    // of a thread's reads in flight together
    const uint32_t o = block_exclusive_scan(mine, sm.list.ss.wsum, &sm.list.ss.total);
    DSA_CHECK(sm.list.ss.total == total, DBG_LIST);
    if (tid < nch) sm.off[tid] = o;
    __syncthreads();
    const int64_t lq = (int64_t)q * ws.nchunk * TK_CHUNK;
    constexpr int PER_MAX = (TK_FCAP + TK_THREADS - 1) / TK_THREADS;
    if (total <= (uint32_t)(PER_MAX / 2 * TK_THREADS))
      copy_lists<PER_MAX / 2>(sm.list, sm.off, nch, total, ws, lq);
    else
      copy_lists<PER_MAX>(sm.list, sm.off, nch, total, ws, lq);
    __syncthreads();
    finalize_list(sm.list, (int)total, (uint32_t)d1, need, k, out);
  } else {
    select_row_streaming(scores + (int64_t)q * ld, n, k, (uint32_t)d1, need, sm.hist1, sm.list.ss, out);
  }
  if (tid == 0 && count) count[q] = k;
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------
#ifdef DSA_DEBUG
DSA_DEBUG_READER(debug_flags_topk)
#endif

static SplitWs split_ws(int nq, int max_len, char* base) {
  const TopkLayout t = topk_layout(nq, max_len);
  SplitWs ws;
  ws.hist = (uint32_t*)(base + t.hist);
  ws.bucket = (uint32_t*)(base + t.bucket);
  ws.cnt = (uint32_t*)(base + t.cnt);
  ws.lkey = (uint32_t*)(base + t.lkey);
  ws.lpos = (int32_t*)(base + t.lpos);
  ws.nchunk = t.nchunk;
  return ws;
}

hipError_t launch_topk(const BatchDev& b, const float* scores, int64_t ld, int k, int32_t* idx,
                       int32_t* count, void* wsp, size_t ws_bytes, hipStream_t st, uint32_t* hist_pre) {
  if (b.nq == 0) return hipSuccess;
  if (!topk_use_split(b.nq, b.max_len)) {
    // as many 16,384-score stretches in registers as the row needs, at most 3
    const int nst = (b.max_len + TK_STRETCH - 1) / TK_STRETCH;
    if (nst <= 1)
      hipLaunchKernelGGL(topk_row_reg_kernel<1>, dim3(b.nq), dim3(TK_THREADS), 0, st, b, scores, ld, k, idx, count,
                         hist_pre);
    else if (nst == 2)
      hipLaunchKernelGGL(topk_row_reg_kernel<2>, dim3(b.nq), dim3(TK_THREADS), 0, st, b, scores, ld, k, idx, count,
                         hist_pre);
    else
      hipLaunchKernelGGL(topk_row_reg_kernel<3>, dim3(b.nq), dim3(TK_THREADS), 0, st, b, scores, ld, k, idx, count,
                         hist_pre);
    return hipGetLastError();
  }
  if (wsp == nullptr || ws_bytes < topk_layout(b.nq, b.max_len).bytes) return hipErrorInvalidValue;
  SplitWs ws = split_ws(b.nq, b.max_len, (char*)wsp);
  dim3 grid(ws.nchunk, b.nq);
  if (hist_pre != nullptr) {
    ws.hist = hist_pre;   // counted by the indexer
  } else {
    ZeroSpans z;
    z.s[0] = ZeroSpan{ws.hist, TK_BINS1, TK_BINS1};
    z.s[1] = ZeroSpan{nullptr, 0, 0};
    hipError_t e = launch_zero(z, b.nq, st);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(topk_hist_kernel, grid, dim3(TK_THREADS), 0, st, b, scores, ld, k, ws);
  }
  hipLaunchKernelGGL(topk_gather_kernel, grid, dim3(TK_THREADS), 0, st, b, scores, ld, k, ws);
  hipLaunchKernelGGL(topk_final_kernel, dim3(b.nq), dim3(TK_THREADS), 0, st, b, scores, ld, k, idx, count, ws);
  return hipGetLastError();
}

}  // namespace dsa
