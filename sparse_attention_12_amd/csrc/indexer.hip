// DSA indexer scores on gfx950.
//
// Score of position s for query q (concept page "Mistral Large 4", sections
// "Where to look" and "Sparse attention"; the 32 x 128 cost per scored
// position fixes the shapes):
//   I[q][s] = sum_{h<32} w[q][h] * max(0, qI[q][h][:] . kI[s][:])
//
// Decode (one query per sequence) is a stream over the query's keys: heads
// sit on the M axis of 16x16x32 MFMA tiles and keys on N, so each lane ends
// with 8 of the 32 head dot products of one key; the ReLU and the weighted
// head sum stay in registers and finish with two cross-lane adds.  Decode
// batches of up to IDX_BAL_MAXQ queries can also count every score they
// store into a per-query histogram of its top TK_BITS1 key bits: the
// top-k's first radix level, built where the scores are made, so the
// selection need not read them a first time to count them.
//
// Prefill (many queries per sequence) is a blocked product: a workgroup
// keeps 32 queries' indexer rows in registers (4 per wave) and streams key
// tiles through LDS, so each key tile read from L2 feeds the block's queries
// of that sequence.
#include "dsa_common.h"
#include "kernels.h"

namespace dsa {

// Zeroes query q's words of every span (see ZeroSpans in kernels.h).
__global__ __launch_bounds__(256) void zero_spans_kernel(ZeroSpans z) {
  const int q = blockIdx.x;
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    if (z.s[s].base == nullptr) continue;
    uint32_t* p = z.s[s].base + (int64_t)q * z.s[s].stride;
    for (int i = threadIdx.x; i < z.s[s].count; i += 256) p[i] = 0u;
  }
}

// Adds a stored score to the workgroup's LDS histogram (bin: the score's
// top TK_BITS1 order-preserving key bits, as the top-k reads them).
template <bool HIST>
__device__ __forceinline__ void count_score(uint32_t* lh, float x) {
  if (HIST) atomicAdd(&lh[score_key(x) >> TK_SHIFT1], 1u);
}

// ---------------------------------------------------------------------------
// decode, bf16
// ---------------------------------------------------------------------------
// v_mfma_f32_16x16x32_bf16 with 16 heads on M (two blocks for 32 heads), 16
// keys on N and the 128-wide contraction in four steps of 32.  Lane
// (c = l%16, g = l/16) loads, for contraction step s, the 16 bytes at
// s*64 + g*16 of key c, so one load instruction covers 64 contiguous bytes
// of each of 16 keys -- a shape that streams at full HBM rate, unlike 32
// keys x 32 bytes.  A step of 32 keys is two such key blocks.
constexpr int IDX_DEC_THREADS = 256;
constexpr int IDX_DEC_WAVES = IDX_DEC_THREADS / 64;
constexpr int IDX_DEC_STEP = 32;       // keys per pipeline stage and wave

struct KeyTile {
  u32x4 v[8];  // [key block kb][contraction step s] at v[kb*4 + s]
};

// Scores of query q's keys [base, end): the four waves of the workgroup
// take interleaved 32-key steps, each wave keeping four steps of loads in
// flight.  Waves are independent (no barriers); with HIST every stored
// score is also counted into the LDS histogram lh.
template <bool HIST>
__device__ __forceinline__ void idx_decode_range(const BatchDev& b, const uint16_t* __restrict__ qI,
                                                 const float* __restrict__ w, const uint16_t* __restrict__ kI,
                                                 float* __restrict__ scores, int64_t ld, int q, int64_t row0,
                                                 int base, int end, uint32_t* lh) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int c16 = lane & 15;  // A row (head within block) / B column (key within block)
  const int g = lane >> 4;    // which 8 of each 32 contraction slots
  int k0 = base + wave * IDX_DEC_STEP;
  if (k0 >= end) return;

  // A operand: head hb*16 + c16, contraction slots s*32 + 8g + [0,8).
  bf16x8 a[2][4];
#pragma unroll
  for (int hb = 0; hb < 2; ++hb) {
    const uint16_t* qrow = qI + ((int64_t)q * HI + hb * 16 + c16) * DI + g * 8;
#pragma unroll
    for (int st = 0; st < 4; ++st) a[hb][st] = as_bf16x8(load16(qrow + st * 32));
  }
  // Accumulator register i of head block hb holds head hb*16 + 4g + i.
  float wr[2][4];
#pragma unroll
  for (int hb = 0; hb < 2; ++hb)
#pragma unroll
    for (int i = 0; i < 4; ++i) wr[hb][i] = w[(int64_t)q * HI + hb * 16 + 4 * g + i];

  const uint16_t* kb = kI + row0 * DI + g * 8;
  float* out = scores + (int64_t)q * ld;
  const int last = end - 1;
  constexpr int WSTEP = IDX_DEC_WAVES * IDX_DEC_STEP;

  // Keys past the range end re-read its last row (a cache hit), so every
  // load is unconditional and four stages stay in flight.  Plain (temporal)
  // loads: the non-temporal hint measured 3-12% slower on long and ragged
  // batches.
  auto load = [&](KeyTile& kt, int k) {
#pragma unroll
    for (int kb2 = 0; kb2 < 2; ++kb2) {
      const uint16_t* p = kb + (int64_t)min(k + kb2 * 16 + c16, last) * DI;
#pragma unroll
      for (int st = 0; st < 4; ++st) kt.v[kb2 * 4 + st] = load16(p + st * 32);
    }
  };
  // The two key blocks' sums end up in every lane group, so lane group kb
  // stores block kb: one store instruction writes the step's 32 scores, a
  // whole 128-byte line (two 64-byte half-line stores cost the decode batch
  // of four 2^20-position sequences 14% of its time).
  auto score = [&](const KeyTile& kt, int k) {
    float part[2];
#pragma unroll
    for (int kb2 = 0; kb2 < 2; ++kb2) {
      f32x4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int st = 0; st < 4; ++st) {
        const bf16x8 bk = as_bf16x8(kt.v[kb2 * 4 + st]);
        acc0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[0][st], bk, acc0, 0, 0, 0);
        acc1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[1][st], bk, acc1, 0, 0, 0);
      }
      float x = 0.0f;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        x = fmaf(wr[0][i], relu(acc0[i]), x);
        x = fmaf(wr[1][i], relu(acc1[i]), x);
      }
      part[kb2] = rows4_sum(x);
    }
    const int key = k + g * 16 + c16;
    if (g < 2 && key < end) {
      const float x = g == 0 ? part[0] : part[1];
      DSA_CHECK(key < ld, DBG_SCORE_COL);
      out[key] = x;
      count_score<HIST>(lh, x);
    }
  };

  KeyTile t0, t1, t2, t3;
  load(t0, k0);
  load(t1, k0 + WSTEP);
  load(t2, k0 + 2 * WSTEP);
  while (true) {
    load(t3, k0 + 3 * WSTEP);
    score(t0, k0);
    if (k0 + WSTEP >= end) break;
    load(t0, k0 + 4 * WSTEP);
    score(t1, k0 + WSTEP);
    if (k0 + 2 * WSTEP >= end) break;
    load(t1, k0 + 5 * WSTEP);
    score(t2, k0 + 2 * WSTEP);
    if (k0 + 3 * WSTEP >= end) break;
    load(t2, k0 + 6 * WSTEP);
    score(t3, k0 + 3 * WSTEP);
    k0 += 4 * WSTEP;
    if (k0 >= end) break;
  }
}

// ---------------------------------------------------------------------------
// decode, fp8 (OCP E4M3 queries and keys, the pages' indexer storage)
// ---------------------------------------------------------------------------
// v_mfma_f32_16x16x128_f8f6f4: 16 heads on M (two blocks for 32 heads), 16
// keys on N, the whole 128-wide contraction in one product.  Lane (c, g)
// holds 32 operand bytes; its contraction slots are taken as key bytes
// [16g, 16g+16) and [64+16g, 64+16g+16) (the query uses the same slots), so
// each load instruction reads 64 contiguous bytes of each of 16 keys.
constexpr int IDX8_STEP = 64;  // keys per pipeline stage and wave (4 key blocks)

struct KeyTile8 {
  u32x4 v[8];  // [key block kb][half] at v[kb*2 + half]
};

__device__ __forceinline__ i32x8 cat32(u32x4 lo, u32x4 hi) {
  return __builtin_bit_cast(i32x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

template <bool HIST>
__device__ __forceinline__ void idx_decode_range_f8(const BatchDev& b, const uint8_t* __restrict__ qI,
                                                    const float* __restrict__ w, const uint8_t* __restrict__ kI,
                                                    float* __restrict__ scores, int64_t ld, int q, int64_t row0,
                                                    int base, int end, uint32_t* lh) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int c16 = lane & 15;
  const int g = lane >> 4;
  int k0 = base + wave * IDX8_STEP;
  if (k0 >= end) return;
  i32x8 a[2];
#pragma unroll
  for (int hb = 0; hb < 2; ++hb) {
    const uint8_t* qrow = qI + ((int64_t)q * HI + hb * 16 + c16) * DI;
    a[hb] = cat32(load16(qrow + 16 * g), load16(qrow + 64 + 16 * g));
  }
  float wr[2][4];
#pragma unroll
  for (int hb = 0; hb < 2; ++hb)
#pragma unroll
    for (int i = 0; i < 4; ++i) wr[hb][i] = w[(int64_t)q * HI + hb * 16 + 4 * g + i];

  const uint8_t* kb = kI + row0 * DI + 16 * g;
  float* out = scores + (int64_t)q * ld;
  const int last = end - 1;
  constexpr int WSTEP = IDX_DEC_WAVES * IDX8_STEP;
  auto load = [&](KeyTile8& kt, int k) {
#pragma unroll
    for (int kb4 = 0; kb4 < 4; ++kb4) {
      const uint8_t* p = kb + (int64_t)min(k + kb4 * 16 + c16, last) * DI;
      kt.v[kb4 * 2 + 0] = load16(p);
      kt.v[kb4 * 2 + 1] = load16(p + 64);
    }
  };
  // lane group kb stores key block kb: one store instruction writes the
  // step's 64 scores (two whole 128-byte lines)
  auto score = [&](const KeyTile8& kt, int k) {
    float part[4];
#pragma unroll
    for (int kb4 = 0; kb4 < 4; ++kb4) {
      const i32x8 bk = cat32(kt.v[kb4 * 2], kt.v[kb4 * 2 + 1]);
      const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
      // format 0 = FP8 E4M3 for both operands, no block scaling
      const f32x4 acc0 = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a[0], bk, zero, 0, 0, 0, 0, 0, 0);
      const f32x4 acc1 = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a[1], bk, zero, 0, 0, 0, 0, 0, 0);
      float x = 0.0f;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        x = fmaf(wr[0][i], relu(acc0[i]), x);
        x = fmaf(wr[1][i], relu(acc1[i]), x);
      }
      part[kb4] = rows4_sum(x);
    }
    const int key = k + g * 16 + c16;
    if (key < end) {
      const float x = g == 0 ? part[0] : (g == 1 ? part[1] : (g == 2 ? part[2] : part[3]));
      DSA_CHECK(key < ld, DBG_SCORE_COL);
      out[key] = x;
      count_score<HIST>(lh, x);
    }
  };

  KeyTile8 t0, t1, t2, t3;
  load(t0, k0);
  load(t1, k0 + WSTEP);
  load(t2, k0 + 2 * WSTEP);
  while (true) {
    load(t3, k0 + 3 * WSTEP);
    score(t0, k0);
    if (k0 + WSTEP >= end) break;
    load(t0, k0 + 4 * WSTEP);
    score(t1, k0 + WSTEP);
    if (k0 + 2 * WSTEP >= end) break;
    load(t1, k0 + 5 * WSTEP);
    score(t2, k0 + 2 * WSTEP);
    if (k0 + 3 * WSTEP >= end) break;
    load(t2, k0 + 6 * WSTEP);
    score(t3, k0 + 3 * WSTEP);
    k0 += 4 * WSTEP;
    if (k0 >= end) break;
  }
}

// Scores of keys [base, end) of query q in the given storage.
template <bool FP8, bool HIST>
__device__ __forceinline__ void idx_decode_any(const BatchDev& b, const void* qI, const float* w, const void* kI,
                                               float* scores, int64_t ld, int q, int64_t row0, int base, int end,
                                               uint32_t* lh) {
  if (FP8)
    idx_decode_range_f8<HIST>(b, (const uint8_t*)qI, w, (const uint8_t*)kI, scores, ld, q, row0, base, end, lh);
  else
    idx_decode_range<HIST>(b, (const uint16_t*)qI, w, (const uint16_t*)kI, scores, ld, q, row0, base, end, lh);
}

// Grid (chunks, queries): workgroup (c, q) scores keys [c*chunk, (c+1)*chunk)
// of query q.  Used for batches of many queries.
template <bool FP8>
__device__ __forceinline__ void idx_decode_chunked(BatchDev b, const void* __restrict__ qI, const float* __restrict__ w,
                                                   const void* __restrict__ kI, float* __restrict__ scores,
                                                   int64_t ld, int chunk) {
  const int q = blockIdx.y;
  const QueryRange r = query_range(b, q);
  const int base = blockIdx.x * chunk;
  if (base >= r.n) return;
  idx_decode_any<FP8, false>(b, qI, w, kI, scores, ld, q, r.row0, base, min(base + chunk, r.n), nullptr);
}

// Balanced decode: the batch's keys, laid end to end in query order, are
// cut into gridDim.x equal ranges, one per workgroup, so ragged lengths
// cost no imbalance and every workgroup streams a long range.  Each
// workgroup first forms the prefix sums of the candidate counts itself.
// With HIST, a workgroup counts its scores of each query into an LDS
// histogram and adds the non-zero bins to hist[q] when it moves past the
// query (a handful of global atomics per query and workgroup: the scores
// crowd into few bins).
template <bool FP8, bool HIST>
__device__ __forceinline__ void idx_decode_bal(BatchDev b, const void* __restrict__ qI, const float* __restrict__ w,
                                               const void* __restrict__ kI, float* __restrict__ scores, int64_t ld,
                                               uint32_t* __restrict__ hist) {
  __shared__ int64_t pre[IDX_BAL_MAXQ + 1];
  __shared__ int64_t wtot[IDX_DEC_WAVES];
  __shared__ uint32_t lh[HIST ? TK_BINS1 : 1];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  if (HIST)
    for (int i = tid; i < TK_BINS1; i += IDX_DEC_THREADS) lh[i] = 0u;
  // candidate counts -> exclusive prefix sums in pre[0..nq]
  constexpr int PER = IDX_BAL_MAXQ / IDX_DEC_THREADS;
  int64_t cnt[PER];
  int64_t mine = 0;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int q = tid * PER + i;
    cnt[i] = q < b.nq ? (int64_t)query_range(b, q).n : 0;
    mine += cnt[i];
  }
  int64_t x = mine;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int64_t y = __shfl_up(x, o);
    if (lane >= o) x += y;
  }
  if (lane == 63) wtot[wave] = x;
  __syncthreads();
  int64_t before = 0;
  for (int v = 0; v < wave; ++v) before += wtot[v];
  int64_t run = before + x - mine;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int q = tid * PER + i;
    if (q <= b.nq) pre[q] = run;
    run += cnt[i];
  }
  __syncthreads();
  const int64_t T = pre[b.nq];
  const int64_t lo = T * blockIdx.x / gridDim.x;
  const int64_t hi = T * (blockIdx.x + 1) / gridDim.x;
  if (lo >= hi) return;
  // first query whose keys end after lo
  int qa = 0, qb = b.nq - 1;
  while (qa < qb) {
    const int m = (qa + qb) >> 1;
    if (pre[m + 1] > lo) qb = m;
    else qa = m + 1;
  }
  for (int q = qa; q < b.nq && pre[q] < hi; ++q) {
    const int64_t s0 = max(lo, pre[q]) - pre[q];
    const int64_t s1 = min(hi, pre[q + 1]) - pre[q];
    if (s0 >= s1) continue;
    const int s = b.q_seq[q];
    idx_decode_any<FP8, HIST>(b, qI, w, kI, scores, ld, q, b.seq_row0[s], (int)s0, (int)s1, lh);
    if (HIST) {
      __syncthreads();
      uint32_t* gq = hist + (int64_t)q * TK_BINS1;
      for (int i = tid; i < TK_BINS1; i += IDX_DEC_THREADS) {
        const uint32_t v = lh[i];
        if (v) {
          atomicAdd(&gq[i], v);
          lh[i] = 0u;
        }
      }
      __syncthreads();
    }
  }
}

// One kernel per storage type, so profiles name what ran.
template <bool HIST>
__global__ __launch_bounds__(IDX_DEC_THREADS) void idx_decode_bf16_bal(BatchDev b, const void* qI, const float* w,
                                                                       const void* kI, float* scores, int64_t ld,
                                                                       uint32_t* hist) {
  idx_decode_bal<false, HIST>(b, qI, w, kI, scores, ld, hist);
}
template <bool HIST>
__global__ __launch_bounds__(IDX_DEC_THREADS) void idx_decode_fp8_bal(BatchDev b, const void* qI, const float* w,
                                                                      const void* kI, float* scores, int64_t ld,
                                                                      uint32_t* hist) {
  idx_decode_bal<true, HIST>(b, qI, w, kI, scores, ld, hist);
}
__global__ __launch_bounds__(IDX_DEC_THREADS) void idx_decode_bf16(BatchDev b, const void* qI, const float* w,
                                                                   const void* kI, float* scores, int64_t ld,
                                                                   int chunk) {
  idx_decode_chunked<false>(b, qI, w, kI, scores, ld, chunk);
}
__global__ __launch_bounds__(IDX_DEC_THREADS) void idx_decode_fp8(BatchDev b, const void* qI, const float* w,
                                                                  const void* kI, float* scores, int64_t ld,
                                                                  int chunk) {
  idx_decode_chunked<true>(b, qI, w, kI, scores, ld, chunk);
}

// ---------------------------------------------------------------------------
// decode, fp32 (VALU; small fp32 workloads)
// ---------------------------------------------------------------------------
constexpr int IDX_F32_THREADS = 256;
constexpr int IDX_F32_HG = 4;                               // threads per key, 8 heads each
constexpr int IDX_F32_KEYS = IDX_F32_THREADS / IDX_F32_HG;  // keys per workgroup

// Thread (key, head group hg) computes sum over heads 8hg..8hg+7 of
// w * ReLU(q_h . k), its eight dot products as independent chains over the
// key row held in registers; the four head groups of a key (adjacent lanes)
// add their sums with DPP lane moves.
__global__ __launch_bounds__(IDX_F32_THREADS) void idx_decode_f32(
    BatchDev b, const float* __restrict__ qI, const float* __restrict__ w,
    const float* __restrict__ kI, float* __restrict__ scores, int64_t ld) {
  constexpr int HPG = HI / IDX_F32_HG;
  __shared__ __attribute__((aligned(16))) float qs[HI * DI];
  __shared__ float wsh[HI];
  const int q = blockIdx.y;
  const QueryRange r = query_range(b, q);
  const int base = blockIdx.x * IDX_F32_KEYS;
  if (base >= r.n) return;
  for (int i = threadIdx.x; i < HI * DI / 4; i += IDX_F32_THREADS)
    ((float4*)qs)[i] = ((const float4*)(qI + (int64_t)q * HI * DI))[i];
  if (threadIdx.x < HI) wsh[threadIdx.x] = w[(int64_t)q * HI + threadIdx.x];
  __syncthreads();
  const int hg = threadIdx.x & (IDX_F32_HG - 1);
  const int key = base + threadIdx.x / IDX_F32_HG;
  // keys past the end compute on the last row (every lane takes part in the
  // lane moves) and store nothing
  const float4* kp = (const float4*)(kI + (r.row0 + min(key, r.n - 1)) * DI);
  float4 kr[DI / 4];
#pragma unroll
  for (int i = 0; i < DI / 4; ++i) kr[i] = kp[i];
  const float4* q4 = (const float4*)qs + hg * HPG * (DI / 4);
  float dot[HPG];
#pragma unroll
  for (int h = 0; h < HPG; ++h) dot[h] = 0.0f;
#pragma unroll
  for (int i = 0; i < DI / 4; ++i) {
#pragma unroll
    for (int h = 0; h < HPG; ++h) {
      const float4 qv = q4[h * (DI / 4) + i];
      dot[h] = fmaf(qv.x, kr[i].x, dot[h]);
      dot[h] = fmaf(qv.y, kr[i].y, dot[h]);
      dot[h] = fmaf(qv.z, kr[i].z, dot[h]);
      dot[h] = fmaf(qv.w, kr[i].w, dot[h]);
    }
  }
  float total = 0.0f;
#pragma unroll
  for (int h = 0; h < HPG; ++h) total = fmaf(wsh[hg * HPG + h], relu(dot[h]), total);
  total += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(total), 0xB1, 0xF, 0xF, false));  // quad_perm [1,0,3,2]
  total += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(total), 0x4E, 0xF, 0xF, false));  // quad_perm [2,3,0,1]
  if (hg == 0 && key < r.n) {
    DSA_CHECK(key < ld, DBG_SCORE_COL);
    scores[(int64_t)q * ld + key] = total;
  }
}

// ---------------------------------------------------------------------------
// prefill, bf16: 32 queries per workgroup
// ---------------------------------------------------------------------------
constexpr int PF_THREADS = 512;
constexpr int PF_WAVES = PF_THREADS / 64;
constexpr int PF_QPW = 4;                    // queries per wave
static_assert(PF_QB == PF_WAVES * PF_QPW, "queries per workgroup");
constexpr int PF_TK = 32;                    // keys per LDS tile

// (key chunk, query block) of a prefill workgroup.  Workgroups go to the 8
// XCDs round-robin in launch order (linear id L -> XCD L % 8), each XCD with
// its own L2; the pairs are numbered chunk-major and XCD x takes the x-th
// contiguous eighth of them, so the workgroups that share a key chunk run
// on one XCD and read it into one L2.  (A remainder of fewer than 8
// workgroups keeps the launch order.)
struct PfTile {
  int chunk, qblock;
};
__device__ inline PfTile prefill_tile() {
  const int nchunk = gridDim.x, nqb = gridDim.y;
  const int n = nchunk * nqb;
  const int L = blockIdx.y * nchunk + blockIdx.x;
  const int per = n / 8;
  const int p = L < 8 * per ? (L % 8) * per + L / 8 : L;
  return PfTile{p / nqb, p % nqb};
}

// The block's queries may belong to several sequences (a prefill batch of
// several chunks): the key chunk is swept once per sequence, the first
// sweep for the sequence of the block's first query, each for every block
// query of that sequence.  Fills sq for the next sequence not yet swept
// (same values in every thread) and returns false when none is left.
struct PfSeq {
  int s;          // sequence
  int nmax;       // most candidates among its queries
  uint32_t mine;  // its queries (bit j: block query j)
  uint32_t done;  // queries swept so far
};
__device__ inline bool next_block_sequence(const int* qseq, const int* ncand, PfSeq& sq) {
  int s = -1;
  for (int j = 0; j < PF_QB; ++j)
    if (s < 0 && !((sq.done >> j) & 1u) && qseq[j] >= 0) s = qseq[j];
  if (s < 0) return false;
  uint32_t mine = 0u;
  int nmax = 0;
  for (int j = 0; j < PF_QB; ++j)
    if (qseq[j] == s) {
      mine |= 1u << j;
      nmax = max(nmax, ncand[j]);
    }
  sq.s = s;
  sq.nmax = nmax;
  sq.mine = mine;
  sq.done |= mine;
  return true;
}

// MULTI: the block's queries may belong to several sequences (one sweep of
// the key chunk per sequence, queries one at a time: a pair in flight spills
// registers on top of the sequence loop); otherwise one sequence, queries in
// branch-free pairs.
template <bool MULTI>
__device__ __forceinline__ void prefill_bf16_body(const BatchDev& b, const uint16_t* __restrict__ qI,
                                                  const float* __restrict__ w, const uint16_t* __restrict__ kI,
                                                  float* __restrict__ scores, int64_t ld, int kc) {
  // Key tile: 32 keys x 16 chunks of 16 B; chunk c of key k sits at slot
  // k*16 + (c ^ (k & 15)) so that the B-operand reads hit distinct banks.
  __shared__ u32x4 ktile[2][PF_TK * 16];
  __shared__ float wl[PF_QB * HI];
  __shared__ int ncand[PF_QB];
  __shared__ int qseq[PF_QB];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int col = lane & 31;
  const int half = lane >> 5;
  const PfTile tile = prefill_tile();
  const int qg0 = tile.qblock * PF_QB;
  const int kbase = tile.chunk * kc;

  if (tid < PF_QB) {
    const int qi = qg0 + tid;
    ncand[tid] = qi < b.nq ? query_range(b, qi).n : 0;
    const int sq_i = qi < b.nq ? b.q_seq[qi] : -1;
    qseq[tid] = (sq_i >= 0 && sq_i < b.nseq) ? sq_i : -1;  // out of range: no candidates, like padding
  }
  for (int i = tid; i < PF_QB * HI; i += PF_THREADS) {
    const int qi = qg0 + i / HI;
    wl[i] = qi < b.nq ? w[(int64_t)qg0 * HI + i] : 0.0f;
  }
  __syncthreads();

  bf16x8 a[PF_QPW][8];
#pragma unroll
  for (int j = 0; j < PF_QPW; ++j) {
    const int ql = wave * PF_QPW + j;
    const int qc = min(qg0 + ql, b.nq - 1);
    const uint16_t* qrow = qI + ((int64_t)qc * HI + col) * DI + half * 8;
#pragma unroll
    for (int t = 0; t < 8; ++t) a[j][t] = as_bf16x8(load16(qrow + t * 16));
  }

  if constexpr (!MULTI) {
    int nmax = 0;
#pragma unroll
    for (int j = 0; j < PF_QB; ++j) nmax = max(nmax, ncand[j]);
    const int kend = min(kbase + kc, nmax);
    if (kbase >= kend) return;
    const int64_t row0 = b.seq_row0[0];
    int nj[PF_QPW];
#pragma unroll
    for (int j = 0; j < PF_QPW; ++j) nj[j] = ncand[wave * PF_QPW + j];
    const int lk = tid >> 4;   // key of the tile this thread stages
    const int lc = tid & 15;   // its 16-byte chunk
    const int lslot = lk * 16 + (lc ^ (lk & 15));
    const uint16_t* kb = kI + row0 * DI + lc * 8;
    // per query, a buffer resource over exactly its candidate columns: a
    // store at a column >= n_cand (or from the upper half-wave, which holds no
    // result) lies outside it and is dropped without a branch
    __amdgpu_buffer_rsrc_t srs[PF_QPW];
#pragma unroll
    for (int j = 0; j < PF_QPW; ++j) {
      const int n = __builtin_amdgcn_readfirstlane(nj[j]);
      srs[j] = __builtin_amdgcn_make_buffer_rsrc(scores + (int64_t)(qg0 + wave * PF_QPW + j) * ld, (short)0,
                                                 (int)((uint32_t)n * 4u), 0x00020000);
    }
    u32x4 pre = load16_nt(kb + (int64_t)min(kbase + lk, kend - 1) * DI);
    int buf = 0;
    for (int k0 = kbase; k0 < kend; k0 += PF_TK) {
      ktile[buf][lslot] = pre;
      __syncthreads();
      if (k0 + PF_TK < kend) pre = load16_nt(kb + (int64_t)min(k0 + PF_TK + lk, kend - 1) * DI);
      bf16x8 bfr[8];
#pragma unroll
      for (int t = 0; t < 8; ++t)
        bfr[t] = as_bf16x8(ktile[buf][col * 16 + ((2 * t + half) ^ (col & 15))]);
      const int soff = half ? (int)0x80000000u : (k0 + col) * 4;
      // the wave's queries two at a time, branch-free: two independent
      // product chains, then their ReLU-weighted head sums
#pragma unroll
      for (int jp = 0; jp < PF_QPW; jp += 2) {
        f32x16 acc0 = {}, acc1 = {};
#pragma unroll
        for (int t = 0; t < 8; ++t) {
          acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[jp][t], bfr[t], acc0, 0, 0, 0);
          acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[jp + 1][t], bfr[t], acc1, 0, 0, 0);
        }
        const float* wq0 = wl + (wave * PF_QPW + jp) * HI + 4 * half;
        const float* wq1 = wq0 + HI;
        float p0 = 0.0f, p1 = 0.0f;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          p0 = fmaf(wq0[8 * (i >> 2) + (i & 3)], relu(acc0[i]), p0);
          p1 = fmaf(wq1[8 * (i >> 2) + (i & 3)], relu(acc1[i]), p1);
        }
        p0 = halves_sum(p0);
        p1 = halves_sum(p1);
        __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, p0), srs[jp], soff, 0, 0);
        __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, p1), srs[jp + 1], soff, 0, 0);
      }
      buf ^= 1;
    }
  } else {
    const int lk = tid >> 4;   // key of the tile this thread stages
    const int lc = tid & 15;   // its 16-byte chunk
    const int lslot = lk * 16 + (lc ^ (lk & 15));
    int buf = 0;
    // one pass over the key chunk per sequence among the block's queries
    PfSeq sq{-1, 0, 0u, 0u};
    while (next_block_sequence(qseq, ncand, sq)) {
      const int kend = min(kbase + kc, sq.nmax);
      if (kbase >= kend) continue;
      const uint16_t* kb = kI + b.seq_row0[sq.s] * DI + lc * 8;
      // candidates of the wave's queries in this pass (none for a query of
      // another sequence)
      int nj[PF_QPW];
#pragma unroll
      for (int j = 0; j < PF_QPW; ++j) {
        const int ql = wave * PF_QPW + j;
        nj[j] = ((sq.mine >> ql) & 1u) ? ncand[ql] : 0;
      }
      u32x4 pre = load16_nt(kb + (int64_t)min(kbase + lk, kend - 1) * DI);
      for (int k0 = kbase; k0 < kend; k0 += PF_TK) {
        ktile[buf][lslot] = pre;
        __syncthreads();
        if (k0 + PF_TK < kend) pre = load16_nt(kb + (int64_t)min(k0 + PF_TK + lk, kend - 1) * DI);
        bf16x8 bfr[8];
#pragma unroll
        for (int t = 0; t < 8; ++t)
          bfr[t] = as_bf16x8(ktile[buf][col * 16 + ((2 * t + half) ^ (col & 15))]);
#pragma unroll
        for (int j = 0; j < PF_QPW; ++j) {
          if (k0 >= nj[j]) continue;
          f32x16 acc = {};
#pragma unroll
          for (int t = 0; t < 8; ++t)
            acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[j][t], bfr[t], acc, 0, 0, 0);
          const float* wq = wl + (wave * PF_QPW + j) * HI + 4 * half;
          float part = 0.0f;
#pragma unroll
          for (int i = 0; i < 16; ++i) part = fmaf(wq[8 * (i >> 2) + (i & 3)], relu(acc[i]), part);
          part = halves_sum(part);
          const int key = k0 + col;
          if (half == 0 && key < nj[j]) scores[(int64_t)(qg0 + wave * PF_QPW + j) * ld + key] = part;
        }
        buf ^= 1;
      }
    }
  }
}

__global__ __launch_bounds__(PF_THREADS) void idx_prefill_bf16(BatchDev b, const uint16_t* __restrict__ qI,
                                                               const float* __restrict__ w,
                                                               const uint16_t* __restrict__ kI,
                                                               float* __restrict__ scores, int64_t ld, int kc) {
  prefill_bf16_body<false>(b, qI, w, kI, scores, ld, kc);
}
__global__ __launch_bounds__(PF_THREADS) void idx_prefill_bf16_multi(BatchDev b, const uint16_t* __restrict__ qI,
                                                                     const float* __restrict__ w,
                                                                     const uint16_t* __restrict__ kI,
                                                                     float* __restrict__ scores, int64_t ld, int kc) {
  prefill_bf16_body<true>(b, qI, w, kI, scores, ld, kc);
}

// ---------------------------------------------------------------------------
// prefill, fp8: 32 queries per workgroup
// ---------------------------------------------------------------------------
// v_mfma_f32_32x32x64_f8f6f4: 32 heads on M, 32 keys on N, two products for
// the 128-wide contraction.  Lane (col, half) holds 32 operand bytes per
// product; its contraction slots are taken as bytes [64*half, 64*half + 64)
// of the row (first product the lower 32, second the upper 32), the same for
// query and key, so each lane reads 64 contiguous bytes of one key.
constexpr int PF8_TK = 256;  // keys per LDS tile (eight 32-key products)

// KC: keys per workgroup, a compile-time constant (this kernel uses every
// register, and a run-time chunk length costs it spills)
template <int KC>
__global__ __launch_bounds__(PF_THREADS) void idx_prefill_fp8(
    BatchDev b, const uint8_t* __restrict__ qI, const float* __restrict__ w,
    const uint8_t* __restrict__ kI, float* __restrict__ scores, int64_t ld) {
  constexpr int kc = KC;
  // Key tile: 256 keys x 8 chunks of 16 B; chunk c of key k sits at slot
  // k*8 + (c ^ ((k >> 1) & 7)), so the 16 keys a quarter-wave reads fall on
  // 16 distinct 16-byte bank groups.
  __shared__ u32x4 ktile[2][PF8_TK * 8];
  __shared__ float wl[PF_QB * HI];
  __shared__ int ncand[PF_QB];
  __shared__ int qseq[PF_QB];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 31;
  const int half = lane >> 5;
  const PfTile tile = prefill_tile();
  const int qg0 = tile.qblock * PF_QB;
  const int kbase = tile.chunk * kc;

  if (tid < PF_QB) {
    const int qi = qg0 + tid;
    ncand[tid] = qi < b.nq ? query_range(b, qi).n : 0;
    const int sq_i = qi < b.nq ? b.q_seq[qi] : -1;
    qseq[tid] = (sq_i >= 0 && sq_i < b.nseq) ? sq_i : -1;  // out of range: no candidates, like padding
  }
  for (int i = tid; i < PF_QB * HI; i += PF_THREADS) {
    const int qi = qg0 + i / HI;
    wl[i] = qi < b.nq ? w[(int64_t)qg0 * HI + i] : 0.0f;
  }
  __syncthreads();

  i32x8 a[PF_QPW][2];
  float wr[PF_QPW][16];
#pragma unroll
  for (int j = 0; j < PF_QPW; ++j) {
    const int ql = wave * PF_QPW + j;
    const int qc = min(qg0 + ql, b.nq - 1);
    const uint8_t* qrow = qI + ((int64_t)qc * HI + col) * DI + half * 64;
    a[j][0] = cat32(load16(qrow), load16(qrow + 16));
    a[j][1] = cat32(load16(qrow + 32), load16(qrow + 48));
#pragma unroll
    for (int i = 0; i < 16; ++i) wr[j][i] = wl[ql * HI + 4 * half + 8 * (i >> 2) + (i & 3)];
  }

  constexpr int TK = PF8_TK;
  constexpr int NR = TK * 8 / PF_THREADS;  // 16-byte chunks each thread stages
  const int lk = tid >> 3;   // key of the tile this thread stages (plus r*PF_THREADS/8)
  const int lc = tid & 7;    // its 16-byte chunk
  const int lslot = lk * 8 + (lc ^ ((lk >> 1) & 7));
  int buf = 0;
  // one pass over the key chunk per sequence among the block's queries
  PfSeq sq{-1, 0, 0u, 0u};
  while (next_block_sequence(qseq, ncand, sq)) {
    const int kend = min(kbase + kc, sq.nmax);
    if (kbase >= kend) continue;
    const uint8_t* kb = kI + b.seq_row0[sq.s] * DI + lc * 16;
    u32x4 pre[NR];
#pragma unroll
    for (int r = 0; r < NR; ++r) pre[r] = load16_nt(kb + (int64_t)min(kbase + lk + (PF_THREADS / 8) * r, kend - 1) * DI);
    // one buffer resource per query over exactly its candidate columns (none
    // for a query of another sequence): a store at a column >= n_cand (or
    // from the upper half-wave, which holds no result) lies outside it and is
    // dropped without a branch
    __amdgpu_buffer_rsrc_t srs[PF_QPW];
#pragma unroll
    for (int j = 0; j < PF_QPW; ++j) {
      const int ql = wave * PF_QPW + j;
      const int n = __builtin_amdgcn_readfirstlane(((sq.mine >> ql) & 1u) ? ncand[ql] : 0);
      srs[j] = __builtin_amdgcn_make_buffer_rsrc(scores + (int64_t)(qg0 + ql) * ld, (short)0,
                                                 (int)((uint32_t)n * 4u), 0x00020000);
    }
    for (int k0 = kbase; k0 < kend; k0 += TK) {
#pragma unroll
      for (int r = 0; r < NR; ++r) ktile[buf][lslot + r * PF_THREADS] = pre[r];
      __syncthreads();
      // next tile (clamped, so the last iteration re-reads an in-range key)
#pragma unroll
      for (int r = 0; r < NR; ++r) pre[r] = load16_nt(kb + (int64_t)min(k0 + TK + lk + (PF_THREADS / 8) * r, kend - 1) * DI);
      const int nsub = min(TK / 32, (kend - k0 + 31) / 32);
      for (int sub = 0; sub < nsub; ++sub) {
        const int kk = sub * 32 + col;
        const int sw = (kk >> 1) & 7;
        const u32x4* krow = &ktile[buf][kk * 8];
        const i32x8 b0 = cat32(krow[(4 * half + 0) ^ sw], krow[(4 * half + 1) ^ sw]);
        const i32x8 b1 = cat32(krow[(4 * half + 2) ^ sw], krow[(4 * half + 3) ^ sw]);
        // all queries of the wave, branch-free, so the products of one query
        // overlap the epilogue of another
        f32x16 acc[PF_QPW];
#pragma unroll
        for (int j = 0; j < PF_QPW; ++j) {
          const f32x16 z = {};
          // format 0 = FP8 E4M3 for both operands, no block scaling
          acc[j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a[j][0], b0, z, 0, 0, 0, 0, 0, 0);
          acc[j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a[j][1], b1, acc[j], 0, 0, 0, 0, 0, 0);
        }
        const int soff = half ? (int)0x80000000u : (k0 + sub * 32 + col) * 4;
#pragma unroll
        for (int j = 0; j < PF_QPW; ++j) {
          float part = 0.0f;
#pragma unroll
          for (int i = 0; i < 16; ++i) part = fmaf(wr[j][i], relu(acc[j][i]), part);
          part = halves_sum(part);
          __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, part), srs[j], soff, 0, 0);
        }
      }
      buf ^= 1;
    }
  }
}

// ---------------------------------------------------------------------------
// host launchers
// ---------------------------------------------------------------------------
#ifdef DSA_DEBUG
DSA_DEBUG_READER(debug_flags_indexer)
#endif

hipError_t launch_zero(const ZeroSpans& z, int nq, hipStream_t st) {
  if (nq == 0 || (z.s[0].base == nullptr && z.s[1].base == nullptr)) return hipSuccess;
  hipLaunchKernelGGL(zero_spans_kernel, dim3(nq), dim3(256), 0, st, z);
  return hipGetLastError();
}

hipError_t launch_index_score(const BatchDev& b, int dtype, const void* qI, const float* w,
                              const void* kI, float* scores, int64_t ld, hipStream_t st, uint32_t* hist,
                              bool* hist_done) {
  if (hist_done) *hist_done = false;
  if (b.nq == 0) return hipSuccess;
  switch (index_kernel(dtype, b.nq, b.nseq)) {
    case IndexKernel::F32: {
      dim3 grid((b.max_len + IDX_F32_KEYS - 1) / IDX_F32_KEYS, b.nq);
      hipLaunchKernelGGL(idx_decode_f32, grid, dim3(IDX_F32_THREADS), 0, st, b, (const float*)qI, w,
                         (const float*)kI, scores, ld);
      break;
    }
    case IndexKernel::Prefill: {
      // a sequence's queries are best contiguous in the batch, so that
      // blocks rarely straddle sequences
      const int kc = prefill_key_chunk(b.nq, b.max_len);
      dim3 grid((b.max_len + kc - 1) / kc, (b.nq + PF_QB - 1) / PF_QB);
      if (dtype == 2) {
        const uint8_t* q8 = (const uint8_t*)qI;
        const uint8_t* k8 = (const uint8_t*)kI;
        if (kc == 8192)
          hipLaunchKernelGGL(idx_prefill_fp8<8192>, grid, dim3(PF_THREADS), 0, st, b, q8, w, k8, scores, ld);
        else if (kc == 4096)
          hipLaunchKernelGGL(idx_prefill_fp8<4096>, grid, dim3(PF_THREADS), 0, st, b, q8, w, k8, scores, ld);
        else if (kc == 2048)
          hipLaunchKernelGGL(idx_prefill_fp8<2048>, grid, dim3(PF_THREADS), 0, st, b, q8, w, k8, scores, ld);
        else
          hipLaunchKernelGGL(idx_prefill_fp8<1024>, grid, dim3(PF_THREADS), 0, st, b, q8, w, k8, scores, ld);
      } else if (b.nseq == 1) {
        hipLaunchKernelGGL(idx_prefill_bf16, grid, dim3(PF_THREADS), 0, st, b, (const uint16_t*)qI, w,
                           (const uint16_t*)kI, scores, ld, kc);
      } else {
        hipLaunchKernelGGL(idx_prefill_bf16_multi, grid, dim3(PF_THREADS), 0, st, b, (const uint16_t*)qI, w,
                           (const uint16_t*)kI, scores, ld, kc);
      }
      break;
    }
    case IndexKernel::Balanced: {
      const dim3 grid(IDX_BAL_GRID), block(IDX_DEC_THREADS);
      if (hist != nullptr) {
        if (dtype == 2)
          hipLaunchKernelGGL(idx_decode_fp8_bal<true>, grid, block, 0, st, b, qI, w, kI, scores, ld, hist);
        else
          hipLaunchKernelGGL(idx_decode_bf16_bal<true>, grid, block, 0, st, b, qI, w, kI, scores, ld, hist);
        if (hist_done) *hist_done = true;
      } else {
        if (dtype == 2)
          hipLaunchKernelGGL(idx_decode_fp8_bal<false>, grid, block, 0, st, b, qI, w, kI, scores, ld, hist);
        else
          hipLaunchKernelGGL(idx_decode_bf16_bal<false>, grid, block, 0, st, b, qI, w, kI, scores, ld, hist);
      }
      break;
    }
    case IndexKernel::Chunked: {
      const int chunk = decode_key_chunk(b.nq, b.max_len);
      dim3 grid((b.max_len + chunk - 1) / chunk, b.nq);
      if (dtype == 2)
        hipLaunchKernelGGL(idx_decode_fp8, grid, dim3(IDX_DEC_THREADS), 0, st, b, qI, w, kI, scores, ld, chunk);
      else
        hipLaunchKernelGGL(idx_decode_bf16, grid, dim3(IDX_DEC_THREADS), 0, st, b, qI, w, kI, scores, ld, chunk);
      break;
    }
  }
  return hipGetLastError();
}

}  // namespace dsa
