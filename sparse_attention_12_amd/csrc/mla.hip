// Sparse MLA read on gfx950 (concept page "Mistral Large 4", sections "What
// to keep", "Where to look" and "Sparse attention").  For query q with
// selected positions S (its row of idx), in absorbed form:
//   l[h][j] = scale * q[h][0:W] . kv[S_j][0:W]
//   o[h]    = sum_j softmax_j(l[h])[j] * kv[S_j][0:512]     (softmax over S only)
//   lse[h]  = log sum_j exp(l[h][j])
// with row width W = 512 + R: R = 64 rotary values, or R = 0 in the layers
// without rotary encoding (every fourth layer, list of changes on the same
// page).  64 x (512 + R + 512) multiply-adds per selected position.
//
// bf16 kernel: one workgroup (8 waves) per (split of the selection, query,
// layer); wave w owns heads 16(w%4)..16(w%4)+15 and half of the row width
// for the logits, half of the latent columns for the values.  Per tile of
// 32 positions the 576-wide bf16 rows are gathered into LDS, then
//   S^T (32 positions x 16 heads) = K_tile . Q_w^T   (MFMA 16x16x32; the two
//   halves of the contraction are summed through LDS)
//   online softmax in the exp2 domain, rescaling the accumulator only when a
//   head's running max grows by more than 2^8
//   O_w^T (256 x 16) += V_tile^T . P^T               (MFMA 16x16x32)
// The S^T accumulator layout puts, in each lane, one head and 8 positions --
// exactly the B operand of the P.V product when the 32 positions of a tile
// are taken in the order {4g..4g+3, 16+4g..16+4g+3} for lane group g, so P
// never leaves registers.  The value operand reads the same LDS tile
// column-wise.  Splits of one query are merged by log-sum-exp in
// mla_combine.
#include <math.h>

#include "dsa_common.h"
#include "kernels.h"

namespace dsa {

struct MlaParams {
  BatchDev b;
  const int32_t* idx;
  int k;
  int nsplit;
  int split_len;
  int n_layers;
  int out_bf16;
  float scale_log2;  // scale * log2(e)
  void* part_o;      // [nsplit][n_layers][nq][64][512] split outputs, each normalised by its
                     // own sum: bf16 for the bf16 kernel, float32 for the fp32 one
  float* part_ml;    // [nsplit][n_layers][nq][64][2]  (max in log2 units, sum)
  MlaLayers L;
};

constexpr float LN2 = 0.69314718055994530942f;

// Workgroups reach the eight XCDs round-robin in dispatch order: workgroup
// L of a one-dimensional grid runs on XCD L % 8.  xcd_item gives XCD x one
// contiguous range of the grid's N items (N/8 of them, one more for the
// first N % 8 XCDs), so items that are numbered together share one L2.  The
// attention and merge grids both number their items (layer, query)-major,
// so the splits of one query's layer read its query rows into one L2 and
// the merge finds their partials there.
__device__ inline int xcd_item(int L, int N) {
  const int x = L & 7;
  const int q8 = N >> 3;
  return x * q8 + min(x, N & 7) + (L >> 3);
}

__device__ inline void store_out4(const MlaParams& p, int layer, int64_t off, f32x4 v) {
  if (p.out_bf16) {
    uint16_t* o = (uint16_t*)p.L.out[layer] + off;
    uint2 pk;
    pk.x = pack_bf16x2(v[0], v[1]);
    pk.y = pack_bf16x2(v[2], v[3]);
    *(uint2*)o = pk;
  } else {
    *(f32x4*)((float*)p.L.out[layer] + off) = v;
  }
}

// ---------------------------------------------------------------------------
// bf16 split kernel
// ---------------------------------------------------------------------------
// One workgroup of 8 waves per (split, query, layer).  Wave w = (h, d) with
// h = w % 4 (heads 16h..16h+15) and d = w / 4:
//   * S^T for its 16 heads over the tile: wave d contracts dims
//     [288d, 288d+288) and the two waves of a head group add their partial
//     logits through LDS (a + b = b + a, so both hold identical logits and
//     take identical softmax steps);
//   * O^T for its 16 heads and latent columns [256d, 256d+256).
// Tiles of 32 selected rows are gathered straight into a ring of three LDS
// buffers; the two wave halves issue alternate tiles, so two tiles are in
// flight while one is consumed.
constexpr int MLA_THREADS = 512;
constexpr int MLA_SPLIT_MAX = KMAX;
constexpr int MLA_VBLK = DC / 16 / 2;           // 16-column value blocks per wave (16)
constexpr float MLA_RESCALE_SLACK = 8.0f;       // log2 units

// Row geometry for rotary width ROPE (64, or 0 without rotary encoding).
template <int ROPE>
struct MlaGeo {
  static constexpr int W = DC + ROPE;                  // 576 or 512 values per row
  static constexpr int ROWB = W * 2;                   // 1,152 or 1,024 bytes per bf16 row
  static constexpr int TILEB = MLA_TILE * ROWB;        // 36,864 or 32,768 bytes per tile
  static constexpr int KSTEPS = W / 32 / 2;            // contraction steps per wave (9 or 8)
  static constexpr int BLOCKS = (ROWB / 128) * (MLA_TILE / 8);  // 1 KB gather blocks per tile (36 or 32)
  static constexpr int WAVE_DMAS = (BLOCKS + MLA_THREADS / 64 - 1) / (MLA_THREADS / 64);  // 5 or 4
  static_assert(WAVE_DMAS * (MLA_THREADS / 64) >= BLOCKS, "every block must be gathered");
  static_assert(WAVE_DMAS <= 7, "wait counts below assume fewer than 16 gathers in flight");
};

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
typedef __attribute__((address_space(3))) void lds_void;

// LDS tile layout: W/64 column groups of 64 latent/rotary values (nine for
// 576-wide rows); group G holds rows 0..31 at 128 bytes each, and row r's
// logical 16-byte chunk c (of the group's eight) sits at chunk slot c ^ (r & 7).
// One gather instruction of a wave fills rows 8w'..8w'+7 of one group: 1 KB,
// written in lane order.
constexpr int MLA_GROUPB = MLA_TILE * 128;  // 4,096 bytes per column group

__device__ inline int tile_off(int row, int chunk) {
  return (chunk >> 3) * MLA_GROUPB + row * 128 + (((chunk & 7) ^ (row & 7)) << 4);
}

struct MlaTileState {
  f32x4 o[MLA_VBLK];
  float m_run;
  float l_part;
};

// Gather tile t into LDS.  A tile is BLOCKS blocks of 1 KB (column group
// i, row octet o); every wave issues exactly WAVE_DMAS gather instructions
// per tile -- blocks WAVE_DMAS*w .. WAVE_DMAS*w + WAVE_DMAS-1, where ids past
// the last block re-load the last block's rows into a scratch slot -- so all
// waves keep the same number of gathers in flight.  Within a block, lane l
// fetches row 8o + l/8, 16-byte chunk ((l % 8) ^ (row & 7)) + 8i, landing
// at lane slot l.

// Selected positions of the rows this lane gathers for tile t (read ahead of
// the gathers, so no gather waits on an LDS read).
template <int ROPE>
__device__ __forceinline__ void mla_rows(int (&pos)[MlaGeo<ROPE>::WAVE_DMAS], const int* sel_l, int t, int lane,
                                         int wave_u) {
  using G = MlaGeo<ROPE>;
#pragma unroll
  for (int jj = 0; jj < G::WAVE_DMAS; ++jj) {
    const int blk = min(wave_u * G::WAVE_DMAS + jj, G::BLOCKS - 1);
    pos[jj] = sel_l[t * MLA_TILE + (blk & 3) * 8 + (lane >> 3)];
  }
}

// The gathers are buffer loads with an LDS destination (MUBUF, not FLAT, so
// the compiler keeps precise LDS wait counts around them) addressed from the
// sequence's first row; sequences up to 2^32 bytes of rows are supported.
template <int ROPE>
__device__ __forceinline__ void mla_issue(uint8_t* buf, uint8_t* dummy, __amdgpu_buffer_rsrc_t kv,
                                          const int (&pos)[MlaGeo<ROPE>::WAVE_DMAS], int lane, int wave_u) {
  using G = MlaGeo<ROPE>;
#pragma unroll
  for (int jj = 0; jj < G::WAVE_DMAS; ++jj) {
    const int id = wave_u * G::WAVE_DMAS + jj;
    const int blk = min(id, G::BLOCKS - 1);
    const int gi = blk >> 2;
    const int oc = blk & 3;
    const int row = oc * 8 + (lane >> 3);
    DSA_CHECK(pos[jj] >= -1, DBG_GATHER_ROW);
    const uint32_t off = (uint32_t)max(pos[jj], 0) * (uint32_t)G::ROWB + (uint32_t)(gi * 8 + ((lane & 7) ^ (row & 7))) * 16u;
    uint8_t* dst = id < G::BLOCKS ? buf + gi * MLA_GROUPB + oc * 1024 : dummy;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(kv, (lds_void*)dst, 16, off, 0, 0, 0);
  }
}

// Partial S^T (32 positions x 16 heads) over this wave's half of the
// contraction; lane (n16, g) gets positions 16*mb + 4g + i of head n16.
template <int ROPE>
__device__ __forceinline__ void mla_partial_logits(const uint8_t* tile, const bf16x8 (&qf)[MlaGeo<ROPE>::KSTEPS], int d,
                                                   int n16, int g, f32x4 (&s)[2]) {
  constexpr int MLA_KSTEPS = MlaGeo<ROPE>::KSTEPS;
  // Row r's logical chunk 4t+g lies in column group t/2 at in-group chunk
  // 4*(t%2) + g.  Loads run two steps ahead; each block keeps two chains.
  const uint8_t* ev[2];
  const uint8_t* od[2];
#pragma unroll
  for (int mb = 0; mb < 2; ++mb) {
    const int row = 16 * mb + n16;
    ev[mb] = tile + tile_off(row, g);
    od[mb] = tile + tile_off(row, 4 + g);
  }
  const int t0 = d * MLA_KSTEPS;
  auto kfrag = [&](int mb, int tt) -> u32x4 {
    const int t = t0 + tt;
    return *(const u32x4*)(((t & 1) ? od[mb] : ev[mb]) + (t >> 1) * MLA_GROUPB);
  };
  f32x4 acc[2][2];
#pragma unroll
  for (int mb = 0; mb < 2; ++mb) acc[mb][0] = acc[mb][1] = f32x4{0.f, 0.f, 0.f, 0.f};
  u32x4 ring[3][2];
  ring[0][0] = kfrag(0, 0);
  ring[0][1] = kfrag(1, 0);
  ring[1][0] = kfrag(0, 1);
  ring[1][1] = kfrag(1, 1);
#pragma unroll
  for (int tt = 0; tt < MLA_KSTEPS; ++tt) {
    if (tt + 2 < MLA_KSTEPS) {
      ring[(tt + 2) % 3][0] = kfrag(0, tt + 2);
      ring[(tt + 2) % 3][1] = kfrag(1, tt + 2);
    }
    acc[0][tt & 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(ring[tt % 3][0]), qf[tt], acc[0][tt & 1], 0, 0, 0);
    acc[1][tt & 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(ring[tt % 3][1]), qf[tt], acc[1][tt & 1], 0, 0, 0);
  }
  // keep the loads two steps ahead of their use: 4 reads, then (2 reads,
  // 2 products) per step, then the last 4 products
  __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
  for (int tt = 0; tt + 2 < MLA_KSTEPS; ++tt) {
    __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
    __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
  }
  __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
  s[0] = acc[0][0] + acc[0][1];
  s[1] = acc[1][0] + acc[1][1];
}

// Online softmax over the tile's logits and O^T += V_tile^T . P^T for this
// wave's 256 latent columns.
// valid: bit j set when the tile's position j is a kept position.
__device__ __forceinline__ void mla_softmax_pv(MlaTileState& st, const uint8_t* tile, const f32x4 (&s)[2], uint32_t valid,
                                               int d, int n16, int g, float scale_log2) {
  float x[8];
  float tmax = -INFINITY;
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const bool ok = (valid >> (16 * mb + 4 * g + i)) & 1u;
      const float v = ok ? s[mb][i] * scale_log2 : -INFINITY;
      x[mb * 4 + i] = v;
      tmax = fmaxf(tmax, v);
    }
  tmax = rows4_max(tmax);
  const bool resc = tmax > st.m_run + MLA_RESCALE_SLACK;
  if (__any(resc)) {
    const float alpha = resc ? __builtin_amdgcn_exp2f(st.m_run - tmax) : 1.0f;
    if (resc) st.m_run = tmax;
    st.l_part *= alpha;
#pragma unroll
    for (int vb = 0; vb < MLA_VBLK; ++vb) st.o[vb] *= alpha;
  }
  float pv[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    // hardware exp2 (no subnormal results: weights below 2^-126 vanish)
    const float ev = __builtin_amdgcn_exp2f(x[e] - st.m_run);
    pv[e] = (x[e] == -INFINITY) ? 0.0f : ev;
    st.l_part += pv[e];
  }
  u32x4 pk;
  pk[0] = pack_bf16x2(pv[0], pv[1]);
  pk[1] = pack_bf16x2(pv[2], pv[3]);
  pk[2] = pack_bf16x2(pv[4], pv[5]);
  pk[3] = pack_bf16x2(pv[6], pv[7]);
  const bf16x8 pb = as_bf16x8(pk);
  __builtin_amdgcn_sched_barrier(0);

  // k-slot e of lane group g is tile row (e < 4 ? 4g + e : 16 + 4g + e - 4).
  // A transposing LDS read gives lane i of a 16-lane group element i%4 of
  // source lane 4j + i/4, so source lane s points at row 4g + s/4 (+16) and
  // latent column c0 + 4(s%4).  Column 256d + 16vb + sdim lies in column
  // group 4d + vb/4 at in-group chunk 2*(vb%4) + sdim/8.
  const int srow0 = 4 * g + (n16 >> 2);
  const int srow1 = srow0 + 16;
  const int sdim = 4 * (n16 & 3);
  const int c0 = 32 * d + (sdim >> 3);
  const int boff = (sdim & 7) << 1;
  const uint8_t* b0[4];
  const uint8_t* b1[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    b0[u] = tile + tile_off(srow0, c0 + 2 * u) + boff;
    b1[u] = tile + tile_off(srow1, c0 + 2 * u) + boff;
  }
  auto vfrag = [&](int vb) -> bf16x8 {
    const int u = vb & 3;
    const int imm = (vb >> 2) * MLA_GROUPB;
    const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(b0[u] + imm));
    const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(b1[u] + imm));
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
  };
  bf16x8 vr[4];
  vr[0] = vfrag(0);
  vr[1] = vfrag(1);
  vr[2] = vfrag(2);
#pragma unroll
  for (int vb = 0; vb < MLA_VBLK; ++vb) {
    if (vb + 3 < MLA_VBLK) vr[(vb + 3) & 3] = vfrag(vb + 3);
    st.o[vb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vr[vb & 3], pb, st.o[vb], 0, 0, 0);
  }
  // transposing reads three blocks ahead of the products
  __builtin_amdgcn_sched_group_barrier(0x100, 6, 1);
#pragma unroll
  for (int vb = 0; vb + 3 < MLA_VBLK; ++vb) {
    __builtin_amdgcn_sched_group_barrier(0x100, 2, 1);
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 1);
  }
  __builtin_amdgcn_sched_group_barrier(0x008, 3, 1);
}

// Workgroup barrier without a memory fence.  __syncthreads() would make
// every wave wait for all of its outstanding gathers (they count as vector
// memory operations); here each wave first waits for exactly what it must
// publish (see the callers), and the empty asm statements keep the compiler
// from moving memory accesses across the barrier.
__device__ __forceinline__ void barrier_no_fence() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

template <int ROPE>
__global__ __launch_bounds__(MLA_THREADS, 1) void mla_bf16_kernel(MlaParams p) {
  using G = MlaGeo<ROPE>;
  constexpr int MLA_KSTEPS = G::KSTEPS;
  constexpr int MLA_WAVE_DMAS = G::WAVE_DMAS;
  // three distinct arrays, so that reads of one tile are known not to alias
  // the asynchronous gathers into the others
  __shared__ __attribute__((aligned(16))) uint8_t tile0[G::TILEB];
  __shared__ __attribute__((aligned(16))) uint8_t tile1[G::TILEB];
  __shared__ __attribute__((aligned(16))) uint8_t tile2[G::TILEB];
  __shared__ __attribute__((aligned(16))) uint8_t scratch_blk[1024];  // target of the filler gathers
  __shared__ int sel_l[MLA_SPLIT_MAX];
  __shared__ __attribute__((aligned(16))) f32x4 xpart[8][64][2];  // partial logits per wave
  const int item = xcd_item(blockIdx.x, p.nsplit * p.b.nq * p.n_layers);
  const int split = item % p.nsplit;
  const int q = (item / p.nsplit) % p.b.nq;
  const int layer = item / (p.nsplit * p.b.nq);
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave_u = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hgrp = wave_u & 3;
  const int d = wave_u >> 2;
  const int n16 = lane & 15;
  const int g = lane >> 4;
  const int j_begin = split * p.split_len;
  const int nent = max(0, min(j_begin + p.split_len, p.k) - j_begin);
  const int head = hgrp * 16 + n16;

  // Q and this split's entries of idx are requested first: neither depends
  // on the sequence, so their round trip overlaps the batch lookups.
  // Q^T (this wave's heads and half of the contraction) as the B operand:
  // head `head`, contraction slots (KSTEPS*d + tt)*32 + 8g + [0,8)
  bf16x8 qf[MLA_KSTEPS];
  {
    const uint16_t* qp = (const uint16_t*)p.L.q[layer] + ((int64_t)q * H + head) * G::W + d * (G::W / 2) + g * 8;
#pragma unroll
    for (int tt = 0; tt < MLA_KSTEPS; ++tt) qf[tt] = as_bf16x8(load16(qp + tt * 32));
  }
  constexpr int SEL_PER = MLA_SPLIT_MAX / MLA_THREADS;
  int selv[SEL_PER];
  {
    const int32_t* sel = p.idx + (int64_t)q * p.k + j_begin;
#pragma unroll
    for (int i = 0; i < SEL_PER; ++i) {
      const int j = tid + i * MLA_THREADS;
      selv[i] = j < nent ? sel[j] : -1;
    }
  }
  const QueryRange r = query_range(p.b, q);
  const int ntiles = r.n > 0 ? (nent + MLA_TILE - 1) / MLA_TILE : 0;
  // this split's selected positions, padded with -1 to whole tiles (at
  // least two: tiles 0 and 1 are always gathered); entries outside [0, n)
  // become -1
#pragma unroll
  for (int i = 0; i < SEL_PER; ++i) {
    const int j = tid + i * MLA_THREADS;
    if (j < max(ntiles, 2) * MLA_TILE) sel_l[j] = (selv[i] >= 0 && selv[i] < r.n) ? selv[i] : -1;
    DSA_CHECK(j >= nent || (selv[i] >= -1 && selv[i] < r.n), DBG_IDX_RANGE);
  }
  // buffer resource over exactly this sequence's rows (raw addressing): a
  // gather outside them reads zeros and touches no memory
  const __amdgpu_buffer_rsrc_t kv = __builtin_amdgcn_make_buffer_rsrc(
      (void*)((const uint16_t*)p.L.kv[layer] + r.row0 * G::W), (short)0, (int)((uint32_t)r.n * (uint32_t)G::ROWB),
      0x00020000);
  MlaTileState st;
#pragma unroll
  for (int vb = 0; vb < MLA_VBLK; ++vb) st.o[vb] = f32x4{0.f, 0.f, 0.f, 0.f};
  st.m_run = -INFINITY;
  st.l_part = 0.0f;
  __syncthreads();

  // tile t goes to buffer t % 3; two tiles are gathered ahead.  Tiles 0
  // and 1 are issued whatever the tile count (a missing tile's entries are
  // -1 and gather row 0, which the kept-position mask then ignores), so the
  // wait below is the same on every path.
  int rows[MLA_WAVE_DMAS];
  mla_rows<ROPE>(rows, sel_l, 0, lane, wave_u);
  mla_issue<ROPE>(tile0, scratch_blk, kv, rows, lane, wave_u);
  mla_rows<ROPE>(rows, sel_l, 1, lane, wave_u);
  mla_issue<ROPE>(tile1, scratch_blk, kv, rows, lane, wave_u);
  mla_rows<ROPE>(rows, sel_l, min(2, max(ntiles, 1) - 1), lane, wave_u);
  // Q (loaded before the gathers) must be in registers before the loop:
  // wait for it alone, leaving both tiles' gathers in flight
  __builtin_amdgcn_s_waitcnt(0x0F70 | (2 * MLA_WAVE_DMAS));  // vmcnt(2 * WAVE_DMAS)
  // From here on Q counts as computed, not loaded: otherwise the compiler
  // drains every gather before the loop because the loop reads registers
  // loaded outside it.
#pragma unroll
  for (int tt = 0; tt < MLA_KSTEPS; ++tt) asm volatile("" : "+v"(qf[tt]));

  auto step = [&](int it, const uint8_t* cur, uint8_t* nxt2) __attribute__((always_inline)) {
    // Every wave waits for its own part of tile `it` (the gathers of tile
    // it+1 stay in flight); after the barrier the tile is complete and tile
    // it-1's buffer is free for tile it+2.
    if (it + 1 < ntiles)
      __builtin_amdgcn_s_waitcnt(0x0070 | MLA_WAVE_DMAS);  // vmcnt(WAVE_DMAS) lgkmcnt(0)
    else
      __builtin_amdgcn_s_waitcnt(0x0070);  // vmcnt(0) lgkmcnt(0)
    barrier_no_fence();
    if (it + 2 < ntiles) mla_issue<ROPE>(nxt2, scratch_blk, kv, rows, lane, wave_u);
    // unconditional (a clamped, harmless re-read at the end), so that the
    // wait counts below need not merge two control paths
    mla_rows<ROPE>(rows, sel_l, min(it + 3, ntiles - 1), lane, wave_u);
    // validity of the tile's 32 positions, read now and folded into a mask
    // after the logits (the read's latency hides behind them)
    const int vpos = sel_l[it * MLA_TILE + (lane & 31)];
    f32x4 s[2];
    __builtin_amdgcn_sched_barrier(0);
    mla_partial_logits<ROPE>(cur, qf, d, n16, g, s);
    __builtin_amdgcn_sched_barrier(0);
    xpart[wave_u][lane][0] = s[0];
    xpart[wave_u][lane][1] = s[1];
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): partial logits written
    barrier_no_fence();
    s[0] += xpart[wave_u ^ 4][lane][0];
    s[1] += xpart[wave_u ^ 4][lane][1];
    const uint32_t valid = (uint32_t)__ballot(vpos >= 0);
    mla_softmax_pv(st, cur, s, valid, d, n16, g, p.scale_log2);
  };
  for (int it = 0; it < ntiles; it += 3) {
    step(it, tile0, tile2);
    if (it + 1 >= ntiles) break;
    step(it + 1, tile1, tile0);
    if (it + 2 >= ntiles) break;
    step(it + 2, tile2, tile1);
  }
  __builtin_amdgcn_s_waitcnt(0x0F70);  // every gather has landed before the LDS is released

  const float l_part = rows4_sum(st.l_part);
  const int64_t qh = (int64_t)q * H + head;
  const int col0 = d * (DC / 2);
  if (p.nsplit == 1) {
    const float inv = l_part > 0.0f ? 1.0f / l_part : 0.0f;
#pragma unroll
    for (int vb = 0; vb < MLA_VBLK; ++vb) store_out4(p, layer, qh * DC + col0 + vb * 16 + 4 * g, st.o[vb] * inv);
    if (d == 0 && g == 0 && p.L.lse[layer])
      p.L.lse[layer][qh] = l_part > 0.0f ? (st.m_run + log2f(l_part)) * LN2 : -INFINITY;
  } else {
    // the split's output normalised by its own sum, in bf16 (half the
    // partial traffic of float32; the merge weighs it by that sum)
    const int64_t slot = ((int64_t)split * p.n_layers + layer) * p.b.nq * H + qh;
    const float inv = l_part > 0.0f ? 1.0f / l_part : 0.0f;
    uint16_t* po = (uint16_t*)p.part_o + slot * DC + col0;
#pragma unroll
    for (int vb = 0; vb < MLA_VBLK; ++vb) {
      const f32x4 v = st.o[vb] * inv;
      uint2 pk;
      pk.x = pack_bf16x2(v[0], v[1]);
      pk.y = pack_bf16x2(v[2], v[3]);
      *(uint2*)(po + vb * 16 + 4 * g) = pk;
    }
    if (d == 0 && g == 0) {
      p.part_ml[slot * 2 + 0] = l_part > 0.0f ? st.m_run : -INFINITY;
      p.part_ml[slot * 2 + 1] = l_part;
    }
  }
}

// ---------------------------------------------------------------------------
// fp32 split kernel (VALU; small fp32 workloads)
// ---------------------------------------------------------------------------
// Thread t = (head group hg = t / 16, part = t % 16) owns heads 4hg..4hg+3
// and a sixteenth of the row: contraction values [part*W/16, +W/16) and value
// columns [32 part, 32 part + 32).  Each row value read from the LDS tile
// serves four heads; the four partial logits are summed over the 16 parts
// (lanes of one DPP row) with lane moves.  The next tile's rows are loaded
// into registers while the current one is consumed.
constexpr int MLA32_THREADS = 256;
constexpr int MLA32_HPT = 4;   // heads per thread
constexpr int MLA32_PARTS = 16;

// Sum over the 16 lanes of a DPP row; every lane of the row gets the sum.
__device__ inline float row16_sum(float x) {
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0xB1, 0xF, 0xF, false));   // quad_perm [1,0,3,2]
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x4E, 0xF, 0xF, false));   // quad_perm [2,3,0,1]
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x141, 0xF, 0xF, false));  // row_half_mirror
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x140, 0xF, 0xF, false));  // row_mirror
  return x;
}

template <int ROPE>
__global__ __launch_bounds__(MLA32_THREADS) void mla_f32_kernel(MlaParams p) {
  constexpr int D = DC + ROPE;              // row width
  constexpr int QS = D / MLA32_PARTS;       // 36 (or 32) contraction values per thread
  constexpr int VS = DC / MLA32_PARTS;      // 32 value columns per thread
  static_assert(QS % 4 == 0 && VS % 4 == 0, "whole float4 runs");
  __shared__ __attribute__((aligned(16))) float tile[MLA32_TILE][D];
  __shared__ int vflag[MLA32_TILE];
  const int split = blockIdx.x;
  const int q = blockIdx.y;
  const int layer = blockIdx.z;
  const int tid = threadIdx.x;
  const int part = tid & (MLA32_PARTS - 1);
  const int head0 = (tid / MLA32_PARTS) * MLA32_HPT;
  const QueryRange r = query_range(p.b, q);
  const int j_begin = split * p.split_len;
  const int j_end = min(j_begin + p.split_len, p.k);
  const float* kv = (const float*)p.L.kv[layer] + r.row0 * D;
  const int32_t* sel = p.idx + (int64_t)q * p.k;
  float qr[MLA32_HPT][QS];
#pragma unroll
  for (int h = 0; h < MLA32_HPT; ++h) {
    const float4* qp = (const float4*)((const float*)p.L.q[layer] + ((int64_t)q * H + head0 + h) * D + part * QS);
#pragma unroll
    for (int i = 0; i < QS / 4; ++i) {
      const float4 v = qp[i];
      qr[h][4 * i] = v.x;
      qr[h][4 * i + 1] = v.y;
      qr[h][4 * i + 2] = v.z;
      qr[h][4 * i + 3] = v.w;
    }
  }
  float acc[MLA32_HPT][VS];
  float m_run[MLA32_HPT], l_run[MLA32_HPT];
#pragma unroll
  for (int h = 0; h < MLA32_HPT; ++h) {
    m_run[h] = -INFINITY;
    l_run[h] = 0.0f;
#pragma unroll
    for (int i = 0; i < VS; ++i) acc[h][i] = 0.0f;
  }
  constexpr int NV = MLA32_TILE * D / 4;  // float4s per tile
  constexpr int PER = (NV + MLA32_THREADS - 1) / MLA32_THREADS;
  float4 nxt[PER];
  bool nok[PER];
  auto fetch = [&](int j0) {
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int c = tid + u * MLA32_THREADS;
      const int rr = c / (D / 4);
      const int ch = c - rr * (D / 4);
      const int j = j0 + rr;
      const int pos = (c < NV && j < j_end) ? sel[j] : -1;
      nok[u] = pos >= 0 && pos < r.n;
      DSA_CHECK(c >= NV || ch != 0 || (pos >= -1 && pos < r.n), DBG_IDX_RANGE);
      nxt[u] = c < NV ? ((const float4*)(kv + (int64_t)(nok[u] ? pos : 0) * D))[ch] : float4{0.f, 0.f, 0.f, 0.f};
    }
  };
  if (j_begin < j_end && r.n > 0) fetch(j_begin);
  for (int j0 = j_begin; j0 < j_end && r.n > 0; j0 += MLA32_TILE) {
    __syncthreads();  // the previous tile is consumed
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int c = tid + u * MLA32_THREADS;
      if (c < NV) {
        const int rr = c / (D / 4);
        const int ch = c - rr * (D / 4);
        ((float4*)tile[rr])[ch] = nxt[u];
        if (ch == 0) vflag[rr] = nok[u];
      }
    }
    __syncthreads();
    if (j0 + MLA32_TILE < j_end) fetch(j0 + MLA32_TILE);
    for (int rr = 0; rr < MLA32_TILE; ++rr) {
      if (!vflag[rr]) continue;
      const float4* krow = (const float4*)(tile[rr] + part * QS);
      float dot[MLA32_HPT] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int i = 0; i < QS / 4; ++i) {
        const float4 v = krow[i];
#pragma unroll
        for (int h = 0; h < MLA32_HPT; ++h) {
          dot[h] = fmaf(qr[h][4 * i], v.x, dot[h]);
          dot[h] = fmaf(qr[h][4 * i + 1], v.y, dot[h]);
          dot[h] = fmaf(qr[h][4 * i + 2], v.z, dot[h]);
          dot[h] = fmaf(qr[h][4 * i + 3], v.w, dot[h]);
        }
      }
      // lazy rescaling: the running max (log2 units) moves only when a logit
      // exceeds it by more than MLA_RESCALE_SLACK, so weights stay <= 2^8
      // and the value update is one multiply-add
      float pw[MLA32_HPT];
      bool resc_any = false;
      float alpha[MLA32_HPT];
#pragma unroll
      for (int h = 0; h < MLA32_HPT; ++h) {
        const float x = row16_sum(dot[h]) * p.scale_log2;
        const bool resc = x > m_run[h] + MLA_RESCALE_SLACK;
        alpha[h] = resc ? exp2f(m_run[h] - x) : 1.0f;
        if (resc) m_run[h] = x;
        resc_any |= resc;
        pw[h] = exp2f(x - m_run[h]);
        l_run[h] = l_run[h] * alpha[h] + pw[h];
      }
      if (__any(resc_any)) {
#pragma unroll
        for (int h = 0; h < MLA32_HPT; ++h)
#pragma unroll
          for (int i = 0; i < VS; ++i) acc[h][i] *= alpha[h];
      }
      const float4* vrow = (const float4*)(tile[rr] + part * VS);
#pragma unroll
      for (int i = 0; i < VS / 4; ++i) {
        const float4 v = vrow[i];
#pragma unroll
        for (int h = 0; h < MLA32_HPT; ++h) {
          acc[h][4 * i] = fmaf(pw[h], v.x, acc[h][4 * i]);
          acc[h][4 * i + 1] = fmaf(pw[h], v.y, acc[h][4 * i + 1]);
          acc[h][4 * i + 2] = fmaf(pw[h], v.z, acc[h][4 * i + 2]);
          acc[h][4 * i + 3] = fmaf(pw[h], v.w, acc[h][4 * i + 3]);
        }
      }
    }
  }
#pragma unroll
  for (int h = 0; h < MLA32_HPT; ++h) {
    const int64_t qh = (int64_t)q * H + head0 + h;
    const float inv = l_run[h] > 0.0f ? 1.0f / l_run[h] : 0.0f;
    if (p.nsplit == 1) {
#pragma unroll
      for (int i = 0; i < VS; i += 4)
        store_out4(p, layer, qh * DC + part * VS + i,
                   f32x4{acc[h][i] * inv, acc[h][i + 1] * inv, acc[h][i + 2] * inv, acc[h][i + 3] * inv});
      if (part == 0 && p.L.lse[layer])
        p.L.lse[layer][qh] = l_run[h] > 0.0f ? (m_run[h] + log2f(l_run[h])) * LN2 : -INFINITY;
    } else {
      const int64_t slot = ((int64_t)split * p.n_layers + layer) * p.b.nq * H + qh;
      float* pa = (float*)p.part_o + slot * DC + part * VS;
#pragma unroll
      for (int i = 0; i < VS; i += 4)
        *(f32x4*)(pa + i) = f32x4{acc[h][i] * inv, acc[h][i + 1] * inv, acc[h][i + 2] * inv, acc[h][i + 3] * inv};
      if (part == 0) {
        p.part_ml[slot * 2 + 0] = l_run[h] > 0.0f ? m_run[h] : -INFINITY;
        p.part_ml[slot * 2 + 1] = l_run[h];
      }
    }
  }
}

// ---------------------------------------------------------------------------
// log-sum-exp merge of the splits of each (query, layer)
// ---------------------------------------------------------------------------
// One wave per (head, query, layer): lane i < nsplit holds split i's
// (max, sum), so the merge weights w_i = 2^(m_i - M) l_i come from two wave
// reductions; then lane l adds up latent columns [8l, 8l + 8) of every
// split's normalised output, four splits' loads in flight at a time.  An
// empty split (max -inf) weighs 0.
constexpr int CMB_THREADS = 256;   // four heads per workgroup
constexpr int CMB_BATCH = 4;

__device__ inline float wave_max(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
  return x;
}
__device__ inline float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o);
  return x;
}

// Eight latent values of a split output: bf16 (one 16-byte load) or
// float32 (two).
template <bool BF16>
__device__ inline void load8(const void* base, int64_t off, float (&v)[8]) {
  if (BF16) {
    const u32x4 x = *(const u32x4*)((const uint16_t*)base + off);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = __uint_as_float(x[i] << 16);
      v[2 * i + 1] = __uint_as_float(x[i] & 0xFFFF0000u);
    }
  } else {
    const f32x4 a = *(const f32x4*)((const float*)base + off);
    const f32x4 c = *(const f32x4*)((const float*)base + off + 4);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[i] = a[i];
      v[4 + i] = c[i];
    }
  }
}

template <bool BF16>
__global__ __launch_bounds__(CMB_THREADS) void mla_combine(MlaParams p) {
  constexpr int HG = H / (CMB_THREADS / 64);  // head groups per (query, layer)
  const int item = xcd_item(blockIdx.x, HG * p.b.nq * p.n_layers);
  const int head = (item % HG) * (CMB_THREADS / 64) + (threadIdx.x >> 6);
  const int q = (item / HG) % p.b.nq;
  const int layer = item / (HG * p.b.nq);
  const int lane = threadIdx.x & 63;
  const int64_t qh = (int64_t)q * H + head;
  const int64_t stride = (int64_t)p.n_layers * p.b.nq * H;  // slots between splits
  const int64_t slot0 = (int64_t)layer * p.b.nq * H + qh;
  float mi = -INFINITY, li = 0.0f;
  if (lane < p.nsplit) {
    mi = p.part_ml[(slot0 + lane * stride) * 2];
    li = p.part_ml[(slot0 + lane * stride) * 2 + 1];
  }
  const float mx = wave_max(mi);
  const float wi = mi == -INFINITY ? 0.0f : exp2f(mi - mx) * li;
  const float den = wave_sum(wi);
  float acc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = 0.0f;
  for (int i0 = 0; i0 < p.nsplit; i0 += CMB_BATCH) {
    float val[CMB_BATCH][8];
    float w[CMB_BATCH];
#pragma unroll
    for (int c = 0; c < CMB_BATCH; ++c) {
      const int i = min(i0 + c, p.nsplit - 1);
      w[c] = i0 + c < p.nsplit ? __shfl(wi, i) : 0.0f;
      load8<BF16>(p.part_o, (slot0 + i * stride) * DC + 8 * lane, val[c]);
    }
#pragma unroll
    for (int c = 0; c < CMB_BATCH; ++c)
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] = fmaf(w[c], val[c][e], acc[e]);
  }
  const float inv = den > 0.0f ? 1.0f / den : 0.0f;
  const int64_t off = qh * DC + 8 * lane;
  store_out4(p, layer, off, f32x4{acc[0] * inv, acc[1] * inv, acc[2] * inv, acc[3] * inv});
  store_out4(p, layer, off + 4, f32x4{acc[4] * inv, acc[5] * inv, acc[6] * inv, acc[7] * inv});
  if (lane == 0 && p.L.lse[layer]) p.L.lse[layer][qh] = den > 0.0f ? (mx + log2f(den)) * LN2 : -INFINITY;
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------
#ifdef DSA_DEBUG
DSA_DEBUG_READER(debug_flags_mla)
#endif

hipError_t launch_mla(const BatchDev& b, int dtype, int rope, const MlaLayers& layers, int n_layers,
                      const int32_t* idx, int k, float scale, int out_dtype, void* ws,
                      size_t ws_bytes, hipStream_t st) {
  if (b.nq == 0 || n_layers == 0) return hipSuccess;
  MlaParams p;
  p.b = b;
  p.idx = idx;
  p.k = k;
  p.n_layers = n_layers;
  p.nsplit = mla_num_splits(dtype, b.nq, k, n_layers);
  p.split_len = mla_split_len(dtype, k, p.nsplit);
  p.nsplit = (k + p.split_len - 1) / p.split_len;
  p.out_bf16 = out_dtype == 1;
  p.scale_log2 = scale * 1.44269504088896340736f;
  p.L = layers;
  p.part_o = nullptr;
  p.part_ml = nullptr;
  if (p.nsplit > 1) {
    const size_t slots = (size_t)p.nsplit * n_layers * b.nq * H;
    if (ws == nullptr || ws_bytes < mla_workspace_bytes(dtype, b.nq, k, n_layers)) return hipErrorInvalidValue;
    p.part_o = ws;
    p.part_ml = (float*)((char*)ws + slots * DC * mla_partial_bytes(dtype));
  }
  dim3 grid(p.nsplit, b.nq, n_layers);
  if (dtype == 0) {
    if (rope)
      hipLaunchKernelGGL(mla_f32_kernel<DR>, grid, dim3(MLA32_THREADS), 0, st, p);
    else
      hipLaunchKernelGGL(mla_f32_kernel<0>, grid, dim3(MLA32_THREADS), 0, st, p);
  } else {
    const dim3 grid1(p.nsplit * b.nq * n_layers);
    if (rope)
      hipLaunchKernelGGL(mla_bf16_kernel<DR>, grid1, dim3(MLA_THREADS), 0, st, p);
    else
      hipLaunchKernelGGL(mla_bf16_kernel<0>, grid1, dim3(MLA_THREADS), 0, st, p);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.nsplit == 1) return e;
  const dim3 cgrid(H / (CMB_THREADS / 64) * b.nq * n_layers);
  if (dtype == 0)
    hipLaunchKernelGGL(mla_combine<false>, cgrid, dim3(CMB_THREADS), 0, st, p);
  else
    hipLaunchKernelGGL(mla_combine<true>, cgrid, dim3(CMB_THREADS), 0, st, p);
  return hipGetLastError();
}

}  // namespace dsa
