// Sparse MLA read on gfx950 (concept page "Mistral Large 4", sections "What
// to keep", "Where to look" and "Sparse attention").  For query q with
// selected positions S (its row of idx), in absorbed form:
//   l[h][j] = scale * q[h][0:576] . kv[S_j][0:576]
//   o[h]    = sum_j softmax_j(l[h])[j] * kv[S_j][0:512]     (softmax over S only)
//   lse[h]  = log sum_j exp(l[h][j])
// 64 x (512 + 64 + 512) multiply-adds per selected position.
//
// bf16 kernel: one workgroup (4 waves) per (split of the selection, query,
// layer); wave w owns heads 16w..16w+15.  Per tile of 32 positions the
// 576-wide bf16 rows are gathered into LDS, then
//   S^T (32 positions x 16 heads) = K_tile . Q_w^T   (18 MFMA 16x16x32 per block)
//   online softmax in the exp2 domain, rescaling the accumulator only when a
//   head's running max grows by more than 2^8
//   O_w^T (512 x 16) += V_tile^T . P^T               (32 MFMA 16x16x32)
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
  float* part_acc;   // [nsplit][n_layers][nq][64][512]
  float* part_ml;    // [nsplit][n_layers][nq][64][2]  (max in log2 units, sum)
  MlaLayers L;
};

constexpr float LN2 = 0.69314718055994530942f;

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
constexpr int MLA_THREADS = 256;
constexpr int MLA_TILE = 32;                    // positions per tile
constexpr int MLA_ROWB = D * 2;                 // 1,152 bytes per bf16 row
constexpr int MLA_CHUNKS = MLA_ROWB / 16;       // 72 chunks of 16 B per row
constexpr int MLA_TILEB = MLA_TILE * MLA_ROWB;  // 36,864 bytes per tile
constexpr int MLA_NBUF = 2;
constexpr int MLA_SPLIT_MAX = KMAX;
static_assert(MLA_TILE * 8 == MLA_THREADS, "one gathering thread per (row, in-group chunk)");
constexpr float MLA_RESCALE_SLACK = 8.0f;       // log2 units

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
typedef __attribute__((address_space(3))) void lds_void;

// LDS tile layout (36,864 bytes): nine column groups of 64 latent/rotary
// values; group G holds rows 0..31 at 128 bytes each, and row r's logical
// 16-byte chunk c (of the group's eight) sits at chunk slot c ^ (r & 7).
// One gather instruction of wave w fills rows 8w..8w+7 of one group: 1 KB,
// written in lane order.
constexpr int MLA_GROUPB = MLA_TILE * 128;  // 4,096 bytes per column group

__device__ inline int tile_off(int row, int chunk) {
  return (chunk >> 3) * MLA_GROUPB + row * 128 + (((chunk & 7) ^ (row & 7)) << 4);
}

struct MlaTileState {
  f32x4 o[DC / 16];
  float m_run;
  float l_part;
};

// Gather tile t of the selection straight into LDS.  Thread (wave w, lane l)
// fetches row 8w + l/8 of the tile: for each column group i, the 16-byte
// chunk ((l % 8) ^ (row & 7)) + 8i, which lands at lane slot l of the 1 KB
// block of (group i, rows 8w..8w+7).
__device__ inline void mla_issue(uint8_t* buf, const uint16_t* kv, const int* sel_l, int nent, int t, int lane,
                                 int wave_u) {
  const int row = wave_u * 8 + (lane >> 3);
  const int j = t * MLA_TILE + row;
  const int pos = j < nent ? sel_l[j] : -1;
  const uint16_t* src = kv + (int64_t)(pos >= 0 ? pos : 0) * D + (((lane & 7) ^ (row & 7)) << 3);
  uint8_t* dst = buf + wave_u * 1024;
#pragma unroll
  for (int i = 0; i < D * 2 / 128; ++i)
    __builtin_amdgcn_global_load_lds((const void*)(src + i * 64), (lds_void*)(dst + i * MLA_GROUPB), 16, 0, 0);
}

// One tile: S^T = K.Q^T, online softmax, O^T += V^T.P^T.
__device__ inline void mla_tile(MlaTileState& st, const uint8_t* tile, const bf16x8 (&qf)[D / 32],
                                const int* sel_l, int nent, int t0, int n16, int g, float scale_log2) {
  // Row r's logical chunk 4t+g lies in column group t/2 at in-group chunk
  // 4*(t%2) + g: two base addresses per row plus an immediate 4096*(t/2).
  // Loads run two steps ahead of the MFMAs; each block keeps two
  // accumulator chains.
  const uint8_t* ev[2];
  const uint8_t* od[2];
#pragma unroll
  for (int mb = 0; mb < 2; ++mb) {
    const int row = 16 * mb + n16;
    ev[mb] = tile + tile_off(row, g);
    od[mb] = tile + tile_off(row, 4 + g);
  }
  auto kfrag = [&](int mb, int t) -> u32x4 {
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
  for (int t = 0; t < D / 32; ++t) {
    if (t + 2 < D / 32) {
      ring[(t + 2) % 3][0] = kfrag(0, t + 2);
      ring[(t + 2) % 3][1] = kfrag(1, t + 2);
    }
    acc[0][t & 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(ring[t % 3][0]), qf[t], acc[0][t & 1], 0, 0, 0);
    acc[1][t & 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(ring[t % 3][1]), qf[t], acc[1][t & 1], 0, 0, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);  // 2 LDS reads
    __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);  // 2 MFMAs
  }
  f32x4 s[2];
  s[0] = acc[0][0] + acc[0][1];
  s[1] = acc[1][0] + acc[1][1];
  __builtin_amdgcn_sched_barrier(0);
  // lane holds one head and positions 16*mb + 4g + i
  float x[8];
  float tmax = -INFINITY;
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int j = t0 + 16 * mb + 4 * g + i;
      const bool ok = j < nent && sel_l[j] >= 0;
      const float v = ok ? s[mb][i] * scale_log2 : -INFINITY;
      x[mb * 4 + i] = v;
      tmax = fmaxf(tmax, v);
    }
  tmax = fmaxf(tmax, __shfl_xor(tmax, 16));
  tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
  const bool resc = tmax > st.m_run + MLA_RESCALE_SLACK;
  if (__any(resc)) {
    const float alpha = resc ? exp2f(st.m_run - tmax) : 1.0f;
    if (resc) st.m_run = tmax;
    st.l_part *= alpha;
#pragma unroll
    for (int db = 0; db < DC / 16; ++db) st.o[db] *= alpha;
  }
  float pv[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    pv[e] = (x[e] == -INFINITY) ? 0.0f : exp2f(x[e] - st.m_run);
    st.l_part += pv[e];
  }
  u32x4 pk;
  pk[0] = pack_bf16x2(pv[0], pv[1]);
  pk[1] = pack_bf16x2(pv[2], pv[3]);
  pk[2] = pack_bf16x2(pv[4], pv[5]);
  pk[3] = pack_bf16x2(pv[6], pv[7]);
  const bf16x8 pb = as_bf16x8(pk);
  __builtin_amdgcn_sched_barrier(0);

  // O^T += V_tile^T . P^T.  k-slot e of lane group g is tile row
  // (e < 4 ? 4g + e : 16 + 4g + e - 4).  A transposing LDS read gives lane
  // i of a 16-lane group element i%4 of source lane 4j + i/4, so source
  // lane s points at row 4g + s/4 (+16) and latent column 16db + 4(s%4).
  // Column 16db + sdim lies in column group db/4, in-group chunk
  // 2*(db%4) + sdim/8: four base addresses per source row plus an
  // immediate 4096*(db/4).
  const int srow0 = 4 * g + (n16 >> 2);
  const int srow1 = srow0 + 16;
  const int sdim = 4 * (n16 & 3);
  const int c0 = sdim >> 3;
  const int boff = (sdim & 7) << 1;
  const uint8_t* b0[4];
  const uint8_t* b1[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    b0[u] = tile + tile_off(srow0, 2 * u + c0) + boff;
    b1[u] = tile + tile_off(srow1, 2 * u + c0) + boff;
  }
  auto vfrag = [&](int db) -> bf16x8 {
    const int u = db & 3;
    const int imm = (db >> 2) * MLA_GROUPB;
    const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(b0[u] + imm));
    const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(b1[u] + imm));
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
  };
  bf16x8 vr[4];
  vr[0] = vfrag(0);
  vr[1] = vfrag(1);
  vr[2] = vfrag(2);
#pragma unroll
  for (int db = 0; db < DC / 16; ++db) {
    if (db + 3 < DC / 16) vr[(db + 3) & 3] = vfrag(db + 3);
    st.o[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vr[db & 3], pb, st.o[db], 0, 0, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 2, 1);  // 2 LDS transpose reads
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 1);  // 1 MFMA
  }
}

__global__ __launch_bounds__(MLA_THREADS, 2) void mla_bf16_kernel(MlaParams p) {
  // two distinct arrays, so that reads of one tile are known not to alias
  // the asynchronous gather into the other
  __shared__ __attribute__((aligned(16))) uint8_t tile0[MLA_TILEB];
  __shared__ __attribute__((aligned(16))) uint8_t tile1[MLA_TILEB];
  __shared__ int sel_l[MLA_SPLIT_MAX];
  const int split = blockIdx.x;
  const int q = blockIdx.y;
  const int layer = blockIdx.z;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave_u = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n16 = lane & 15;
  const int g = lane >> 4;
  const QueryRange r = query_range(p.b, q);
  const int j_begin = split * p.split_len;
  const int nent = max(0, min(j_begin + p.split_len, p.k) - j_begin);
  const int ntiles = r.n > 0 ? (nent + MLA_TILE - 1) / MLA_TILE : 0;
  const int head = wave_u * 16 + n16;

  // this split's selected positions; entries outside [0, n) become -1
  {
    const int32_t* sel = p.idx + (int64_t)q * p.k + j_begin;
    for (int j = tid; j < nent; j += MLA_THREADS) {
      const int pos = sel[j];
      sel_l[j] = (pos >= 0 && pos < r.n) ? pos : -1;
    }
  }
  // Q_w^T as the B operand: head `head`, contraction slots t*32 + 8g + [0,8)
  bf16x8 qf[D / 32];
  {
    const uint16_t* qp = (const uint16_t*)p.L.q[layer] + ((int64_t)q * H + head) * D + g * 8;
#pragma unroll
    for (int t = 0; t < D / 32; ++t) qf[t] = as_bf16x8(load16(qp + t * 32));
  }
  const uint16_t* kv = (const uint16_t*)p.L.kv[layer] + r.row0 * D;
  MlaTileState st;
#pragma unroll
  for (int db = 0; db < DC / 16; ++db) st.o[db] = f32x4{0.f, 0.f, 0.f, 0.f};
  st.m_run = -INFINITY;
  st.l_part = 0.0f;
  __syncthreads();

  if (ntiles > 0) mla_issue(tile0, kv, sel_l, nent, 0, lane, wave_u);
  for (int it = 0; it < ntiles; it += 2) {
    __builtin_amdgcn_s_waitcnt(0x3F70);  // vmcnt(0): this thread's part of tile `it` landed
    __syncthreads();                     // every part landed; the other buffer is free
    if (it + 1 < ntiles) mla_issue(tile1, kv, sel_l, nent, it + 1, lane, wave_u);
    mla_tile(st, tile0, qf, sel_l, nent, it * MLA_TILE, n16, g, p.scale_log2);
    if (it + 1 >= ntiles) break;
    __builtin_amdgcn_s_waitcnt(0x3F70);
    __syncthreads();
    if (it + 2 < ntiles) mla_issue(tile0, kv, sel_l, nent, it + 2, lane, wave_u);
    mla_tile(st, tile1, qf, sel_l, nent, (it + 1) * MLA_TILE, n16, g, p.scale_log2);
  }

  float l_part = st.l_part;
  l_part += __shfl_xor(l_part, 16);
  l_part += __shfl_xor(l_part, 32);
  const int64_t qh = (int64_t)q * H + head;
  if (p.nsplit == 1) {
    const float inv = l_part > 0.0f ? 1.0f / l_part : 0.0f;
#pragma unroll
    for (int db = 0; db < DC / 16; ++db) store_out4(p, layer, qh * DC + db * 16 + 4 * g, st.o[db] * inv);
    if (g == 0 && p.L.lse[layer])
      p.L.lse[layer][qh] = l_part > 0.0f ? (st.m_run + log2f(l_part)) * LN2 : -INFINITY;
  } else {
    const int64_t slot = ((int64_t)split * p.n_layers + layer) * p.b.nq * H + qh;
    float* acc = p.part_acc + slot * DC;
#pragma unroll
    for (int db = 0; db < DC / 16; ++db) *(f32x4*)(acc + db * 16 + 4 * g) = st.o[db];
    if (g == 0) {
      p.part_ml[slot * 2 + 0] = l_part > 0.0f ? st.m_run : -INFINITY;
      p.part_ml[slot * 2 + 1] = l_part;
    }
  }
}

// ---------------------------------------------------------------------------
// fp32 split kernel (VALU; small fp32 workloads)
// ---------------------------------------------------------------------------
constexpr int MLA32_THREADS = 256;
constexpr int MLA32_TILE = 8;

__global__ __launch_bounds__(MLA32_THREADS) void mla_f32_kernel(MlaParams p) {
  __shared__ __attribute__((aligned(16))) float tile[MLA32_TILE][D];
  __shared__ int vflag[MLA32_TILE];
  const int split = blockIdx.x;
  const int q = blockIdx.y;
  const int layer = blockIdx.z;
  const int tid = threadIdx.x;
  const int head = tid >> 2;   // 4 threads per head
  const int part = tid & 3;    // quarter of the contraction / of the value dims
  const QueryRange r = query_range(p.b, q);
  const int j_begin = split * p.split_len;
  const int j_end = min(j_begin + p.split_len, p.k);
  const float* kv = (const float*)p.L.kv[layer] + r.row0 * D;
  const int32_t* sel = p.idx + (int64_t)q * p.k;
  constexpr int QS = D / 4;   // 144 contraction dims per thread
  constexpr int VS = DC / 4;  // 128 value dims per thread
  float qr[QS];
  {
    const float* qp = (const float*)p.L.q[layer] + ((int64_t)q * H + head) * D + part * QS;
#pragma unroll
    for (int i = 0; i < QS; ++i) qr[i] = qp[i];
  }
  float acc[VS];
#pragma unroll
  for (int i = 0; i < VS; ++i) acc[i] = 0.0f;
  float m_run = -INFINITY, l_run = 0.0f;
  for (int j0 = j_begin; j0 < j_end && r.n > 0; j0 += MLA32_TILE) {
    __syncthreads();
    for (int c = tid; c < MLA32_TILE * D / 4; c += MLA32_THREADS) {
      const int rr = c / (D / 4);
      const int ch = c - rr * (D / 4);
      const int j = j0 + rr;
      const int pos = j < j_end ? sel[j] : -1;
      const bool ok = pos >= 0 && pos < r.n;
      ((float4*)tile[rr])[ch] = ((const float4*)(kv + (int64_t)(ok ? pos : 0) * D))[ch];
      if (ch == 0) vflag[rr] = ok;
    }
    __syncthreads();
    for (int rr = 0; rr < MLA32_TILE; ++rr) {
      if (!vflag[rr]) continue;
      const float* row = tile[rr];
      float dot = 0.0f;
#pragma unroll
      for (int i = 0; i < QS; ++i) dot = fmaf(qr[i], row[part * QS + i], dot);
      dot += __shfl_xor(dot, 1);
      dot += __shfl_xor(dot, 2);
      const float x = dot * p.scale_log2;
      const float m_new = fmaxf(m_run, x);
      const float alpha = exp2f(m_run - m_new);
      const float pw = exp2f(x - m_new);
      l_run = l_run * alpha + pw;
#pragma unroll
      for (int i = 0; i < VS; ++i) acc[i] = fmaf(acc[i], alpha, pw * row[part * VS + i]);
      m_run = m_new;
    }
  }
  const int64_t qh = (int64_t)q * H + head;
  if (p.nsplit == 1) {
    const float inv = l_run > 0.0f ? 1.0f / l_run : 0.0f;
#pragma unroll
    for (int i = 0; i < VS; i += 4)
      store_out4(p, layer, qh * DC + part * VS + i,
                 f32x4{acc[i] * inv, acc[i + 1] * inv, acc[i + 2] * inv, acc[i + 3] * inv});
    if (part == 0 && p.L.lse[layer])
      p.L.lse[layer][qh] = l_run > 0.0f ? (m_run + log2f(l_run)) * LN2 : -INFINITY;
  } else {
    const int64_t slot = ((int64_t)split * p.n_layers + layer) * p.b.nq * H + qh;
    float* pa = p.part_acc + slot * DC + part * VS;
#pragma unroll
    for (int i = 0; i < VS; i += 4) *(f32x4*)(pa + i) = f32x4{acc[i], acc[i + 1], acc[i + 2], acc[i + 3]};
    if (part == 0) {
      p.part_ml[slot * 2 + 0] = l_run > 0.0f ? m_run : -INFINITY;
      p.part_ml[slot * 2 + 1] = l_run;
    }
  }
}

// ---------------------------------------------------------------------------
// log-sum-exp merge of the splits of each (query, layer)
// ---------------------------------------------------------------------------
constexpr int CMB_THREADS = 256;
constexpr int CMB_HEADS = 8;   // heads per workgroup: 32 threads x 16 values each

__global__ __launch_bounds__(CMB_THREADS) void mla_combine(MlaParams p) {
  const int q = blockIdx.x;
  const int layer = blockIdx.y;
  const int head = blockIdx.z * CMB_HEADS + (threadIdx.x >> 5);
  const int part = threadIdx.x & 31;
  constexpr int VS = DC / 32;   // 16 value dims per thread
  const int64_t qh = (int64_t)q * H + head;
  const int64_t stride = (int64_t)p.n_layers * p.b.nq * H;  // slots between splits
  const int64_t slot0 = (int64_t)layer * p.b.nq * H + qh;
  float mx = -INFINITY;
  for (int i = 0; i < p.nsplit; ++i) mx = fmaxf(mx, p.part_ml[(slot0 + i * stride) * 2]);
  f32x4 acc[VS / 4];
#pragma unroll
  for (int v = 0; v < VS / 4; ++v) acc[v] = f32x4{0.f, 0.f, 0.f, 0.f};
  float den = 0.0f;
  if (mx != -INFINITY) {
    for (int i = 0; i < p.nsplit; ++i) {
      const int64_t slot = slot0 + i * stride;
      const float mi = p.part_ml[slot * 2];
      if (mi == -INFINITY) continue;
      const float wgt = exp2f(mi - mx);
      den += wgt * p.part_ml[slot * 2 + 1];
      const f32x4* pa = (const f32x4*)(p.part_acc + slot * DC) + part;
#pragma unroll
      for (int v = 0; v < VS / 4; ++v) acc[v] += wgt * pa[32 * v];
    }
  }
  const float inv = den > 0.0f ? 1.0f / den : 0.0f;
#pragma unroll
  for (int v = 0; v < VS / 4; ++v) store_out4(p, layer, qh * DC + 4 * (part + 32 * v), acc[v] * inv);
  if (part == 0 && p.L.lse[layer]) p.L.lse[layer][qh] = den > 0.0f ? (mx + log2f(den)) * LN2 : -INFINITY;
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------
constexpr int MLA_TARGET_BLOCKS = 512;  // two workgroups per compute unit

int mla_num_splits(int dtype, int nq, int k, int n_layers) {
  const int tile = dtype == 0 ? MLA32_TILE : MLA_TILE;
  const int max_split = (k + tile - 1) / tile;
  const int base = nq * n_layers;
  int ns = base > 0 ? (MLA_TARGET_BLOCKS + base - 1) / base : 1;
  const int cap = dtype == 0 ? 64 : 16;
  ns = min(ns, min(cap, max_split));
  return max(ns, 1);
}

static int split_len_of(int dtype, int k, int ns) {
  const int tile = dtype == 0 ? MLA32_TILE : MLA_TILE;
  int len = (k + ns - 1) / ns;
  return (len + tile - 1) / tile * tile;
}

size_t mla_workspace_bytes(int dtype, int nq, int k, int n_layers) {
  const int ns = mla_num_splits(dtype, nq, k, n_layers);
  if (ns <= 1) return 0;
  const size_t slots = (size_t)ns * n_layers * nq * H;
  return slots * DC * sizeof(float) + slots * 2 * sizeof(float);
}

hipError_t launch_mla(const BatchDev& b, int dtype, const MlaLayers& layers, int n_layers,
                      const int32_t* idx, int k, float scale, int out_dtype, void* ws,
                      size_t ws_bytes, hipStream_t st) {
  if (b.nq == 0 || n_layers == 0) return hipSuccess;
  MlaParams p;
  p.b = b;
  p.idx = idx;
  p.k = k;
  p.n_layers = n_layers;
  p.nsplit = mla_num_splits(dtype, b.nq, k, n_layers);
  p.split_len = split_len_of(dtype, k, p.nsplit);
  p.nsplit = (k + p.split_len - 1) / p.split_len;
  p.out_bf16 = out_dtype == 1;
  p.scale_log2 = scale * 1.44269504088896340736f;
  p.L = layers;
  p.part_acc = nullptr;
  p.part_ml = nullptr;
  if (p.nsplit > 1) {
    const size_t slots = (size_t)p.nsplit * n_layers * b.nq * H;
    if (ws == nullptr || ws_bytes < mla_workspace_bytes(dtype, b.nq, k, n_layers)) return hipErrorInvalidValue;
    p.part_acc = (float*)ws;
    p.part_ml = (float*)ws + slots * DC;
  }
  dim3 grid(p.nsplit, b.nq, n_layers);
  if (dtype == 0)
    hipLaunchKernelGGL(mla_f32_kernel, grid, dim3(MLA32_THREADS), 0, st, p);
  else
    hipLaunchKernelGGL(mla_bf16_kernel, grid, dim3(MLA_THREADS), 0, st, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.nsplit == 1) return e;
  hipLaunchKernelGGL(mla_combine, dim3(b.nq, n_layers, H / CMB_HEADS), dim3(CMB_THREADS), 0, st, p);
  return hipGetLastError();
}

}  // namespace dsa
