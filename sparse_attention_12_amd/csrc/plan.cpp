// Launch planning (see plan.h): workspace layouts and batch-shape-dependent
// grid choices, shared by the launchers and the C ABI layer.
#include "plan.h"

#include <math.h>

namespace dsa {

namespace {
size_t round256(size_t x) { return (x + 255) & ~(size_t)255; }
}  // namespace

// ---------------------------------------------------------------------------
// top-k
// ---------------------------------------------------------------------------
bool topk_use_split(int nq, int max_len) {
  return nq <= TK_ROWS_SPLIT_MAX && max_len > TK_ROW_MAX_LEN && (int64_t)max_len <= (int64_t)TK_THREADS * TK_CHUNK;
}

TopkLayout topk_layout(int nq, int max_len) {
  TopkLayout t;
  t.nchunk = (max_len + TK_CHUNK - 1) / TK_CHUNK;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off += round256(bytes);
    return at;
  };
  t.hist = take((size_t)nq * TK_BINS1 * 4);
  t.bucket = take((size_t)nq * 4 * 4);
  t.cnt = take((size_t)nq * t.nchunk * 4);
  t.lkey = take((size_t)nq * t.nchunk * TK_CHUNK * 4);
  t.lpos = take((size_t)nq * t.nchunk * TK_CHUNK * 4);
  t.bytes = off;
  return t;
}

size_t topk_workspace_bytes(int nq, int max_len, int k) {
  (void)k;
  if (nq <= 0 || max_len <= 0 || !topk_use_split(nq, max_len)) return 0;
  return topk_layout(nq, max_len).bytes;
}

// ---------------------------------------------------------------------------
// indexer
// ---------------------------------------------------------------------------
IndexKernel index_kernel(int dtype, int nq, int nseq) {
  if (dtype == 0) return IndexKernel::F32;
  // at least a block's worth of queries per sequence on average
  if (nq >= PF_QB && (int64_t)nq >= (int64_t)PF_QB * nseq) return IndexKernel::Prefill;
  if (nq <= IDX_BAL_MAXQ) return IndexKernel::Balanced;
  return IndexKernel::Chunked;
}

// The largest power of two in [512, 4096] that still gives about 2,048
// workgroups for the padded batch (nq x max_len), so short or ragged
// batches keep every compute unit streaming.
int decode_key_chunk(int nq, int max_len) {
  const int64_t keys = (int64_t)nq * max_len;
  int chunk = 4096;
  while (chunk > 512 && keys / chunk < 2048) chunk >>= 1;
  return chunk;
}

// Chunks of PF_KC keys, halved (to PF_KC_MIN at the shortest) while the grid
// has fewer than PF_MIN_GRID workgroups (few, short sequences).
int prefill_key_chunk(int nq, int max_len) {
  const int64_t nqb = (nq + PF_QB - 1) / PF_QB;
  int kc = PF_KC;
  while (kc > PF_KC_MIN && (int64_t)((max_len + kc - 1) / kc) * nqb < PF_MIN_GRID) kc >>= 1;
  return kc;
}

// ---------------------------------------------------------------------------
// sparse MLA
// ---------------------------------------------------------------------------
namespace {
constexpr int MLA_TARGET_BLOCKS = 256;  // one workgroup per compute unit
}

int mla_num_splits(int dtype, int nq, int k, int n_layers) {
  const int tile = dtype == 0 ? MLA32_TILE : MLA_TILE;
  const int max_split = (k + tile - 1) / tile;
  const int64_t base = (int64_t)nq * n_layers;
  int ns = base > 0 ? (int)((MLA_TARGET_BLOCKS + base - 1) / base) : 1;
  const int cap = dtype == 0 ? 64 : 16;
  ns = ns < cap ? ns : cap;
  ns = ns < max_split ? ns : max_split;
  return ns > 1 ? ns : 1;
}

int mla_split_len(int dtype, int k, int nsplit) {
  const int tile = dtype == 0 ? MLA32_TILE : MLA_TILE;
  const int len = (k + nsplit - 1) / nsplit;
  return (len + tile - 1) / tile * tile;
}

size_t mla_workspace_bytes(int dtype, int nq, int k, int n_layers) {
  const int ns = mla_num_splits(dtype, nq, k, n_layers);
  if (ns <= 1) return 0;
  const size_t slots = (size_t)ns * n_layers * nq * H;
  return slots * DC * mla_partial_bytes(dtype) + slots * 2 * sizeof(float);
}

// ---------------------------------------------------------------------------
// fused decode workspace
// ---------------------------------------------------------------------------
FusedLayout fused_layout(int nq, int max_len, int k, int n_layers) {
  FusedLayout f;
  size_t off = 0;
  f.score_ld = ((int64_t)max_len + 3) & ~(int64_t)3;
  f.scores = off;
  off = round256(off + (size_t)nq * (size_t)f.score_ld * sizeof(float));
  f.idx = off;
  off = round256(off + (size_t)nq * (size_t)k * sizeof(int32_t));
  f.hist = off;
  off = round256(off + (size_t)nq * TK_BINS1 * sizeof(uint32_t));
  f.topk = off;
  off = round256(off + topk_workspace_bytes(nq, max_len, k));
  f.mla = off;
  size_t m = 0;
  for (int n = 1; n <= n_layers; ++n)
    for (int dt = 0; dt < 2; ++dt) {
      const size_t x = mla_workspace_bytes(dt, nq, k, n);
      m = x > m ? x : m;
    }
  f.bytes = round256(off + m);
  return f;
}

// ---------------------------------------------------------------------------
// rotary frequencies
// ---------------------------------------------------------------------------
// Pair i of the rotary part turns at omega_i = 10000^(-i/32) radians per
// position.  Under YaRN (original window 512, stretch 2,048) a pair whose
// wavelength 2 pi / omega_i fits 32 times into the window is left alone, a
// pair whose wavelength is longer than the window is slowed by the full
// stretch, and the pairs between the longest unchanged and the shortest
// fully slowed wavelength are slowed by a factor interpolated linearly in
// the pair index; LeRoPE scales frequency i by the learned e^{alpha_i}.
void rope_frequencies(const float* alpha, double* out) {
  constexpr int pairs = DR / 2;
  const double window = 512.0, stretch = 2048.0, min_turns = 32.0;
  double omega[pairs];
  int longest_kept = -1, shortest_slowed = pairs;
  for (int i = 0; i < pairs; ++i) {
    omega[i] = exp(-log(10000.0) * (double)i / (double)pairs);
    const double wavelength = 2.0 * M_PI / omega[i];
    if (wavelength * min_turns <= window) longest_kept = i;                    // wavelengths grow with i
    if (wavelength > window && shortest_slowed == pairs) shortest_slowed = i;
  }
  for (int i = 0; i < pairs; ++i) {
    double ramp = (double)(i - longest_kept) / (double)(shortest_slowed - longest_kept);
    ramp = ramp < 0.0 ? 0.0 : (ramp > 1.0 ? 1.0 : ramp);
    double f = omega[i] * (1.0 - ramp * (1.0 - 1.0 / stretch));
    if (alpha) f *= exp((double)alpha[i]);
    out[i] = f;
  }
}

}  // namespace dsa
