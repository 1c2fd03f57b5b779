// Launch planning shared by the kernels and the host side: the fixed shapes,
// the kernels' fixed geometry, the workspace layouts and the grid choices
// that depend on the batch shape.  Plain C++ with no HIP dependency, so the
// host side can be built and checked on its own.
#pragma once
#include <stddef.h>
#include <stdint.h>

namespace dsa {

// Shapes fixed by the concept page ("What to keep", "Where to look",
// "Sparse attention").
constexpr int HI = 32;    // indexer heads
constexpr int DI = 128;   // indexer head width
constexpr int H = 64;     // attention heads
constexpr int DC = 512;   // latent (= value) width
constexpr int DR = 64;    // rotary key width
constexpr int D = 576;    // cache row
constexpr int KMAX = 2048;

// ---------------------------------------------------------------------------
// top-k
// ---------------------------------------------------------------------------
constexpr int TK_THREADS = 1024;
constexpr int TK_BITS1 = 12;                 // first radix level: top 12 key bits
constexpr int TK_BINS1 = 1 << TK_BITS1;
constexpr int TK_SHIFT1 = 32 - TK_BITS1;
constexpr int TK_CHUNK = 8192;               // scores per workgroup in the split path
constexpr int TK_ROWS_SPLIT_MAX = 255;       // batches with more rows use one workgroup per row
constexpr int TK_ROW_MAX_LEN = 49152;        // rows up to this take one workgroup per row at any batch size

// Few rows longer than TK_ROW_MAX_LEN take the split path (it needs one
// finalize thread per chunk of the longest row).
bool topk_use_split(int nq, int max_len);

// Byte offsets of the split path's workspace parts.
struct TopkLayout {
  size_t hist;     // [nq][TK_BINS1] uint32  first-level histogram
  size_t bucket;   // [nq][4] uint32         threshold bucket, entries above it, entries in it
  size_t cnt;      // [nq][nchunk] uint32    candidate-list lengths
  size_t lkey;     // [nq][nchunk * TK_CHUNK] uint32
  size_t lpos;     // [nq][nchunk * TK_CHUNK] int32
  size_t bytes;    // total
  int nchunk;
};
TopkLayout topk_layout(int nq, int max_len);
size_t topk_workspace_bytes(int nq, int max_len, int k);

// ---------------------------------------------------------------------------
// indexer
// ---------------------------------------------------------------------------
constexpr int IDX_BAL_MAXQ = 1024;   // decode batches up to this many queries cut their keys evenly
constexpr int IDX_BAL_GRID = 512;    // workgroups of that kernel
constexpr int PF_QB = 32;            // queries per prefill workgroup
constexpr int PF_KC = 8192;          // keys per prefill workgroup (at most)
constexpr int PF_KC_MIN = 1024;      // shortest prefill key chunk
constexpr int PF_MIN_GRID = 512;     // prefill workgroups the chunk length aims for

enum class IndexKernel { F32, Prefill, Balanced, Chunked };
IndexKernel index_kernel(int dtype, int nq, int nseq);
// Keys per workgroup of the chunked decode grid.
int decode_key_chunk(int nq, int max_len);
// Keys per workgroup of the prefill grid.
int prefill_key_chunk(int nq, int max_len);

// ---------------------------------------------------------------------------
// sparse MLA
// ---------------------------------------------------------------------------
constexpr int MLA_TILE = 32;         // positions per bf16 tile
constexpr int MLA32_TILE = 8;        // positions per fp32 tile
int mla_num_splits(int dtype, int nq, int k, int n_layers);
int mla_split_len(int dtype, int k, int nsplit);
// Bytes per value of a split's output: bf16 for the bf16 kernel, float32
// for the fp32 one.
inline size_t mla_partial_bytes(int dtype) { return dtype == 0 ? 4 : 2; }
size_t mla_workspace_bytes(int dtype, int nq, int k, int n_layers);

// ---------------------------------------------------------------------------
// fused decode workspace
// ---------------------------------------------------------------------------
struct FusedLayout {
  int64_t score_ld;  // row stride of the scores: max_len rounded up to a multiple of 4 (16-byte rows)
  size_t scores;   // [nq][score_ld] float32
  size_t idx;      // [nq][k] int32 (when the caller passes no idx_out)
  size_t hist;     // [nq][TK_BINS1] uint32: the indexer's score histogram, zero between calls
  size_t topk;     // top-k workspace
  size_t mla;      // MLA split partials
  size_t bytes;    // total
};
// A launch over fewer layers can take more MLA splits: sized for every
// group of 1..n_layers layers, both element types.
FusedLayout fused_layout(int nq, int max_len, int k, int n_layers);

// ---------------------------------------------------------------------------
// rotary frequencies (host, double precision)
// ---------------------------------------------------------------------------
void rope_frequencies(const float* alpha, double* out);

}  // namespace dsa
