// Internal interface between the C ABI (pq_api.cpp) and the kernels
// (pq_kernels.hip).  Not installed; the public header is include/pq.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pq.h"

namespace pqi {

constexpr int kMaxBits = 8;
constexpr int kMaxCells = 640;          // 583 cells at 8 bits

// fp32 codebook and the geometry of the uniform search grid the kernels build
// in LDS: cell k (0 <= k < ncell) is centred on (k - half) w and stores the
// boundary nearest to its centre together with the codes and centroids on
// both sides, so code = base + (y > boundary) is exact for every y that rounds
// to the cell (w is 0.9 of the smallest boundary gap).  Each cell is stored
// nrep times so that the 16 lanes of one LDS access group read distinct banks.
struct CodecTables {
  float cent[1 << kMaxBits];
  float beta[(1 << kMaxBits) - 1];
  uint8_t cell_best[kMaxCells];   // index of the boundary nearest to each cell's centre
  int nbound;
  int ncell;        // 2 * half + 1
  int half;
  int nrep;         // copies of each cell (16: one per lane of a 16-lane group, else 1)
  float cell_w;
  float cell_inv_w;
};

struct QuantArgs {
  const void* x;
  int64_t n_blocks;
  const uint8_t* signs;
  const uint16_t* proj;
  uint8_t* codes;
  uint16_t* norms;
  uint8_t* qbits;
  uint16_t* rnorms;
  int m;
  int pbits;          // 0: a byte per code; 1..7: codes bit-packed at pbits bits each
  CodecTables t;
};

struct DequantArgs {
  const uint8_t* codes;
  const uint16_t* norms;
  int64_t n_blocks;
  const uint8_t* signs;
  void* out;
  int pbits;          // as in QuantArgs
  CodecTables t;
};

struct SketchArgs {
  const uint16_t* keys;
  int64_t n_keys;
  const uint16_t* proj;
  uint8_t* bits;
  uint16_t* norms;
  int m;
  // optional split by outlier channels (oidx == nullptr: the whole key): key t of a head
  // (n_keys = heads * seq_len) belongs to group t / group_size, whose n_out channels are
  // oidx[(head * n_groups + group) * n_out ..]; part 0 sketches the key without them,
  // part 1 the key on them only
  const uint8_t* oidx;
  int64_t seq_len, n_groups;
  int group_size, n_out, part;
};

struct OutlierArgs {
  const uint16_t* keys;    // [n_heads][seq_len][d] bf16
  int64_t n_heads, seq_len, n_groups;
  int d, group_size, n_out;
  uint8_t* oidx;           // [n_heads][n_groups][n_out]
};

struct ProjectArgs {
  const uint16_t* q;
  int64_t n_q;
  const uint16_t* proj;
  float* sq;               // row i at sq + (i / rows_per_group) * group_stride + (i % rows_per_group) * m
  int d;
  int m;
  int64_t rows_per_group;  // n_q for a plain [n_q][m] output
  int64_t group_stride;    // in floats
};

struct ScoreArgs {
  const float* sq;
  const uint8_t* bits;
  const uint16_t* norms;
  float* scores;
  int64_t n_keys;
  int m;
  int batch;
  int kv_heads;
  int q_heads;
  int accumulate;          // add the estimate to the scores already there
};

// Prepared queries of the two-stage score, per KV head (byte offsets from the head's
// start; stride prep_head_bytes(d, m)):
//   qrot   float[16][d]   H (D q) of query row r (rows >= n_q are zero)
//   sq     float[16][m]   G q
//   meta   float scale[2][16] (code term, QJL term), int32 isum[2][16]
//   frag_c int8 limbs of rint(qrot / scale) in MFMA A-fragment order, 3 x (d/64) x 1 KiB
//   frag_q the same for sq, 3 x (m/64) x 1 KiB
constexpr int kScoreRows = 16;
constexpr int kMaxScoreBits = 4;
constexpr int kMaxPlanes = 1 << (kMaxScoreBits - 1);
constexpr float kLimbRange = 2080768.0f;       // 127 * 16384 + 127 * 128 + 127

__host__ __device__ constexpr int64_t prep_off_sq(int d) { return (int64_t)kScoreRows * d * 4; }
__host__ __device__ constexpr int64_t prep_off_meta(int d, int m) { return prep_off_sq(d) + (int64_t)kScoreRows * m * 4; }
__host__ __device__ constexpr int64_t prep_off_frag_c(int d, int m) { return prep_off_meta(d, m) + 256; }
__host__ __device__ constexpr int64_t prep_off_frag_q(int d, int m) { return prep_off_frag_c(d, m) + 3 * (d / 64) * 1024; }
__host__ __device__ constexpr int64_t prep_head_bytes(int d, int m) { return prep_off_frag_q(d, m) + 3 * (m / 64) * 1024; }

// p-th subset (in increasing order of its bit mask) of the code bits {0 .. bits-1} with
// an odd number of elements.
__host__ __device__ constexpr uint32_t plane_mask(int bits, int p) {
  int seen = 0;
  for (uint32_t mask = 1; mask < (1u << bits); ++mask) {
    if (__builtin_popcount(mask) & 1) {
      if (seen == p) return mask;
      ++seen;
    }
  }
  return 0;
}

struct QueryPrepArgs {
  const uint16_t* q;       // [n_heads][n_q][d] bf16
  const uint8_t* signs;
  const uint16_t* proj;    // G, m x d bf16 (NULL when m == 0)
  unsigned char* prep;     // n_heads * prep_head_bytes(d, m)
  int n_heads, n_q, d, m;
};

struct TwoStageArgs {
  const unsigned char* prep;
  const uint8_t* codes;    // [n_heads][n_tok][d]
  const uint16_t* norms;   // [n_heads][n_tok]
  const uint8_t* qbits;    // [n_heads][n_tok][m/8]
  const uint16_t* rnorms;  // [n_heads][n_tok]
  float* scores;           // [n_heads][n_q][n_tok]
  int64_t n_tok;
  int n_heads, n_q, m;
  int packed;              // codes bit-packed at the code width ([n_heads][n_tok][d*bits/8])
  // c[code] = sum_p alpha[p] s_p(code), s_p = +1 when popcount(code & plane_mask[p]) is odd,
  // else -1 (the odd-subset Walsh expansion of an antisymmetric codebook)
  double alpha[kMaxPlanes];
};

// Decode attention over the quantized cache.  The fused kernel gives each wave a range of
// tiles_per_range 16-token tiles of one KV head and one slice of attn_cols(d) value columns;
// the kAttnWaves ranges of a workgroup merge into one partial result in the work buffer:
//   ml  float2[n_heads][n_parts][16]      running max (base-2 logits) and sum of exp2
//   o   float[n_heads][n_parts][16][d]    sum_t exp2(z_t - max) n16_t / d c[code_t], rotated basis
// and the combine kernel merges those with the window and rotates back.
constexpr int kAttnMaxWin = 4096;         // window tokens held in LDS by the combine kernel
// fused-kernel waves aimed for over all heads: every wave resident at once on the 256 CUs
// (two per SIMD; one at d = 512, whose register use allows one)
__host__ __device__ constexpr int attn_target_waves(int d) { return d >= 512 ? 1024 : 2048; }
constexpr int kAttnWaves = 4;             // ranges (waves) per workgroup

#ifndef PQ_ATTN_MAX_COLS
#define PQ_ATTN_MAX_COLS 512       // value columns one wave of the fused kernel accumulates
#endif
__host__ __device__ constexpr int attn_cols(int d) { return d <= PQ_ATTN_MAX_COLS ? d : PQ_ATTN_MAX_COLS; }
// LDS of the in-workgroup merge: maxima and sums of every wave, two slots of 16 x attn_cols(d)
__host__ __device__ constexpr int attn_merge_lds(int d) { return 2 * kAttnWaves * 16 * 4 + 2 * 16 * attn_cols(d) * 4; }

struct AttnPlan {
  int n_ranges;              // per head
  int n_parts;               // per head: workgroups of kAttnWaves ranges
  int64_t tiles_per_range;
};

inline AttnPlan attn_plan(int d, int n_heads, int64_t n_tok) {
  AttnPlan p{0, 0, 0};
  const int64_t n_tiles = (n_tok + 15) >> 4;
  if (n_tiles == 0 || n_heads <= 0) return p;
  const int64_t slices = d / attn_cols(d);
  int64_t want = attn_target_waves(d) / ((int64_t)n_heads * slices);
  if (want < 1) want = 1;
  if (want > n_tiles) want = n_tiles;
  p.tiles_per_range = (n_tiles + want - 1) / want;
  p.n_ranges = (int)((n_tiles + p.tiles_per_range - 1) / p.tiles_per_range);
  p.n_parts = (p.n_ranges + kAttnWaves - 1) / kAttnWaves;
  return p;
}

inline int64_t attn_work_bytes(int d, int n_heads, int64_t n_tok) {
  const AttnPlan p = attn_plan(d, n_heads, n_tok);
  return (int64_t)n_heads * p.n_parts * kScoreRows * (8 + (int64_t)d * 4);
}

struct AttnArgs {
  const unsigned char* prep;  // pq_query_prep of the queries with the key signs (and G)
  const uint8_t* k_codes;     // [n_heads][n_tok][d] (packed: [n_heads][n_tok][d*bits/8])
  const uint16_t* k_norms;    // [n_heads][n_tok] fp16
  const uint8_t* k_qbits;     // [n_heads][n_tok][m/8]
  const uint16_t* k_rnorms;   // [n_heads][n_tok] fp16
  const uint8_t* v_codes;     // like k_codes
  const uint16_t* v_norms;    // [n_heads][n_tok] fp16
  const uint8_t* v_signs;     // d/8 bytes
  const uint16_t* k_win;      // [n_heads][n_win][d] bf16
  const uint16_t* v_win;      // [n_heads][n_win][d] bf16
  const uint16_t* q;          // [n_heads][n_q][d] bf16
  float* work_ml;             // partial maxima and sums
  float* work_o;              // partial outputs
  float* out;                 // [n_heads][n_q][d] fp32
  int64_t n_tok, n_win, tiles_per_range;
  int n_heads, n_q, m, n_ranges, n_parts, packed;
  double scale_log2;          // softmax scale times log2(e)
  double alpha[kMaxPlanes];   // key codebook, odd-Walsh coefficients (as TwoStageArgs)
  float vcent[1 << kMaxScoreBits];   // value codebook centroids
};

// Block-diagonal rotation for block sizes d that are not powers of two: d is split into the
// powers of two of its binary expansion, largest first, and each part gets its own
// Walsh-Hadamard transform; y = sqrt(d / d_k) H_k (D x)_k / ||x|| on part k.
constexpr int kBdMinD = 64, kBdMaxD = 4096;   // d a multiple of 32 in this range
// Dense rotation (a d x d orthogonal matrix) with the codebook of one sphere coordinate's law:
// d a multiple of 16 up to 128 (the matrix is held in LDS)
constexpr int kDenseMaxD = 512;

struct BdArgs {
  const void* x;              // quantize input [n_blocks][d], fp32 or bf16
  uint8_t* codes;             // [n_blocks][d], one code per byte
  const uint8_t* ccodes;      // dequantize input codes
  uint16_t* norms;            // quantize output, fp16
  const uint16_t* cnorms;     // dequantize input norms
  void* out;                  // dequantize output [n_blocks][d], fp32 or bf16
  const uint8_t* signs;       // d/8 bytes (block-diagonal rotation)
  const float* rot;           // d x d row-major fp32 (dense rotation)
  int64_t n_blocks;
  int d, bits;
  float cent[1 << kMaxBits];  // centroids, ascending
  float beta[(1 << kMaxBits) - 1];   // boundaries, ascending (fp32 rounding of the double ones)
  float beta_lo[(1 << kMaxBits) - 1];   // double boundary - beta (the dense rotation's exact recheck)
  // search grid of the block-diagonal quantize (as CodecTables; the kernel finds each cell's
  // nearest boundary itself)
  int ncell, half, nrep;
  float cell_w, cell_inv_w;
};

// one tensor of a grouped call (the public pq_tensor record, in device memory)
using TensorDesc = ::pq_tensor;

struct LaunchCfg {
  int cu_count;
  int max_lds;       // bytes of LDS one workgroup may use
};

hipError_t launch_quantize(int d, bool in_bf16, const QuantArgs& a, const LaunchCfg& c, hipStream_t s);
hipError_t launch_quantize_lo(int d, bool in_bf16, const QuantArgs& a, const LaunchCfg& c, hipStream_t s);  // d <= 128
hipError_t launch_quantize_hi(int d, bool in_bf16, const QuantArgs& a, const LaunchCfg& c, hipStream_t s);  // d >= 256
hipError_t launch_dequantize(int d, bool out_bf16, const DequantArgs& a, const LaunchCfg& c, hipStream_t s);
hipError_t launch_sketch(int d, const SketchArgs& a, const LaunchCfg& c, hipStream_t s);
hipError_t launch_outliers(const OutlierArgs& a, hipStream_t s);
hipError_t launch_project(const ProjectArgs& a, hipStream_t s);
hipError_t launch_score(const ScoreArgs& a, const LaunchCfg& c, hipStream_t s);
hipError_t launch_query_prep(const QueryPrepArgs& a, hipStream_t s);
hipError_t launch_two_stage(int d, int bits, const TwoStageArgs& a, const LaunchCfg& c, hipStream_t s);
hipError_t launch_attention(int d, int bits, const AttnArgs& a, hipStream_t s);
hipError_t launch_quantize_bd(bool in_bf16, const BdArgs& a, const LaunchCfg& c, hipStream_t s);
hipError_t launch_quantize_many(int d, bool in_bf16, const QuantArgs& a, const TensorDesc* tab, int n_tensors,
                                const LaunchCfg& c, hipStream_t s);
hipError_t launch_dequantize_many(int d, bool out_bf16, const DequantArgs& a, const TensorDesc* tab, int n_tensors,
                                  const LaunchCfg& c, hipStream_t s);
hipError_t launch_dequantize_bd(bool out_bf16, const BdArgs& a, const LaunchCfg& c, hipStream_t s);
hipError_t launch_quantize_dense(bool in_bf16, const BdArgs& a, const LaunchCfg& c, hipStream_t s);
hipError_t launch_dequantize_dense(bool out_bf16, const BdArgs& a, const LaunchCfg& c, hipStream_t s);
hipError_t launch_stream_probe(const uint8_t* in, uint16_t* out, int64_t n, const LaunchCfg& c, hipStream_t s);

}  // namespace pqi
