// Internal interface between the C ABI (pq_api.cpp) and the kernels
// (pq_kernels.hip).  Not installed; the public header is include/pq.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pqi {

constexpr int kMaxBits = 8;
constexpr int kMaxCells = 4096;

// fp32 codebook and the geometry of the uniform search grid the kernels build
// in LDS: cell k (0 <= k < ncell) is centred on (k - half) w and stores the
// boundary nearest to its centre together with the codes and centroids on
// both sides, so code = base + (y > boundary) is exact for every y that rounds
// to the cell (w is 0.9 of the smallest boundary gap).  Each cell is stored
// nrep times so that the 16 lanes of one LDS access group read distinct banks.
struct CodecTables {
  float cent[1 << kMaxBits];
  float beta[(1 << kMaxBits) - 1];
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
  CodecTables t;
};

struct DequantArgs {
  const uint8_t* codes;
  const uint16_t* norms;
  int64_t n_blocks;
  const uint8_t* signs;
  void* out;
  CodecTables t;
};

struct SketchArgs {
  const uint16_t* keys;
  int64_t n_keys;
  const uint16_t* proj;
  uint8_t* bits;
  uint16_t* norms;
  int m;
};

struct ProjectArgs {
  const uint16_t* q;
  int64_t n_q;
  const uint16_t* proj;
  float* sq;
  int d;
  int m;
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
};

struct LaunchCfg {
  int cu_count;
  int max_lds;       // bytes of LDS one workgroup may use
};

hipError_t launch_quantize(int d, bool in_bf16, const QuantArgs& a, const LaunchCfg& c, hipStream_t s);
hipError_t launch_dequantize(int d, bool out_bf16, const DequantArgs& a, const LaunchCfg& c, hipStream_t s);
hipError_t launch_sketch(int d, const SketchArgs& a, const LaunchCfg& c, hipStream_t s);
hipError_t launch_project(const ProjectArgs& a, hipStream_t s);
hipError_t launch_score(const ScoreArgs& a, const LaunchCfg& c, hipStream_t s);

}  // namespace pqi
