// Host-side launch interface between the C ABI layer and the kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nvfp4q {

struct Workspace;

// Arguments of the rowwise paths (quantize and RMSNorm).
struct RowArgs {
  const void* x;
  int dtype;  // element type of x, gamma, beta and y (nvfp4q_dtype)
  int64_t rows, cols, ld_x;
  const void* gamma;
  const void* beta;
  float woff, eps;
  void* y;
  int64_t ld_y;
  uint8_t* codes;
  int64_t ldc;
  uint8_t* scales;
  int64_t lds;
  Workspace* ws;
  uint32_t nparts;          // partial maxima written by the amax pass (set by the launcher)
  float* rs;                // RMSNorm: per-row 1/rms written by the amax pass, or NULL
  const float* amax_in;
  float* amax_out;
  float* scale_out;
  bool sr;
  uint64_t seed;
  uint32_t offset;
};

// Arguments of the per-head QK norm (in place).
struct QkArgs {
  void* q;
  void* k;
  const void* wq;
  const void* wk;
  int64_t tokens, ldq, ldk;
  int hq, hk, d;
  float woff, eps;
  int dtype;  // element type of q, k and the weights (nvfp4q_dtype)
};

// Arguments of the 2D (rowwise + columnwise) path.
struct TwoDArgs {
  const void* x;
  int64_t rows, cols, ld_x;
  uint8_t *rcodes, *rscales;
  int64_t rldc, rlds;
  uint8_t *ccodes, *cscales;
  int64_t cldc, clds;
  Workspace* ws;
  uint32_t nparts;
  const float* amax_in;
  float* amax_out;
  float* scale_out;
  int dtype;     // element type of x (nvfp4q_dtype)
  int experts;   // stacked weights (grid y); rows is the rows of one weight
  bool tile16;  // one scale per 16 x 16 tile (both planes)
  bool sr;
  uint64_t seed;
  uint32_t offset;
};

// Largest row stride of the grouped path's input in 2-byte elements (2^25
// bytes; fp32 rows: half as many elements): its loads reach 32 rows past a
// base row with 32-bit byte offsets.
constexpr int64_t kGroupedMaxLd = (int64_t)1 << 24;

// Arguments of the grouped path (columnwise and/or rowwise planes).
struct GroupArgs {
  const void* x;
  int dtype;  // element type of x (nvfp4q_dtype)
  int64_t rows, cols, ld_x;
  const int32_t* offsets;
  int32_t groups;
  int32_t* poff_out;
  bool rht;
  uint32_t mask;
  bool col;                       // columnwise plane requested
  uint8_t *codes, *scales;
  int64_t ldc, lds;
  const float* amax_in;
  float* amax_out;
  float* scale_out;
  bool row;                       // rowwise plane requested
  uint8_t *rcodes, *rscales;
  int64_t rldc, rlds;
  const float* ramax_in;
  float* ramax_out;
  float* rscale_out;
  Workspace* ws;
  bool sr;
  bool fast;  // fast math: no bf16 round-through of the transform's output
  uint64_t seed;
  uint32_t offset;
};

hipError_t launch_empty_scale(float* amax_out, float* scale_out, int n, hipStream_t s);
// Amax pass over a [rows, cols] tensor; returns the number of partials it
// writes through `nparts`. tensors > 1: that many stacked [rows, cols]
// tensors, the partials of tensor e in slots e * nparts onwards.
hipError_t launch_amax_rows(const RowArgs& a, hipStream_t s, uint32_t* nparts, int tensors = 1);
hipError_t launch_quant_rows(const RowArgs& a, hipStream_t s);
// Two-pass RMSNorm: with amax_pass, the amax pass (sets *nparts); otherwise the
// encode pass (reads a.nparts partials when a.amax_in is NULL).
hipError_t launch_rmsnorm_pass(const RowArgs& a, bool amax_pass, hipStream_t s, uint32_t* nparts);
// Streaming RMSNorm passes (need a.rs): the amax pass without a bias, which
// also writes a.rs, and the encode pass, which reads it.
hipError_t launch_rms_stream_amax(const RowArgs& a, hipStream_t s, uint32_t* nparts);
hipError_t launch_rms_stream_quant(const RowArgs& a, hipStream_t s);
// Widest row of input type `dtype` the RMSNorm passes take (2-byte types
// 32768, fp32 16384), and the widest whose gamma and beta the streaming and
// one-launch kernels stage in LDS (16384): wider rows take the
// cooperative-row passes.
int rms_max_cols(int dtype);
int rms_stage_max_cols();
// One-launch RMSNorm + rowwise encode for at most rms_fused_max_rows() rows
// (codes required, amax computed in the launch; uses and advances the
// workspace's one-launch state words).
hipError_t launch_rms_fused(const RowArgs& a, hipStream_t s);
int rms_fused_max_rows();

hipError_t launch_quant_2d(const TwoDArgs& a, hipStream_t s);
hipError_t launch_qk_norm(const QkArgs& a, hipStream_t s);

// Grouped path.
hipError_t launch_grouped(const GroupArgs& a, hipStream_t s);
// Workspace slots the grouped path's amax pass needs for `planes` planes (a
// bound independent of the size of x).
int64_t grouped_partials(int64_t rows, int64_t cols, int groups, int planes);

}  // namespace nvfp4q
