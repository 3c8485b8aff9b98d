// Shared pieces of the rowwise kernels (see kernels_rows.hip for the layout):
// the block-per-lane row mapping and the two-pass RMSNorm kernels. The
// RMSNorm instantiations for each row width (in superchunks of 1024 columns)
// are compiled in kernels_rms_*.hip so that they build in parallel.
#pragma once
#include "device.hpp"
#include "launch.hpp"

#include <cstdlib>

namespace nvfp4q {

constexpr int kThreads = kWGThreads;
constexpr uint32_t kSuper = 1024;  // columns per superchunk (64 lanes x 16)

struct Blk {
  uint4 lo, hi;  // 16 bf16 values of one block
};

__device__ __forceinline__ void widen16(const Blk& b, float v[16]) {
  widen8(b.lo, v);
  widen8(b.hi, v + 8);
}

// The lane's block at column `col` of a row (zero when outside the row).
template <bool FULL>
__device__ __forceinline__ Blk load_blk(const uint16_t* xr, uint32_t col, uint32_t cols) {
  Blk b;
  if (FULL) {
    b.lo = *reinterpret_cast<const uint4*>(xr + col);
    b.hi = *reinterpret_cast<const uint4*>(xr + col + 8);
  } else {
    b.lo = ld16(xr + col, col < cols);
    b.hi = ld16(xr + col + 8, col < cols);
  }
  return b;
}

// ------------------------------------------------------------------ launchers
inline uint32_t grid_rows(int64_t rows, int64_t max_wgs = 4096) {
  int64_t wgs = (rows + kWavesPerWG - 1) / kWavesPerWG;
  if (wgs > max_wgs) wgs = max_wgs;
  if (wgs < 1) wgs = 1;
  return (uint32_t)wgs;
}

// ------------------------------------------------------------------ RMSNorm
// y = bf16_rne(((gamma + c) * x) * r [+ beta]), r = 1/sqrt(ss/K + eps), ss the
// fp32 sum of squares of the row ("CuTeDSL at Perplexity", QK Norm).
template <int NSC>
__device__ __forceinline__ float row_rs(const Blk (&q)[NSC], float inv_k, float eps) {
  float ss = 0.0f;
#pragma unroll
  for (int c = 0; c < NSC; ++c) {
    const uint32_t w[8] = {q[c].lo.x, q[c].lo.y, q[c].lo.z, q[c].lo.w, q[c].hi.x, q[c].hi.y, q[c].hi.z, q[c].hi.w};
#pragma unroll
    for (int i = 0; i < 8; ++i)
      ss = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w[i]), __builtin_bit_cast(bf16x2, w[i]), ss, false);
  }
  ss = wave_sum(ss);
  return __builtin_amdgcn_rsqf(ss * inv_k + eps);  // v_rsq_f32, within 1 ulp
}

__device__ __forceinline__ uint4 pack8_bf16(const float v[8]) {
  uint4 y;
  y.x = pack_bf16(v[0], v[1]);
  y.y = pack_bf16(v[2], v[3]);
  y.z = pack_bf16(v[4], v[5]);
  y.w = pack_bf16(v[6], v[7]);
  return y;
}

// Row parameters in LDS as fp32, filled once per workgroup: RN(gamma + c)
// (c the weight offset) and beta when present.
template <bool BIAS>
__device__ __forceinline__ void stage_params(const uint16_t* __restrict__ gamma, const uint16_t* __restrict__ beta,
                                             float woff, uint32_t cols, float* gsh, float* bsh) {
  for (uint32_t c8 = threadIdx.x; c8 * 8 < cols; c8 += blockDim.x) {
    float gv[8];
    widen8(*reinterpret_cast<const uint4*>(gamma + c8 * 8), gv);
#pragma unroll
    for (int i = 0; i < 8; ++i) gv[i] = gv[i] + woff;
    *reinterpret_cast<float4*>(gsh + c8 * 8) = make_float4(gv[0], gv[1], gv[2], gv[3]);
    *reinterpret_cast<float4*>(gsh + c8 * 8 + 4) = make_float4(gv[4], gv[5], gv[6], gv[7]);
    if constexpr (BIAS) {
      float bv[8];
      widen8(*reinterpret_cast<const uint4*>(beta + c8 * 8), bv);
      *reinterpret_cast<float4*>(bsh + c8 * 8) = make_float4(bv[0], bv[1], bv[2], bv[3]);
      *reinterpret_cast<float4*>(bsh + c8 * 8 + 4) = make_float4(bv[4], bv[5], bv[6], bv[7]);
    }
  }
}

__device__ __forceinline__ void lds16(const float* p, float v[16]) {
#pragma unroll
  for (int i = 0; i < 16; i += 4) {
    const float4 a = *reinterpret_cast<const float4*>(p + i);
    v[i] = a.x; v[i + 1] = a.y; v[i + 2] = a.z; v[i + 3] = a.w;
  }
}

// Loads one row; a row index past the end is clamped to the last row (its
// values are then never used). FULL: every superchunk lies inside the row.
template <int NSC, bool FULL>
__device__ __forceinline__ void load_row(const uint16_t* __restrict__ x, int64_t ld_x, uint32_t r, uint32_t rows,
                                         uint32_t cols, int lane, Blk (&q)[NSC]) {
  const uint16_t* xr = x + (int64_t)(r < rows ? r : rows - 1) * ld_x;
#pragma unroll
  for (int c = 0; c < NSC; ++c) q[c] = load_blk<FULL>(xr, c * kSuper + lane * 16, cols);
}

// One row of the two-pass form (NSC superchunks in registers).
// AMAX: returns the row's max |y|. Without a bias that is
// RN(max |RN(x * g)| * r): y = RN(RN(x * g) * r) is monotone in |RN(x * g)|
// for the row's fixed r > 0, so r is applied once per row.
// Otherwise: normalize, round to bf16 (optionally store y) and encode (CODES).
template <int NSC, bool FULL, bool BIAS, bool AMAX, bool SR, bool CODES>
__device__ __forceinline__ float rms_row(const RowArgs& a, uint32_t r, const Blk (&q)[NSC], const float* gsh,
                                         const float* bsh, GScale g, const float* rcp_tab, float inv_k, int lane) {
  const uint32_t cols = (uint32_t)a.cols;
  const uint32_t nbr = cols >> 4;
  const float rs = row_rs<NSC>(q, inv_k, a.eps);
  float mrow = 0.0f;
#pragma unroll
  for (int c = 0; c < NSC; ++c) {
    const uint32_t col = c * kSuper + lane * 16;
    const bool ok = FULL || col < cols;
    const uint32_t lcol = ok ? col : 0;
    float v[16], gv[16];
    widen16(q[c], v);
    lds16(gsh + lcol, gv);
#pragma unroll
    for (int i = 0; i < 16; ++i) v[i] = v[i] * gv[i];
    if constexpr (AMAX && !BIAS) {
      mrow = fmaxf(mrow, max16_abs(v));
      continue;
    }
    if constexpr (BIAS) {
      float bv[16];
      lds16(bsh + lcol, bv);
#pragma unroll
      for (int i = 0; i < 16; ++i) v[i] = __builtin_fmaf(v[i], rs, bv[i]);
    } else {
#pragma unroll
      for (int i = 0; i < 16; ++i) v[i] = v[i] * rs;
    }
    if constexpr (AMAX) {
      mrow = fmaxf(mrow, max16_abs(v));
    } else {
      const uint4 y0 = pack8_bf16(v), y1 = pack8_bf16(v + 8);
      if (a.y != nullptr) {
        if (ok) {
          uint16_t* yr = (uint16_t*)a.y + (int64_t)r * a.ld_y + col;
          *reinterpret_cast<uint4*>(yr) = y0;
          *reinterpret_cast<uint4*>(yr + 8) = y1;
        }
      }
      if constexpr (CODES) {
        widen8(y0, v);
        widen8(y1, v + 8);
        uint32_t sc;
        const uint2 w =
            encode_block16<SR>(v, g, rcp_tab, sc, (uint64_t)r * nbr + (col >> 4), a.seed, a.offset, 0);
        if (ok) {
          *reinterpret_cast<uint2*>(a.codes + (int64_t)r * a.ldc + (col >> 1)) = w;
          a.scales[(int64_t)r * a.lds + (col >> 4)] = (uint8_t)sc;
        }
      }
    }
  }
  if constexpr (AMAX) return BIAS ? mrow : mrow * rs;
  return 0.0f;
}

// Two-pass form: one wave per token at a time, the next row's loads in flight
// while a row is processed. AMAX: the workgroup's max |y| into its partial slot.
template <int NSC, bool FULL, bool BIAS, bool AMAX, bool SR, bool CODES>
__global__ __launch_bounds__(kThreads) void k_rmsnorm(const RowArgs a) {
  extern __shared__ float params[];  // gamma + c [cols], then beta [cols]
  __shared__ float rcp_tab[128];
  const uint32_t rows = (uint32_t)a.rows, cols = (uint32_t)a.cols;
  const uint16_t* __restrict__ x = (const uint16_t*)a.x;
  const int lane = threadIdx.x & 63;
  const uint32_t wave = (blockIdx.x * kThreads + threadIdx.x) >> 6;
  const uint32_t nwaves = (gridDim.x * kThreads) >> 6;
  Blk qa[NSC], qb[NSC];
  load_row<NSC, FULL>(x, a.ld_x, wave, rows, cols, lane, qa);  // first row in flight before the staging
  float* gsh = params;
  float* bsh = params + cols;
  stage_params<BIAS>((const uint16_t*)a.gamma, (const uint16_t*)a.beta, a.woff, cols, gsh, bsh);
  GScale g = {1.0f, 1.0f};
  if constexpr (!AMAX && CODES) g = consume_scales(a.ws, a.nparts, a.amax_in, a.amax_out, a.scale_out, rcp_tab);
  else __syncthreads();
  const float inv_k = 1.0f / (float)cols;
  float mloc = 0.0f;
  for (uint32_t r = wave; r < rows; r += 2 * nwaves) {
    const bool more = r + nwaves < rows;
    if (more) load_row<NSC, FULL>(x, a.ld_x, r + nwaves, rows, cols, lane, qb);
    mloc = fmaxf(mloc, rms_row<NSC, FULL, BIAS, AMAX, SR, CODES>(a, r, qa, gsh, bsh, g, rcp_tab, inv_k, lane));
    if (!more) break;
    if (r + 2 * nwaves < rows) load_row<NSC, FULL>(x, a.ld_x, r + 2 * nwaves, rows, cols, lane, qa);
    mloc = fmaxf(mloc, rms_row<NSC, FULL, BIAS, AMAX, SR, CODES>(a, r + nwaves, qb, gsh, bsh, g, rcp_tab,
                                                                        inv_k, lane));
  }
  if constexpr (AMAX) {
    // max |bf16(y)| = bf16(max |y|): round-to-nearest-even is monotone.
    publish_partial(a.ws, bf_lo(pack_bf16(mloc, mloc) & 0xFFFFu));
  }
}

// Empty tensor: amax 0, S_dec 1.
// ---- two-pass RMSNorm dispatch
// Workgroups per launch: rows / 4 (one row per wave) up to NVFP4Q_RMS_WGS
// (default 1024, i.e. 16 waves per CU); past that each wave takes several rows
// with the next one prefetched.
inline int64_t rms_wgs() {
  static int64_t v = [] {
    const char* e = getenv("NVFP4Q_RMS_WGS");
    return e ? (int64_t)atoll(e) : (int64_t)1024;
  }();
  return v;
}

template <int NSC, bool BIAS, bool AMAX, bool SR, bool CODES>
static void launch_rms_t(const RowArgs& a, hipStream_t s) {
  const size_t lds = (size_t)a.cols * sizeof(float) * (BIAS ? 2 : 1);
  const dim3 grid(grid_rows(a.rows, rms_wgs())), block(kThreads);
  if (a.cols == NSC * (int64_t)kSuper)
    hipLaunchKernelGGL((k_rmsnorm<NSC, true, BIAS, AMAX, SR, CODES>), grid, block, lds, s, a);
  else
    hipLaunchKernelGGL((k_rmsnorm<NSC, false, BIAS, AMAX, SR, CODES>), grid, block, lds, s, a);
}

// Modes: the amax pass, y only, y and/or codes with RTNE or SR.
template <int NSC, bool BIAS>
static void launch_rms_mode(const RowArgs& a, bool amax_pass, hipStream_t s) {
  if (amax_pass) launch_rms_t<NSC, BIAS, true, false, false>(a, s);
  else if (a.codes == nullptr) launch_rms_t<NSC, BIAS, false, false, false>(a, s);
  else if (a.sr) launch_rms_t<NSC, BIAS, false, true, true>(a, s);
  else launch_rms_t<NSC, BIAS, false, false, true>(a, s);
}

template <int NSC>
void launch_rms_nsc(const RowArgs& a, bool amax_pass, hipStream_t s) {
  if (a.beta) launch_rms_mode<NSC, true>(a, amax_pass, s);
  else launch_rms_mode<NSC, false>(a, amax_pass, s);
}

}  // namespace nvfp4q
