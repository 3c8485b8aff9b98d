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
__device__ __forceinline__ float inv_rms(float ss, float inv_k, float eps) {
  return __builtin_amdgcn_rsqf(ss * inv_k + eps);  // v_rsq_f32, within 1 ulp
}

// Sum of squares of 8 bf16 pairs added to ss (v_dot2c_f32_bf16).
__device__ __forceinline__ float sumsq8(const uint4 q, float ss) {
  const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
  for (int i = 0; i < 4; ++i)
    ss = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w[i]), __builtin_bit_cast(bf16x2, w[i]), ss, false);
  return ss;
}

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
  return inv_rms(wave_sum(ss), inv_k, eps);
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
//
// LDS layout: the 16 values lane l needs for superchunk c (columns
// c*1024 + 16l .. +15) sit as four 16-byte quads at quad index
// (4c + q) * 64 + l, q = 0..3. One ds_read_b128 of a wave then reads 1 KiB
// contiguous (no bank conflicts; with the plain layout the lanes' 64-byte
// stride made every read a multi-way conflict). The area holds whole
// superchunks: param_floats(cols) floats per parameter.
__host__ __device__ constexpr uint32_t param_floats(uint32_t cols) { return (cols + kSuper - 1) / kSuper * kSuper; }
__device__ __forceinline__ uint32_t pidx(uint32_t col) {
  return ((((col >> 10) * 4 + ((col >> 2) & 3)) * 64 + ((col >> 4) & 63)) << 2) + (col & 3);
}

// 8 columns starting at column c8 * 8.
template <bool BIAS>
__device__ __forceinline__ void put_params(uint4 gq, uint4 bq, uint32_t c8, float woff, float* gsh, float* bsh) {
  float gv[8];
  widen8(gq, gv);
#pragma unroll
  for (int i = 0; i < 8; ++i) gv[i] = gv[i] + woff;
  const uint32_t i0 = pidx(c8 * 8), i1 = pidx(c8 * 8 + 4);
  *reinterpret_cast<float4*>(gsh + i0) = make_float4(gv[0], gv[1], gv[2], gv[3]);
  *reinterpret_cast<float4*>(gsh + i1) = make_float4(gv[4], gv[5], gv[6], gv[7]);
  if constexpr (BIAS) {
    float bv[8];
    widen8(bq, bv);
    *reinterpret_cast<float4*>(bsh + i0) = make_float4(bv[0], bv[1], bv[2], bv[3]);
    *reinterpret_cast<float4*>(bsh + i1) = make_float4(bv[4], bv[5], bv[6], bv[7]);
  }
}

template <bool BIAS>
__device__ __forceinline__ void stage_params(const uint16_t* __restrict__ gamma, const uint16_t* __restrict__ beta,
                                             float woff, uint32_t cols, float* gsh, float* bsh) {
  for (uint32_t c8 = threadIdx.x; c8 * 8 < cols; c8 += blockDim.x) {
    const uint4 gq = *reinterpret_cast<const uint4*>(gamma + c8 * 8);
    uint4 bq = make_uint4(0u, 0u, 0u, 0u);
    if constexpr (BIAS) bq = *reinterpret_cast<const uint4*>(beta + c8 * 8);
    put_params<BIAS>(gq, bq, c8, woff, gsh, bsh);
  }
}

// The same in two steps (see partials_issue): the loads of the first
// 2 * kThreads * 8 columns, then the LDS stores and the remaining columns.
struct ParamsPre {
  uint4 g[2], b[2];
};
template <bool BIAS>
__device__ __forceinline__ ParamsPre params_issue(const uint16_t* gamma, const uint16_t* beta, uint32_t cols) {
  ParamsPre p;
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const uint32_t c8 = threadIdx.x + k * kThreads;
    p.g[k] = ld16(gamma + c8 * 8, c8 * 8 < cols);
    p.b[k] = BIAS ? ld16(beta + c8 * 8, c8 * 8 < cols) : make_uint4(0u, 0u, 0u, 0u);
  }
  return p;
}
template <bool BIAS>
__device__ __forceinline__ void params_finish(const ParamsPre& p, const uint16_t* gamma, const uint16_t* beta,
                                              float woff, uint32_t cols, float* gsh, float* bsh) {
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const uint32_t c8 = threadIdx.x + k * kThreads;
    if (c8 * 8 < cols) put_params<BIAS>(p.g[k], p.b[k], c8, woff, gsh, bsh);
  }
  for (uint32_t c8 = threadIdx.x + 2 * kThreads; c8 * 8 < cols; c8 += kThreads) {
    const uint4 gq = *reinterpret_cast<const uint4*>(gamma + c8 * 8);
    uint4 bq = make_uint4(0u, 0u, 0u, 0u);
    if constexpr (BIAS) bq = *reinterpret_cast<const uint4*>(beta + c8 * 8);
    put_params<BIAS>(gq, bq, c8, woff, gsh, bsh);
  }
}

// The 16 parameter values of the block starting at column `col` (a multiple
// of 16).
__device__ __forceinline__ void lds16(const float* base, uint32_t col, float v[16]) {
  const float* p = base + pidx(col);
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const float4 a = *reinterpret_cast<const float4*>(p + q * 256);
    v[4 * q] = a.x; v[4 * q + 1] = a.y; v[4 * q + 2] = a.z; v[4 * q + 3] = a.w;
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
  if constexpr (AMAX) {
    if (a.rs != nullptr && lane == 0) a.rs[r] = rs;
  }
  float mrow = 0.0f;
#pragma unroll
  for (int c = 0; c < NSC; ++c) {
    const uint32_t col = c * kSuper + lane * 16;
    const bool ok = FULL || col < cols;
    const uint32_t lcol = ok ? col : 0;
    float v[16], gv[16];
    widen16(q[c], v);
    lds16(gsh, lcol, gv);
#pragma unroll
    for (int i = 0; i < 16; ++i) v[i] = v[i] * gv[i];
    if constexpr (AMAX && !BIAS) {
      mrow = fmaxf(mrow, max16_abs(v));
      continue;
    }
    if constexpr (BIAS) {
      float bv[16];
      lds16(bsh, lcol, bv);
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
  float* bsh = params + param_floats(cols);
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
  const size_t lds = (size_t)param_floats((uint32_t)a.cols) * sizeof(float) * (BIAS ? 2 : 1);
  const int64_t max_wgs = AMAX && rms_wgs() > kRowPartials ? kRowPartials : rms_wgs();
  const dim3 grid(grid_rows(a.rows, max_wgs)), block(kThreads);
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
