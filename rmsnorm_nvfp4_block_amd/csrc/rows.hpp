// Shared pieces of the rowwise kernels (see kernels_rows.hip for the layout):
// the block-per-lane row mapping, the RMSNorm helpers and the LDS layout of
// the row parameters, used by kernels_rms_stream.hip and kernels_rms_coop.hip.
#pragma once
#include "device.hpp"
#include "launch.hpp"

#include <cstdlib>

namespace nvfp4q {

constexpr int kThreads = kWGThreads;
constexpr uint32_t kSuper = 1024;  // columns per superchunk (64 lanes x 16)

// ------------------------------------------------------------------ input types
// Element types of x on the paths that take more than bf16 (the values of
// nvfp4q_dtype): a 16-byte load holds 8 bf16 or fp16 values or 4 fp32 values.
enum InType { kInBF16 = 0, kInFP16 = 1, kInFP32 = 2 };
template <int T>
constexpr int in_size() { return T == kInFP32 ? 4 : 2; }

// The raw 16 elements of one block (two or four 16-byte loads).
template <int T>
struct Raw16 {
  uint4 q[in_size<T>()];
};
// Elements col .. col + 15 of a row (zeros when !ok).
template <int T>
__device__ __forceinline__ Raw16<T> load_raw16(const void* xr, uint32_t col, bool ok) {
  Raw16<T> b;
  const char* p = (const char*)xr + (size_t)col * in_size<T>();
#pragma unroll
  for (int l = 0; l < in_size<T>(); ++l) b.q[l] = ld16(p + 16 * l, ok);
  return b;
}
// fp16 pair to fp32 (exact).
__device__ __forceinline__ float h_lo(uint32_t w) { return (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xFFFFu)); }
__device__ __forceinline__ float h_hi(uint32_t w) { return (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16)); }
__device__ __forceinline__ void widen8_h(const uint4 q, float v[8]) {
  v[0] = h_lo(q.x); v[1] = h_hi(q.x);
  v[2] = h_lo(q.y); v[3] = h_hi(q.y);
  v[4] = h_lo(q.z); v[5] = h_hi(q.z);
  v[6] = h_lo(q.w); v[7] = h_hi(q.w);
}
template <int T>
__device__ __forceinline__ void widen_raw16(const Raw16<T>& b, float v[16]) {
  if constexpr (T == kInBF16) {
    widen8(b.q[0], v);
    widen8(b.q[1], v + 8);
  } else if constexpr (T == kInFP16) {
    widen8_h(b.q[0], v);
    widen8_h(b.q[1], v + 8);
  } else {
#pragma unroll
    for (int l = 0; l < 4; ++l) {
      v[4 * l] = __uint_as_float(b.q[l].x);
      v[4 * l + 1] = __uint_as_float(b.q[l].y);
      v[4 * l + 2] = __uint_as_float(b.q[l].z);
      v[4 * l + 3] = __uint_as_float(b.q[l].w);
    }
  }
}
// 8 elements of type T at element index i of p, as fp32.
template <int T>
__device__ __forceinline__ void load8_t(const void* p, uint32_t i, float v[8]) {
  const char* b = (const char*)p + (size_t)i * in_size<T>();
  if constexpr (T == kInFP32) {
    const uint4 a = *reinterpret_cast<const uint4*>(b), c = *reinterpret_cast<const uint4*>(b + 16);
    v[0] = __uint_as_float(a.x); v[1] = __uint_as_float(a.y); v[2] = __uint_as_float(a.z); v[3] = __uint_as_float(a.w);
    v[4] = __uint_as_float(c.x); v[5] = __uint_as_float(c.y); v[6] = __uint_as_float(c.z); v[7] = __uint_as_float(c.w);
  } else {
    const uint4 a = *reinterpret_cast<const uint4*>(b);
    if constexpr (T == kInBF16) widen8(a, v);
    else widen8_h(a, v);
  }
}

// 16 fp32 values rounded to nearest even in type T (fp32: unchanged), in place,
// when the rounded values are not stored.
template <int T>
__device__ __forceinline__ void round16(float v[16]) {
#pragma unroll
  for (int k = 0; k < 16; ++k) {
    if constexpr (T == kInBF16) v[k] = bf16_round(v[k]);
    else if constexpr (T == kInFP16) v[k] = (float)(_Float16)v[k];
  }
}

// 16 fp32 values rounded to nearest even in type T (fp32: unchanged), stored at
// element index i of p when ok, and returned as fp32 in v (the rounded values).
template <int T>
__device__ __forceinline__ void round_store16(float v[16], void* p, uint32_t i, bool ok) {
  char* b = (char*)p + (size_t)i * in_size<T>();
  if constexpr (T == kInFP32) {
    if (ok) {
#pragma unroll
      for (int l = 0; l < 4; ++l)
        *reinterpret_cast<uint4*>(b + 16 * l) = make_uint4(__float_as_uint(v[4 * l]), __float_as_uint(v[4 * l + 1]),
                                                           __float_as_uint(v[4 * l + 2]), __float_as_uint(v[4 * l + 3]));
    }
  } else {
    uint32_t w[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      if constexpr (T == kInBF16) {
        w[k] = pack_bf16(v[2 * k], v[2 * k + 1]);
      } else {
        w[k] = (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)v[2 * k]) |
               ((uint32_t)__builtin_bit_cast(uint16_t, (_Float16)v[2 * k + 1]) << 16);
      }
    }
    if (ok) {
      *reinterpret_cast<uint4*>(b) = make_uint4(w[0], w[1], w[2], w[3]);
      *reinterpret_cast<uint4*>(b + 16) = make_uint4(w[4], w[5], w[6], w[7]);
    }
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      v[2 * k] = T == kInBF16 ? bf_lo(w[k]) : h_lo(w[k]);
      v[2 * k + 1] = T == kInBF16 ? bf_hi(w[k]) : h_hi(w[k]);
    }
  }
}

// Round a (non-negative) fp32 value to nearest even in type T.
template <int T>
__device__ __forceinline__ float round_t(float m) {
  if constexpr (T == kInBF16) return bf_lo(pack_bf16(m, m) & 0xFFFFu);
  else if constexpr (T == kInFP16) return (float)(_Float16)m;
  else return m;
}

// max |v| over the values of one 16-byte load
template <int T>
__device__ __forceinline__ float max_abs16b(const uint4 q) {
  if constexpr (T == kInFP32) {
    return fmaxf(fmaxf(fabsf(__uint_as_float(q.x)), fabsf(__uint_as_float(q.y))),
                 fmaxf(fabsf(__uint_as_float(q.z)), fabsf(__uint_as_float(q.w))));
  } else {
    float v[8];
    if constexpr (T == kInBF16) widen8(q, v);
    else widen8_h(q, v);
    return max8_abs(v);
  }
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

// fp16 or fp32 row parameters (the input's type): a plain staging loop, 8
// columns per step, into the same LDS layout.
template <bool BIAS, int T>
__device__ __forceinline__ void stage_params_t(const void* gamma, const void* beta, float woff, uint32_t cols,
                                               float* gsh, float* bsh) {
  for (uint32_t c8 = threadIdx.x; c8 * 8 < cols; c8 += kThreads) {
    float gv[8], bv[8];
    load8_t<T>(gamma, c8 * 8, gv);
    if constexpr (BIAS) load8_t<T>(beta, c8 * 8, bv);
#pragma unroll
    for (int i = 0; i < 8; ++i) gv[i] = gv[i] + woff;
    const uint32_t i0 = pidx(c8 * 8), i1 = pidx(c8 * 8 + 4);
    *reinterpret_cast<float4*>(gsh + i0) = make_float4(gv[0], gv[1], gv[2], gv[3]);
    *reinterpret_cast<float4*>(gsh + i1) = make_float4(gv[4], gv[5], gv[6], gv[7]);
    if constexpr (BIAS) {
      *reinterpret_cast<float4*>(bsh + i0) = make_float4(bv[0], bv[1], bv[2], bv[3]);
      *reinterpret_cast<float4*>(bsh + i1) = make_float4(bv[4], bv[5], bv[6], bv[7]);
    }
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

}  // namespace nvfp4q
