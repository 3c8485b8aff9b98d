// Per-head RMSNorm of attention heads (QK norm) for gfx950, in place.
//
// A lane takes 8 consecutive elements of one head (one 16-byte load), so a
// head of D elements spans D / 8 neighbouring lanes (8, 16 or 32) and a wave
// normalizes 64 / (D / 8) heads at once. The sum of squares meets in DPP
// steps inside each lane group (quad swaps, then mirrors over 8 and 16 lanes,
// and a swap of 16-lane halves for 32), which leave the same total in every
// lane of the group. Heads are numbered token-major over the q heads and then
// the k heads of each token, so one launch covers both tensors; each lane
// picks its tensor, its weight and its address on its own. Measured on 4096
// tokens x (32 + 8) heads of 128 with one head per lane: 8 elements per lane
// 17.4 us, 16 20.3 us, 32 26.6 us (NVFP4Q_QK_EPL selects).
//
// "CuTeDSL at Perplexity", QK Norm: per-head norm for heads of 64, 128 or 256
// elements, 128 bits per thread, several heads per warp, a butterfly
// reduction within the head's threads, y = (w + c) * (x * rsqrt(sum x^2 / D +
// eps)) written back in place.
#include "rows.hpp"

#include <cstdlib>

namespace nvfp4q {

namespace {

// Sum over the kTph lanes of a head (aligned groups of 2, 4, 8, 16 or 32 lanes).
template <int TPH>
__device__ __forceinline__ float head_sum(float v) {
  v += dpp_f<kDppXor1>(v);
  if constexpr (TPH >= 4) v += dpp_f<kDppXor2>(v);
  if constexpr (TPH >= 8) v += dpp_f<kDppHalfMirror>(v);
  if constexpr (TPH >= 16) v += dpp_f<kDppMirror>(v);
  if constexpr (TPH >= 32) v += __shfl_xor(v, 16, 64);
  return v;
}

// 8 elements of type T to fp32 and back (round to nearest even).
template <int T>
__device__ __forceinline__ void widen_in8(const uint4* q, float v[8]) {
  if constexpr (T == kInBF16) {
    widen8(q[0], v);
  } else if constexpr (T == kInFP16) {
    widen8_h(q[0], v);
  } else {
    const uint32_t w[8] = {q[0].x, q[0].y, q[0].z, q[0].w, q[1].x, q[1].y, q[1].z, q[1].w};
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = __uint_as_float(w[i]);
  }
}
template <int T>
__device__ __forceinline__ void narrow_out8(const float v[8], uint4* q) {
  if constexpr (T == kInBF16) {
    q[0] = pack8_bf16(v);
  } else if constexpr (T == kInFP16) {
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      w[i] = (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)v[2 * i]) |
             ((uint32_t)__builtin_bit_cast(uint16_t, (_Float16)v[2 * i + 1]) << 16);
    q[0] = make_uint4(w[0], w[1], w[2], w[3]);
  } else {
    q[0] = make_uint4(__float_as_uint(v[0]), __float_as_uint(v[1]), __float_as_uint(v[2]), __float_as_uint(v[3]));
    q[1] = make_uint4(__float_as_uint(v[4]), __float_as_uint(v[5]), __float_as_uint(v[6]), __float_as_uint(v[7]));
  }
}

// E elements per lane (8, 16 or 32) of element type T; each lane works on H
// heads, kHpw heads apart (a wave on H consecutive groups of heads), with all
// of their loads issued before any of their arithmetic.
template <int D, int E, int H, int T>
__global__ __launch_bounds__(kThreads) void k_qk_norm(const QkArgs a) {
  constexpr uint32_t kTph = D / E;              // lanes per head
  constexpr uint32_t kHpw = 64 / kTph;          // heads per wave and group
  constexpr int kG = E / 8;                     // groups of 8 elements per lane
  constexpr int kL = in_size<T>() / 2;          // 16-byte loads per group of 8
  const uint32_t lane = threadIdx.x & 63;
  const uint64_t wave = ((uint64_t)blockIdx.x * kThreads + threadIdx.x) >> 6;
  const uint32_t sub = lane % kTph;
  const uint32_t hpt = (uint32_t)(a.hq + a.hk);  // heads per token
  char* x[H];
  bool live[H];
  uint4 xq[H][kG * kL], wq[H][kG * kL];
#pragma unroll
  for (int h = 0; h < H; ++h) {
    const uint64_t head = (wave * H + h) * kHpw + lane / kTph;
    live[h] = head < (uint64_t)a.tokens * hpt;
    const uint64_t t = live[h] ? head / hpt : 0;
    const uint32_t j = live[h] ? (uint32_t)(head - t * hpt) : 0;
    const bool isq = j < (uint32_t)a.hq;
    const int64_t el = isq ? (int64_t)t * a.ldq + (int64_t)j * D : (int64_t)t * a.ldk + (int64_t)(j - a.hq) * D;
    x[h] = (char*)(isq ? a.q : a.k) + (el + sub * E) * in_size<T>();
    const char* w = (const char*)(isq ? a.wq : a.wk) + (size_t)sub * E * in_size<T>();
#pragma unroll
    for (int l = 0; l < kG * kL; ++l) xq[h][l] = ld16(x[h] + 16 * l, live[h]);
#pragma unroll
    for (int l = 0; l < kG * kL; ++l) wq[h][l] = ld16(w + 16 * l, live[h]);
  }
#pragma unroll
  for (int h = 0; h < H; ++h) {
    float v[kG][8];
    float ss = 0.0f;
#pragma unroll
    for (int gi = 0; gi < kG; ++gi) {
      widen_in8<T>(xq[h] + gi * kL, v[gi]);
      if constexpr (T == kInBF16) {
        ss = sumsq8(xq[h][gi], ss);
      } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) ss = __builtin_fmaf(v[gi][i], v[gi][i], ss);
      }
    }
    ss = head_sum<kTph>(ss);
    const float r = inv_rms(ss, 1.0f / (float)D, a.eps);
#pragma unroll
    for (int gi = 0; gi < kG; ++gi) {
      float g[8];
      widen_in8<T>(wq[h] + gi * kL, g);
#pragma unroll
      for (int i = 0; i < 8; ++i) v[gi][i] = (g[i] + a.woff) * (v[gi][i] * r);
      uint4 o[kL];
      narrow_out8<T>(v[gi], o);
      if (live[h]) {
#pragma unroll
        for (int l = 0; l < kL; ++l) *reinterpret_cast<uint4*>(x[h] + 16 * (gi * kL + l)) = o[l];
      }
    }
  }
}

// Heads per lane: NVFP4Q_QK_HPL (1, 2 or 4), default 2. Measured on 4096
// tokens x (32 + 8) heads of 128 (bf16): 17.5, 16.1 and 16.5-16.7 us (twice
// the bytes in flight per wave at two heads; at four, fewer waves).
int qk_hpl() {
  static int v = [] {
    const char* e = getenv("NVFP4Q_QK_HPL");
    const int n = e ? atoi(e) : 2;
    return n == 1 || n == 4 ? n : 2;
  }();
  return v;
}

// Elements per lane: NVFP4Q_QK_EPL (8, 16 or 32), default 8.
int qk_epl() {
  static int v = [] {
    const char* e = getenv("NVFP4Q_QK_EPL");
    const int n = e ? atoi(e) : 8;
    return n == 16 || n == 32 ? n : 8;
  }();
  return v;
}

template <int D, int E, int H, int T>
hipError_t launch_qk_deht(const QkArgs& a, hipStream_t s) {
  constexpr uint64_t kHpw = 64 / (D / E);
  const uint64_t heads = (uint64_t)a.tokens * (uint64_t)(a.hq + a.hk);
  const uint64_t waves = (heads + kHpw * H - 1) / (kHpw * H);
  const uint64_t wgs = (waves + kWavesPerWG - 1) / kWavesPerWG;
  if (wgs == 0) return hipSuccess;
  hipLaunchKernelGGL((k_qk_norm<D, E, H, T>), dim3((uint32_t)wgs), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

template <int D, int E, int T>
hipError_t launch_qk_det(const QkArgs& a, hipStream_t s) {
  if (qk_hpl() == 2) return launch_qk_deht<D, E, 2, T>(a, s);
  return qk_hpl() == 4 ? launch_qk_deht<D, E, 4, T>(a, s) : launch_qk_deht<D, E, 1, T>(a, s);
}

template <int D, int T>
hipError_t launch_qk_dt(const QkArgs& a, hipStream_t s) {
  if (qk_epl() == 16) return launch_qk_det<D, 16, T>(a, s);
  return qk_epl() == 32 ? launch_qk_det<D, 32, T>(a, s) : launch_qk_det<D, 8, T>(a, s);
}

template <int D>
hipError_t launch_qk_d(const QkArgs& a, hipStream_t s) {
  if (a.dtype == kInFP16) return launch_qk_dt<D, kInFP16>(a, s);
  if (a.dtype == kInFP32) return launch_qk_dt<D, kInFP32>(a, s);
  return launch_qk_dt<D, kInBF16>(a, s);
}

}  // namespace

hipError_t launch_qk_norm(const QkArgs& a, hipStream_t s) {
  if (a.d == 64) return launch_qk_d<64>(a, s);
  if (a.d == 128) return launch_qk_d<128>(a, s);
  if (a.d == 256) return launch_qk_d<256>(a, s);
  return hipErrorInvalidValue;
}

}  // namespace nvfp4q
