// Per-head RMSNorm of attention heads (QK norm) for gfx950, in place.
//
// A lane takes 16 consecutive elements of one head (two 16-byte loads), so a
// head of D elements spans D / 16 neighbouring lanes (4, 8 or 16) and a wave
// normalizes 64 / (D / 16) heads at once. The sum of squares meets in DPP
// steps inside each lane group (quad swaps, then a mirror over 8 and over 16
// lanes), which leave the same total in every lane of the group. Heads are
// numbered token-major over the q heads and then the k heads of each token,
// so one launch covers both tensors; each lane picks its tensor, its weight
// and its address on its own.
//
// "CuTeDSL at Perplexity", QK Norm: per-head norm for heads of 64, 128 or 256
// elements, several heads per warp, a butterfly reduction within the head's
// threads, y = (w + c) * (x * rsqrt(sum x^2 / D + eps)) written back in place.
#include "rows.hpp"

namespace nvfp4q {

namespace {

template <int D>
__device__ __forceinline__ float head_sum(float v) {
  v += dpp_f<kDppXor1>(v);
  v += dpp_f<kDppXor2>(v);
  if constexpr (D >= 128) v += dpp_f<kDppHalfMirror>(v);
  if constexpr (D >= 256) v += dpp_f<kDppMirror>(v);
  return v;
}

template <int D>
__global__ __launch_bounds__(kThreads) void k_qk_norm(const QkArgs a) {
  constexpr uint32_t kTph = D / 16;   // lanes per head
  constexpr uint32_t kHpw = 64 / kTph;  // heads per wave
  const uint32_t lane = threadIdx.x & 63;
  const uint64_t wave = ((uint64_t)blockIdx.x * kThreads + threadIdx.x) >> 6;
  const uint64_t head = wave * kHpw + lane / kTph;
  const uint32_t sub = lane % kTph;
  const uint32_t hpt = (uint32_t)(a.hq + a.hk);  // heads per token
  const bool live = head < (uint64_t)a.tokens * hpt;
  const uint64_t t = live ? head / hpt : 0;
  const uint32_t j = live ? (uint32_t)(head - t * hpt) : 0;
  const bool isq = j < (uint32_t)a.hq;
  uint16_t* x = isq ? (uint16_t*)a.q + (int64_t)t * a.ldq + (int64_t)j * D
                    : (uint16_t*)a.k + (int64_t)t * a.ldk + (int64_t)(j - a.hq) * D;
  x += sub * 16;
  const uint16_t* w = (const uint16_t*)(isq ? a.wq : a.wk) + sub * 16;
  const uint4 x0 = ld16(x, live), x1 = ld16(x + 8, live);
  const uint4 w0 = ld16(w, live), w1 = ld16(w + 8, live);
  const float ss = head_sum<D>(sumsq8(x1, sumsq8(x0, 0.0f)));
  const float r = inv_rms(ss, 1.0f / (float)D, a.eps);
  float v[16], g[16];
  widen8(x0, v);
  widen8(x1, v + 8);
  widen8(w0, g);
  widen8(w1, g + 8);
#pragma unroll
  for (int i = 0; i < 16; ++i) v[i] = (g[i] + a.woff) * (v[i] * r);
  if (live) {
    *reinterpret_cast<uint4*>(x) = pack8_bf16(v);
    *reinterpret_cast<uint4*>(x + 8) = pack8_bf16(v + 8);
  }
}

template <int D>
hipError_t launch_qk_d(const QkArgs& a, hipStream_t s) {
  const uint64_t heads = (uint64_t)a.tokens * (uint64_t)(a.hq + a.hk);
  const uint64_t waves = (heads + 64 / (D / 16) - 1) / (64 / (D / 16));
  const uint64_t wgs = (waves + kWavesPerWG - 1) / kWavesPerWG;
  if (wgs == 0) return hipSuccess;
  hipLaunchKernelGGL(k_qk_norm<D>, dim3((uint32_t)wgs), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_qk_norm(const QkArgs& a, hipStream_t s) {
  if (a.d == 64) return launch_qk_d<64>(a, s);
  if (a.d == 128) return launch_qk_d<128>(a, s);
  if (a.d == 256) return launch_qk_d<256>(a, s);
  return hipErrorInvalidValue;
}

}  // namespace nvfp4q
