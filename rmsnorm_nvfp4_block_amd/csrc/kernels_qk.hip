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
// tokens x (32 + 8) heads of 128: 8 elements per lane 17.4 us, 16 20.3 us,
// 32 26.6 us (NVFP4Q_QK_EPL selects).
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

// E elements per lane (8, 16 or 32: one, two or four 16-byte loads).
template <int D, int E>
__global__ __launch_bounds__(kThreads) void k_qk_norm(const QkArgs a) {
  constexpr uint32_t kTph = D / E;      // lanes per head
  constexpr uint32_t kHpw = 64 / kTph;  // heads per wave
  constexpr int kL = E / 8;             // 16-byte loads per lane
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
  x += sub * E;
  const uint16_t* w = (const uint16_t*)(isq ? a.wq : a.wk) + sub * E;
  uint4 xq[kL], wq[kL];
#pragma unroll
  for (int l = 0; l < kL; ++l) xq[l] = ld16(x + 8 * l, live);
#pragma unroll
  for (int l = 0; l < kL; ++l) wq[l] = ld16(w + 8 * l, live);
  float ss = 0.0f;
#pragma unroll
  for (int l = 0; l < kL; ++l) ss = sumsq8(xq[l], ss);
  ss = head_sum<kTph>(ss);
  const float r = inv_rms(ss, 1.0f / (float)D, a.eps);
#pragma unroll
  for (int l = 0; l < kL; ++l) {
    float v[8], g[8];
    widen8(xq[l], v);
    widen8(wq[l], g);
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = (g[i] + a.woff) * (v[i] * r);
    if (live) *reinterpret_cast<uint4*>(x + 8 * l) = pack8_bf16(v);
  }
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

template <int D, int E>
hipError_t launch_qk_de(const QkArgs& a, hipStream_t s) {
  constexpr uint64_t kHpw = 64 / (D / E);
  const uint64_t heads = (uint64_t)a.tokens * (uint64_t)(a.hq + a.hk);
  const uint64_t waves = (heads + kHpw - 1) / kHpw;
  const uint64_t wgs = (waves + kWavesPerWG - 1) / kWavesPerWG;
  if (wgs == 0) return hipSuccess;
  hipLaunchKernelGGL((k_qk_norm<D, E>), dim3((uint32_t)wgs), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

template <int D>
hipError_t launch_qk_d(const QkArgs& a, hipStream_t s) {
  if (qk_epl() == 16) return launch_qk_de<D, 16>(a, s);
  return qk_epl() == 32 ? launch_qk_de<D, 32>(a, s) : launch_qk_de<D, 8>(a, s);
}

}  // namespace

hipError_t launch_qk_norm(const QkArgs& a, hipStream_t s) {
  if (a.d == 64) return launch_qk_d<64>(a, s);
  if (a.d == 128) return launch_qk_d<128>(a, s);
  if (a.d == 256) return launch_qk_d<256>(a, s);
  return hipErrorInvalidValue;
}

}  // namespace nvfp4q
