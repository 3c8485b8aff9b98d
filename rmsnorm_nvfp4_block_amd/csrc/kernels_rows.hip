// Rowwise kernels for gfx950: tensor amax, rowwise NVFP4 quantization and the
// fused RMSNorm + rowwise NVFP4 passes.
//
// Layout: one wave owns one row at a time. A row is cut into chunks of 512
// columns; in each chunk lane l holds the 8 consecutive bf16 values at columns
// 8l .. 8l+7 (one 128-bit load; the wave covers 1 KiB contiguous). A 16-element
// block is the lane pair (2m, 2m+1): its amax is one DPP exchange, each lane
// then encodes its own 8 values and writes 4 code bytes, so a wave's code
// stores are 256 contiguous bytes ("CuTeDSL at Perplexity", prefill and decode
// specialization: 128-bit accesses per thread; "[nvfp4_training] Optimize
// CuteDSL kernels for NVFP4 training", Optimization items 6 and 7: bf16
// widening by shift, full-width code stores).
#include "device.hpp"
#include "launch.hpp"

namespace nvfp4q {

constexpr int kThreads = 256;        // 4 waves per workgroup
constexpr int kWavesPerWG = kThreads / kWave;

// ------------------------------------------------------------------ helpers
__device__ __forceinline__ uint4 load16(const uint16_t* p, bool ok) {
  uint4 z = {0u, 0u, 0u, 0u};
  return ok ? *reinterpret_cast<const uint4*>(p) : z;
}

// Reduce a per-lane float max over the workgroup, then (thread 0) fold it into
// the workspace accumulator `slot` and elect the last workgroup, which turns
// the accumulator into the per-tensor scales and resets the state.
__device__ __forceinline__ void wg_amax_and_finalize(float m, Workspace* ws, int slot, float* amax_out,
                                                     float* scale_out) {
  __shared__ float red[kWavesPerWG];
  m = wave_max(m);
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  if (lane == 0) red[wid] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    float t = red[0];
    for (int i = 1; i < kWavesPerWG; ++i) t = fmaxf(t, red[i]);
    atomic_max_f32_nonneg(&ws->amax_bits[slot], t);
    if (arrive_last(&ws->count, gridDim.x)) {
      float a = load_amax(&ws->amax_bits[slot]);
      GScale g = global_scale(a);
      ws->enc[slot] = g.enc;
      ws->dec[slot] = g.dec;
      ws->amax[slot] = a;
      if (amax_out) amax_out[slot] = a;
      if (scale_out) scale_out[slot] = g.dec;
      __hip_atomic_store(&ws->amax_bits[slot], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

// Global scales for a quantize pass: from amax_in when given (and workgroup 0
// reports them), otherwise from the workspace result written by the amax pass.
__device__ __forceinline__ GScale pass_scales(const Workspace* ws, const float* amax_in, float* amax_out,
                                              float* scale_out) {
  if (amax_in) {
    float a = *amax_in;
    GScale g = global_scale(a);
    if (blockIdx.x == 0 && threadIdx.x == 0) {
      if (amax_out) *amax_out = a;
      if (scale_out) *scale_out = g.dec;
    }
    return g;
  }
  GScale g;
  g.enc = ws->enc[0];
  g.dec = ws->dec[0];
  return g;
}

// Encode one lane's half block (8 values): returns the packed code word and the
// block's scale code. The partner lane (lane ^ 1) holds the other half.
template <bool SR>
__device__ __forceinline__ uint32_t encode_half(float v[8], GScale g, uint32_t& sc, uint64_t blk, uint64_t seed,
                                                uint32_t offset, uint32_t tag) {
  float m = max8_abs(v);
  float bm = fmaxf(m, swap_pair(m));
  sc = block_scale(bm, g.enc);
  float rc = encode_mult(sc, g.dec);
#pragma unroll
  for (int i = 0; i < 8; ++i) v[i] = v[i] * rc;
  if constexpr (SR) {
    U4 w = block_random(blk, tag, seed, offset);
    const bool odd = (threadIdx.x & 1) != 0;
    return sr_pack8(v, odd ? w.z : w.x, odd ? w.w : w.y);
  } else {
    return rtne_pack8(v);
  }
}

// ------------------------------------------------------------------ amax
// amax of a [rows, cols] bf16 tensor into workspace slot 0 (+ scales).
constexpr int kAmaxUnroll = 4;
__global__ __launch_bounds__(kThreads) void k_amax_rows(const uint16_t* __restrict__ x, uint32_t rows,
                                                        uint32_t cols, int64_t ld_x, Workspace* ws,
                                                        float* amax_out, float* scale_out) {
  const int lane = threadIdx.x & 63;
  const uint32_t wave = (blockIdx.x * kThreads + threadIdx.x) >> 6;
  const uint32_t nwaves = (gridDim.x * kThreads) >> 6;
  const uint32_t nch = (cols + 511) >> 9;
  float m = 0.0f;
  for (uint32_t r = wave; r < rows; r += nwaves) {
    const uint16_t* xr = x + (int64_t)r * ld_x;
    for (uint32_t c0 = 0; c0 < nch; c0 += kAmaxUnroll) {
      uint4 q[kAmaxUnroll];
#pragma unroll
      for (int u = 0; u < kAmaxUnroll; ++u) {
        uint32_t col = (c0 + u) * 512 + lane * 8;
        q[u] = load16(xr + col, (c0 + u) < nch && col < cols);
      }
#pragma unroll
      for (int u = 0; u < kAmaxUnroll; ++u) {
        float v[8];
        widen8(q[u], v);
        m = fmaxf(m, max8_abs(v));
      }
    }
  }
  wg_amax_and_finalize(m, ws, 0, amax_out, scale_out);
}

// ------------------------------------------------------------------ quantize
constexpr int kQuantUnroll = 4;
template <bool SR>
__global__ __launch_bounds__(kThreads) void k_quant_rows(const uint16_t* __restrict__ x, uint32_t rows,
                                                         uint32_t cols, int64_t ld_x, uint8_t* __restrict__ codes,
                                                         int64_t ldc, uint8_t* __restrict__ scales, int64_t lds,
                                                         const Workspace* ws, const float* amax_in,
                                                         float* amax_out, float* scale_out, uint64_t seed,
                                                         uint32_t offset) {
  const GScale g = pass_scales(ws, amax_in, amax_out, scale_out);
  const int lane = threadIdx.x & 63;
  const uint32_t wave = (blockIdx.x * kThreads + threadIdx.x) >> 6;
  const uint32_t nwaves = (gridDim.x * kThreads) >> 6;
  const uint32_t nch = (cols + 511) >> 9;
  const uint32_t nbr = cols >> 4;  // blocks per row
  for (uint32_t r = wave; r < rows; r += nwaves) {
    const uint16_t* xr = x + (int64_t)r * ld_x;
    uint8_t* cr = codes + (int64_t)r * ldc;
    uint8_t* sr = scales + (int64_t)r * lds;
    for (uint32_t c0 = 0; c0 < nch; c0 += kQuantUnroll) {
      uint4 q[kQuantUnroll];
#pragma unroll
      for (int u = 0; u < kQuantUnroll; ++u) {
        uint32_t col = (c0 + u) * 512 + lane * 8;
        q[u] = load16(xr + col, (c0 + u) < nch && col < cols);
      }
#pragma unroll
      for (int u = 0; u < kQuantUnroll; ++u) {
        const uint32_t col = (c0 + u) * 512 + lane * 8;
        const bool ok = (c0 + u) < nch && col < cols;
        float v[8];
        widen8(q[u], v);
        uint32_t sc;
        uint32_t word = encode_half<SR>(v, g, sc, (uint64_t)r * nbr + (col >> 4), seed, offset, 0);
        if (ok) {
          *reinterpret_cast<uint32_t*>(cr + (col >> 1)) = word;
          if ((lane & 1) == 0) sr[col >> 4] = (uint8_t)sc;
        }
      }
    }
  }
}

// ------------------------------------------------------------------ RMSNorm
// One wave per token; NCH chunks of 512 columns stay in registers. Pass 1
// (AMAX) folds max |y| into the tensor amax; pass 2 normalizes again,
// rounds y to bf16 (optionally storing it) and quantizes it rowwise.
// y = bf16_rne(((gamma + c) * x) * r [+ beta]) with r = 1/sqrt(ss/K + eps), ss the
// fp32 sum of squares ("CuTeDSL at Perplexity", QK Norm).
template <int NCH, bool BIAS, bool AMAX, bool SR, bool YOUT, bool CODES>
__global__ __launch_bounds__(kThreads) void k_rmsnorm(const uint16_t* __restrict__ x, uint32_t rows,
                                                      uint32_t cols, int64_t ld_x,
                                                      const uint16_t* __restrict__ gamma,
                                                      const uint16_t* __restrict__ beta, float woff, float eps,
                                                      uint16_t* __restrict__ y_out, int64_t ld_y,
                                                      uint8_t* __restrict__ codes, int64_t ldc,
                                                      uint8_t* __restrict__ scales, int64_t lds, Workspace* ws,
                                                      const float* amax_in, float* amax_out, float* scale_out,
                                                      uint64_t seed, uint32_t offset) {
  GScale g = {1.0f, 1.0f};
  if constexpr (!AMAX && CODES) g = pass_scales(ws, amax_in, amax_out, scale_out);
  const int lane = threadIdx.x & 63;
  const uint32_t wave = (blockIdx.x * kThreads + threadIdx.x) >> 6;
  const uint32_t nwaves = (gridDim.x * kThreads) >> 6;
  const uint32_t nbr = cols >> 4;
  const float inv_k = 1.0f / (float)cols;
  float mloc = 0.0f;
  for (uint32_t r = wave; r < rows; r += nwaves) {
    const uint16_t* xr = x + (int64_t)r * ld_x;
    uint4 q[NCH];
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      uint32_t col = c * 512 + lane * 8;
      q[c] = load16(xr + col, col < cols);
    }
    float ss = 0.0f;
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      ss = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, q[c].x), __builtin_bit_cast(bf16x2, q[c].x), ss, false);
      ss = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, q[c].y), __builtin_bit_cast(bf16x2, q[c].y), ss, false);
      ss = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, q[c].z), __builtin_bit_cast(bf16x2, q[c].z), ss, false);
      ss = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, q[c].w), __builtin_bit_cast(bf16x2, q[c].w), ss, false);
    }
    ss = wave_sum(ss);
    const float rs = 1.0f / sqrtf(ss * inv_k + eps);
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      const uint32_t col = c * 512 + lane * 8;
      const bool ok = col < cols;
      float v[8], gv[8];
      widen8(q[c], v);
      widen8(load16(gamma + col, ok), gv);
      float bv[8];
      if constexpr (BIAS) widen8(load16(beta + col, ok), bv);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        float t = v[i] * (gv[i] + woff);
        if constexpr (BIAS) v[i] = fmaf(t, rs, bv[i]);
        else v[i] = t * rs;
      }
      if constexpr (AMAX) {
        mloc = fmaxf(mloc, ok ? max8_abs(v) : 0.0f);
      } else {
        uint4 yb;
        yb.x = pack_bf16(v[0], v[1]);
        yb.y = pack_bf16(v[2], v[3]);
        yb.z = pack_bf16(v[4], v[5]);
        yb.w = pack_bf16(v[6], v[7]);
        if constexpr (YOUT) {
          if (ok) *reinterpret_cast<uint4*>(y_out + (int64_t)r * ld_y + col) = yb;
        }
        if constexpr (CODES) {
          widen8(yb, v);
          uint32_t sc;
          uint32_t word = encode_half<SR>(v, g, sc, (uint64_t)r * nbr + (col >> 4), seed, offset, 0);
          if (ok) {
            *reinterpret_cast<uint32_t*>(codes + (int64_t)r * ldc + (col >> 1)) = word;
            if ((lane & 1) == 0) scales[(int64_t)r * lds + (col >> 4)] = (uint8_t)sc;
          }
        }
      }
    }
  }
  if constexpr (AMAX) {
    // max |bf16(y)| = bf16(max |y|): round-to-nearest-even is monotone.
    float mb = bf_lo(pack_bf16(mloc, mloc) & 0xFFFFu);
    wg_amax_and_finalize(mb, ws, 0, amax_out, scale_out);
  }
}

// Empty tensor: amax 0, S_dec 1.
__global__ void k_empty_scale(float* amax_out, float* scale_out, int n) {
  int i = threadIdx.x;
  if (i < n) {
    if (amax_out) amax_out[i] = 0.0f;
    if (scale_out) scale_out[i] = 1.0f;
  }
}

// ------------------------------------------------------------------ launchers
static inline uint32_t grid_rows(int64_t rows) {
  int64_t wgs = (rows + kWavesPerWG - 1) / kWavesPerWG;
  if (wgs > 4096) wgs = 4096;
  if (wgs < 1) wgs = 1;
  return (uint32_t)wgs;
}

hipError_t launch_empty_scale(float* amax_out, float* scale_out, int n, hipStream_t s) {
  if (!amax_out && !scale_out) return hipSuccess;
  hipLaunchKernelGGL(k_empty_scale, dim3(1), dim3(64), 0, s, amax_out, scale_out, n);
  return hipGetLastError();
}

hipError_t launch_amax_rows(const RowArgs& a, hipStream_t s) {
  // about two passes' worth of waves in flight per CU; never more workgroups than rows need
  int64_t wgs = (a.rows + kWavesPerWG - 1) / kWavesPerWG;
  if (wgs > 1024) wgs = 1024;
  if (wgs < 1) wgs = 1;
  hipLaunchKernelGGL(k_amax_rows, dim3((uint32_t)wgs), dim3(kThreads), 0, s, (const uint16_t*)a.x,
                     (uint32_t)a.rows, (uint32_t)a.cols, a.ld_x, a.ws, a.amax_out, a.scale_out);
  return hipGetLastError();
}

hipError_t launch_quant_rows(const RowArgs& a, hipStream_t s) {
  dim3 grid(grid_rows(a.rows)), block(kThreads);
  if (a.sr)
    hipLaunchKernelGGL(k_quant_rows<true>, grid, block, 0, s, (const uint16_t*)a.x, (uint32_t)a.rows,
                       (uint32_t)a.cols, a.ld_x, a.codes, a.ldc, a.scales, a.lds, a.ws, a.amax_in, a.amax_out,
                       a.scale_out, a.seed, a.offset);
  else
    hipLaunchKernelGGL(k_quant_rows<false>, grid, block, 0, s, (const uint16_t*)a.x, (uint32_t)a.rows,
                       (uint32_t)a.cols, a.ld_x, a.codes, a.ldc, a.scales, a.lds, a.ws, a.amax_in, a.amax_out,
                       a.scale_out, a.seed, a.offset);
  return hipGetLastError();
}

template <int NCH, bool BIAS, bool AMAX, bool SR, bool YOUT, bool CODES>
static void launch_rms_t(const RowArgs& a, hipStream_t s) {
  hipLaunchKernelGGL((k_rmsnorm<NCH, BIAS, AMAX, SR, YOUT, CODES>), dim3(grid_rows(a.rows)), dim3(kThreads), 0, s,
                     (const uint16_t*)a.x, (uint32_t)a.rows, (uint32_t)a.cols, a.ld_x, (const uint16_t*)a.gamma,
                     (const uint16_t*)a.beta, a.woff, a.eps, (uint16_t*)a.y, a.ld_y, a.codes, a.ldc, a.scales,
                     a.lds, a.ws, a.amax_in, a.amax_out, a.scale_out, a.seed, a.offset);
}

template <int NCH, bool BIAS>
static void launch_rms_mode(const RowArgs& a, bool amax_pass, hipStream_t s) {
  const bool yout = a.y != nullptr, codes = a.codes != nullptr;
  if (amax_pass) {
    launch_rms_t<NCH, BIAS, true, false, false, false>(a, s);
  } else if (!codes) {
    launch_rms_t<NCH, BIAS, false, false, true, false>(a, s);
  } else if (a.sr) {
    if (yout) launch_rms_t<NCH, BIAS, false, true, true, true>(a, s);
    else launch_rms_t<NCH, BIAS, false, true, false, true>(a, s);
  } else {
    if (yout) launch_rms_t<NCH, BIAS, false, false, true, true>(a, s);
    else launch_rms_t<NCH, BIAS, false, false, false, true>(a, s);
  }
}

template <int NCH>
static void launch_rms_bias(const RowArgs& a, bool amax_pass, hipStream_t s) {
  if (a.beta) launch_rms_mode<NCH, true>(a, amax_pass, s);
  else launch_rms_mode<NCH, false>(a, amax_pass, s);
}

// Register-resident row variants: smallest instantiated chunk count that
// covers the row.
int rms_max_cols() { return 32 * 512; }

hipError_t launch_rmsnorm_pass(const RowArgs& a, bool amax_pass, hipStream_t s) {
  const int64_t need = (a.cols + 511) / 512;
  if (need <= 1) launch_rms_bias<1>(a, amax_pass, s);
  else if (need <= 2) launch_rms_bias<2>(a, amax_pass, s);
  else if (need <= 4) launch_rms_bias<4>(a, amax_pass, s);
  else if (need <= 8) launch_rms_bias<8>(a, amax_pass, s);
  else if (need <= 14) launch_rms_bias<14>(a, amax_pass, s);
  else if (need <= 16) launch_rms_bias<16>(a, amax_pass, s);
  else if (need <= 24) launch_rms_bias<24>(a, amax_pass, s);
  else if (need <= 32) launch_rms_bias<32>(a, amax_pass, s);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace nvfp4q
