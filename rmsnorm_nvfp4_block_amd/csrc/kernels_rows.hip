// Rowwise kernels for gfx950: tensor amax and rowwise NVFP4 quantization.
//
// Layout: one wave owns one row at a time. A row is cut into superchunks of
// 1024 columns; in each superchunk lane l holds one whole 16-element block,
// columns 16l .. 16l+15, read as two adjacent 16-byte loads (together the wave
// reads 2 KiB contiguous). The block amax, its scale and its 16 codes are then
// computed in-lane, once per block, and the codes leave as one 8-byte store per
// lane (the wave writes 512 contiguous bytes); the scale bytes of a wave are
// 64 contiguous bytes ("CuTeDSL at Perplexity", prefill and decode
// specialization: 128-bit accesses per thread; "[nvfp4_training] Optimize
// CuteDSL kernels for NVFP4 training", Optimization items 6 and 7: bf16
// widening by shift, full-width 64-bit code stores).
//
// Scales: block scale = E4M3(RN(RN(bmax/6) * S_enc)) with the division done by
// div6(); the encode multiplier comes from a 128-entry table of
// RN(1 / RN(f32(code) * S_dec)) that each workgroup fills in LDS, since the
// product takes at most 127 values per tensor ("[nvfp4_training] ...", Fast
// math).
//
// The amax pass and the encode pass are two launches: the kernel boundary is
// the grid-wide barrier between them ("CuTeDSL at Perplexity", grid
// synchronization). A single launch with an in-kernel grid barrier was
// measured slower on MI355X: a cooperative launch costs about 20 us, and even
// with the whole grid resident every form of the wait tried (tagged slots,
// per-group flags, one arrival counter) costs more than the 1.6 us of a
// kernel boundary in a graph, since it is a chain of device-scope round trips
// through memory (the probe kernels of bench.py --ceilings).
// The RMSNorm passes are in kernels_rms_stream.hip and kernels_rms_coop.hip.
#include "rows.hpp"

#include <cstdlib>

namespace nvfp4q {

// ------------------------------------------------------------------ amax
// A wave takes one span of 16 KB of one row at a time (8192 bf16 or fp16
// columns, 4096 fp32) and issues all of its 16-byte loads at once through
// a buffer resource that ends at the row's last column, so reads past cols
// return zero without guards. A launch over several stacked tensors of `rows`
// rows each (grid y = tensor) keeps one set of partials per tensor.
// At most 256 workgroups per tensor (one per CU; each wave loops over its
// spans): the encode pass reduces that many partials in every workgroup.
// Measured on 8192 x 8192 (full step): 2048 workgroups 89.6 us, 1024 86.0,
// 512 85.8, 256 84.7, 192 88.1, 128 95.1.
constexpr int kAmaxLoads = 16;
constexpr int kAmaxMaxWGs = 256;
template <int T>
__global__ __launch_bounds__(kThreads) void k_amax_rows(const RowArgs a) {
  constexpr uint32_t kSpan = kAmaxLoads * 1024 / in_size<T>();  // elements per span (16 KB)
  const char* __restrict__ x = (const char*)a.x + (int64_t)blockIdx.y * a.rows * a.ld_x * in_size<T>();
  const uint32_t rows = (uint32_t)a.rows, cols = (uint32_t)a.cols;
  const uint32_t lane = threadIdx.x & 63;
  const uint32_t wave = (uint32_t)__builtin_amdgcn_readfirstlane((int)((blockIdx.x * kThreads + threadIdx.x) >> 6));
  const uint32_t nwaves = (gridDim.x * kThreads) >> 6;
  const uint32_t ngrp = (cols + kSpan - 1) / kSpan;  // spans per row
  const uint64_t units = (uint64_t)rows * ngrp;
  float m = 0.0f;
  for (uint64_t u = wave; u < units; u += nwaves) {
    const uint32_t r = (uint32_t)(u / ngrp), c0 = (uint32_t)(u - (uint64_t)r * ngrp) * kSpan;
    const uint32_t left = cols - c0 < kSpan ? cols - c0 : kSpan;
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(x + ((int64_t)r * a.ld_x + c0) * in_size<T>()), (short)0, (int)(left * in_size<T>()), 0x00020000);
    uint4 q[kAmaxLoads];
#pragma unroll
    for (int k = 0; k < kAmaxLoads; ++k) {
      const auto t = __builtin_amdgcn_raw_buffer_load_b128(rs, (uint32_t)k * 1024u + lane * 16u, 0, 0);
      q[k] = make_uint4(t[0], t[1], t[2], t[3]);
    }
#pragma unroll
    for (int k = 0; k < kAmaxLoads; ++k) m = fmaxf(m, max_abs16b<T>(q[k]));
  }
  publish_partial(a.ws, m);
}

// ------------------------------------------------------------------ quantize
template <bool SR, int T>
__global__ __launch_bounds__(kThreads) void k_quant_rows(const RowArgs a) {
  __shared__ float rcp_tab[128];
  const GScale g = consume_scales(a.ws, a.nparts, a.amax_in, a.amax_out, a.scale_out, rcp_tab);
  const char* __restrict__ x = (const char*)a.x;
  const uint32_t rows = (uint32_t)a.rows, cols = (uint32_t)a.cols;
  const int lane = threadIdx.x & 63;
  const uint32_t wave = (blockIdx.x * kThreads + threadIdx.x) >> 6;
  const uint32_t nwaves = (gridDim.x * kThreads) >> 6;
  const uint32_t nsc = (cols + kSuper - 1) / kSuper;
  const uint32_t nbr = cols >> 4;  // blocks per row
  for (uint32_t r = wave; r < rows; r += nwaves) {
    const char* xr = x + (int64_t)r * a.ld_x * in_size<T>();
    uint8_t* cr = a.codes + (int64_t)r * a.ldc;
    uint8_t* sr = a.scales + (int64_t)r * a.lds;
    for (uint32_t s0 = 0; s0 < nsc; s0 += 2) {
      Raw16<T> b[2];
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const uint32_t col = (s0 + u) * kSuper + lane * 16;
        b[u] = load_raw16<T>(xr, col, (s0 + u) < nsc && col < cols);
      }
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const uint32_t col = (s0 + u) * kSuper + lane * 16;
        float v[16];
        widen_raw16<T>(b[u], v);
        uint32_t sc;
        const uint2 w = encode_block16<SR>(v, g, rcp_tab, sc, (uint64_t)r * nbr + (col >> 4), a.seed, a.offset, 0);
        if ((s0 + u) < nsc && col < cols) {
          __builtin_nontemporal_store((uint64_t)w.x | ((uint64_t)w.y << 32), reinterpret_cast<uint64_t*>(cr + (col >> 1)));
          __builtin_nontemporal_store((uint8_t)sc, sr + (col >> 4));
        }
      }
    }
  }
}

__global__ void k_empty_scale(float* amax_out, float* scale_out, int n) {
  const int i = threadIdx.x;
  if (i < n) {
    if (amax_out) amax_out[i] = 0.0f;
    if (scale_out) scale_out[i] = 1.0f;
  }
}

// ------------------------------------------------------------------ launchers
hipError_t launch_empty_scale(float* amax_out, float* scale_out, int n, hipStream_t s) {
  if (!amax_out && !scale_out) return hipSuccess;
  hipLaunchKernelGGL(k_empty_scale, dim3(1), dim3(64), 0, s, amax_out, scale_out, n);
  return hipGetLastError();
}

// Workgroups of the amax pass at most: NVFP4Q_AMAX_WGS (1 .. 2048), default
// kAmaxMaxWGs.
int64_t amax_wgs() {
  static int64_t v = [] {
    const char* e = getenv("NVFP4Q_AMAX_WGS");
    const int64_t n = e ? (int64_t)atoll(e) : (int64_t)kAmaxMaxWGs;
    return n < 1 ? (int64_t)1 : n > 2048 ? (int64_t)2048 : n;
  }();
  return v;
}

hipError_t launch_amax_rows(const RowArgs& a, hipStream_t s, uint32_t* nparts, int tensors) {
  const int64_t span = kAmaxLoads * 1024 / (a.dtype == kInFP32 ? 4 : 2);  // elements per span
  const int64_t units = a.rows * ((a.cols + span - 1) / span);  // one per wave at most
  int64_t wgs = (units + kWavesPerWG - 1) / kWavesPerWG;
  if (wgs > amax_wgs()) wgs = amax_wgs();
  if (wgs < 1) wgs = 1;
  *nparts = (uint32_t)wgs;
  const dim3 grid((uint32_t)wgs, (uint32_t)tensors);
  if (a.dtype == kInFP16) hipLaunchKernelGGL(k_amax_rows<kInFP16>, grid, dim3(kThreads), 0, s, a);
  else if (a.dtype == kInFP32) hipLaunchKernelGGL(k_amax_rows<kInFP32>, grid, dim3(kThreads), 0, s, a);
  else hipLaunchKernelGGL(k_amax_rows<kInBF16>, grid, dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_quant_rows(const RowArgs& a, hipStream_t s) {
  dim3 grid(grid_rows(a.rows)), block(kThreads);
  if (a.dtype == kInFP16) {
    if (a.sr) hipLaunchKernelGGL((k_quant_rows<true, kInFP16>), grid, block, 0, s, a);
    else hipLaunchKernelGGL((k_quant_rows<false, kInFP16>), grid, block, 0, s, a);
  } else if (a.dtype == kInFP32) {
    if (a.sr) hipLaunchKernelGGL((k_quant_rows<true, kInFP32>), grid, block, 0, s, a);
    else hipLaunchKernelGGL((k_quant_rows<false, kInFP32>), grid, block, 0, s, a);
  } else {
    if (a.sr) hipLaunchKernelGGL((k_quant_rows<true, kInBF16>), grid, block, 0, s, a);
    else hipLaunchKernelGGL((k_quant_rows<false, kInBF16>), grid, block, 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace nvfp4q
