// Streaming form of the two RMSNorm + rowwise NVFP4 passes.
//
// A row's 1/rms is known only after its whole sum of squares; the
// cooperative-row kernels (kernels_rms_coop.hip) meet that with a workgroup
// barrier per row. Here the amax pass writes each row's 1/rms into the
// workspace, so the encode pass reads it back and no pass waits on a row:
// a wave walks its rows one 1024-column superchunk at a time (lane l: the
// 16-element block at columns 16l..16l+15) with kDepth superchunks in flight,
// and compute overlaps the loads of the superchunks behind it.
//
//  * Amax pass (no bias): per lane, the running sum of squares and the
//    running max |RN(x * (gamma + c))| of the current row; at the row's last
//    superchunk, r = 1/rms from the wave sum, r goes to the workspace, and
//    RN(max * r) joins the wave's maximum. Since y = RN(RN(x * g) * r) is
//    monotone in |RN(x * g)| for the row's fixed r > 0, that is the row's
//    max |y|. With a bias the max depends on r element by element; that case
//    keeps the cooperative-row amax pass (which also stores r).
//  * Encode pass: y = RN(RN(x * g) * r) [+ beta, fused], rounded to the
//    input's type, then the block encode, as in the cooperative-row pass;
//    codes and scale bytes leave with non-temporal stores (they are not read
//    again by this call). Lane k of a wave holds r of the wave's k-th row (a
//    wave has at most 64 rows; the launcher sizes the grid for it).
//
// The ring of superchunks is refilled only in iterations that have a next
// one, and the last iteration issues no loads: a refill that may or may not
// happen makes the compiler copy the ring at the loop back edge, and the copy
// waits for the refill loads to land.
//
// The element type T of x (bf16, fp16 or fp32) is a template parameter: a
// block is two or four 16-byte loads, gamma and beta come in T, y is rounded
// to nearest even in T (fp32: not rounded further), and bf16 keeps its
// dot-product sum of squares and two-step parameter staging.
//
// "CuTeDSL at Perplexity", QK Norm (the normalization) and grid
// synchronization (the kernel boundary between the amax and the encode pass).
#include <type_traits>

#include "rows.hpp"

namespace nvfp4q {

namespace {

constexpr int kDepth = 4;              // superchunks in flight per wave
constexpr uint32_t kMaxWaveRows = 64;  // rows per wave in the encode pass

// Row and superchunk of a wave's next load or next block to process; the
// wave's rows are wave, wave + nwaves, ...; k counts the wave's rows.
struct Cursor {
  uint32_t row, sc, k;
  __device__ __forceinline__ void next(uint32_t nsc, uint32_t nwaves) {
    if (++sc == nsc) {
      sc = 0;
      row += nwaves;
      ++k;
    }
  }
};

// The lane's block at column `col` of row xr (zero when outside the row).
template <bool FULL, int T>
__device__ __forceinline__ Raw16<T> load_blk_t(const char* xr, uint32_t col, uint32_t cols) {
  if constexpr (FULL) {
    Raw16<T> b;
    const char* p = xr + (size_t)col * in_size<T>();
#pragma unroll
    for (int l = 0; l < in_size<T>(); ++l) b.q[l] = *reinterpret_cast<const uint4*>(p + 16 * l);
    return b;
  } else {
    return load_raw16<T>(xr, col, col < cols);
  }
}

template <int T>
__device__ __forceinline__ const char* row_ptr(const RowArgs& a, uint32_t row) {
  return (const char*)a.x + (int64_t)row * a.ld_x * in_size<T>();
}

template <bool FULL, int T>
__device__ __forceinline__ Raw16<T> load_at(const RowArgs& a, Cursor c, uint32_t cols, int lane) {
  return load_blk_t<FULL, T>(row_ptr<T>(a, c.row), c.sc * kSuper + lane * 16, cols);
}

// Refill of a slot with the item at `ld` (item number `item`); past the
// wave's last item `ld` stays on that item (a cache hit).
template <bool FULL, int T>
__device__ __forceinline__ void refill(const RowArgs& a, Raw16<T>& slot, Cursor& ld, uint32_t item, uint32_t n,
                                       uint32_t nsc, uint32_t nwaves, uint32_t cols, int lane) {
  slot = load_at<FULL, T>(a, ld, cols, lane);
  if (item + 1 < n) ld.next(nsc, nwaves);
}

// Wave index with the wave-uniform part kept in scalar registers.
__device__ __forceinline__ uint32_t wave_id() {
  return blockIdx.x * kWavesPerWG + (uint32_t)__builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
}

__device__ __forceinline__ uint32_t wave_rows(uint32_t wave, uint32_t nwaves, uint32_t rows) {
  return wave < rows ? (rows - 1 - wave) / nwaves + 1 : 0;
}

// Row parameters into LDS: bf16 in two steps around the ring's first loads
// (issue, then finish after the fill), other types by a plain loop after it.
template <bool BIAS, int T>
__device__ __forceinline__ ParamsPre stage_issue(const RowArgs& a, uint32_t cols) {
  if constexpr (T == kInBF16) return params_issue<BIAS>((const uint16_t*)a.gamma, (const uint16_t*)a.beta, cols);
  return ParamsPre{};
}
template <bool BIAS, int T>
__device__ __forceinline__ void stage_finish(const ParamsPre& pp, const RowArgs& a, uint32_t cols, float* gsh,
                                             float* bsh) {
  if constexpr (T == kInBF16)
    params_finish<BIAS>(pp, (const uint16_t*)a.gamma, (const uint16_t*)a.beta, a.woff, cols, gsh, bsh);
  else
    stage_params_t<BIAS, T>(a.gamma, a.beta, a.woff, cols, gsh, bsh);
}

// ------------------------------------------------------------------ amax pass
struct AmaxAcc {
  float ss, m, macc;
};

template <bool FULL, int T>
__device__ __forceinline__ void amax_item(const RowArgs& a, const Raw16<T>& b, const Cursor& pc, const float* gsh,
                                          uint32_t nsc, uint32_t cols, float inv_k, int lane, AmaxAcc& acc) {
  float v[16], gv[16];
  widen_raw16<T>(b, v);
  if constexpr (T == kInBF16) {
    acc.ss = sumsq8(b.q[1], sumsq8(b.q[0], acc.ss));
  } else {
#pragma unroll
    for (int k = 0; k < 16; ++k) acc.ss = __builtin_fmaf(v[k], v[k], acc.ss);
  }
  const uint32_t col = pc.sc * kSuper + lane * 16;
  lds16(gsh, (FULL || col < cols) ? col : 0, gv);
#pragma unroll
  for (int k = 0; k < 16; ++k) v[k] = v[k] * gv[k];
  acc.m = fmaxf(acc.m, max16_abs(v));
  if (pc.sc == nsc - 1) {
    const float r = inv_rms(wave_sum(acc.ss), inv_k, a.eps);
    if (lane == 0) a.rs[pc.row] = r;
    acc.macc = fmaxf(acc.macc, acc.m * r);
    acc.ss = 0.0f;
    acc.m = 0.0f;
  }
}

template <bool FULL, int T>
__global__ __launch_bounds__(kThreads) void k_rms_amax_stream(const RowArgs a) {
  extern __shared__ float gsh[];  // gamma + c [cols]
  const uint32_t rows = (uint32_t)a.rows, cols = (uint32_t)a.cols;
  const int lane = threadIdx.x & 63;
  const uint32_t wave = wave_id(), nwaves = gridDim.x * kWavesPerWG;
  const uint32_t nsc = (cols + kSuper - 1) / kSuper;
  const uint32_t n = wave_rows(wave, nwaves, rows) * nsc;
  // the prologue's loads first: loads complete in issue order
  const ParamsPre pp = stage_issue<false, T>(a, cols);
  // unconditional fill (a wave without rows reads the last row): a fill that
  // may be skipped would make every later wait a wait for all loads
  Raw16<T> ring[kDepth];
  Cursor ld{wave < rows ? wave : rows - 1, 0, 0};
#pragma unroll
  for (int d = 0; d < kDepth; ++d) refill<FULL, T>(a, ring[d], ld, d, n, nsc, nwaves, cols, lane);
  stage_finish<false, T>(pp, a, cols, gsh, nullptr);
  __syncthreads();
  const float inv_k = 1.0f / (float)cols;
  AmaxAcc acc{0.0f, 0.0f, 0.0f};
  Cursor pc{wave, 0, 0};
  for (uint32_t base = 0; base < n; base += kDepth) {
    if (base + kDepth < n) {
#pragma unroll
      for (int d = 0; d < kDepth; ++d) {
        amax_item<FULL, T>(a, ring[d], pc, gsh, nsc, cols, inv_k, lane, acc);
        refill<FULL, T>(a, ring[d], ld, base + kDepth + d, n, nsc, nwaves, cols, lane);
        pc.next(nsc, nwaves);
      }
    } else {
#pragma unroll
      for (int d = 0; d < kDepth; ++d) {
        if (base + d < n) {
          amax_item<FULL, T>(a, ring[d], pc, gsh, nsc, cols, inv_k, lane, acc);
          pc.next(nsc, nwaves);
        }
      }
    }
  }
  // max |RN_T(y)| = RN_T(max |y|): round-to-nearest-even is monotone.
  publish_partial(a.ws, round_t<T>(acc.macc));
}

// ------------------------------------------------------------------ encode pass
// y = v rounded to nearest even in T, stored at (row, col) of y when y is
// asked for and the block is inside the row; v becomes the rounded values.
// (Y: y is asked for, a compile-time choice of the caller.)
template <int T, bool Y>
__device__ __forceinline__ void round_y(const RowArgs& a, float (&v)[16], uint32_t row, uint32_t col, bool ok) {
  if constexpr (!Y) {
    round16<T>(v);
    return;
  }
  if constexpr (T == kInBF16) {
    const uint4 y0 = pack8_bf16(v), y1 = pack8_bf16(v + 8);
    if (ok) {
      uint16_t* yr = (uint16_t*)a.y + (int64_t)row * a.ld_y + col;
      *reinterpret_cast<uint4*>(yr) = y0;
      *reinterpret_cast<uint4*>(yr + 8) = y1;
    }
    widen8(y0, v);
    widen8(y1, v + 8);
  } else {
    round_store16<T>(v, (char*)a.y + ((int64_t)row * a.ld_y + col) * in_size<T>(), 0u, ok);
  }
}

__device__ __forceinline__ void st_nt8(uint8_t* p, uint2 w) {
  __builtin_nontemporal_store((uint64_t)w.x | ((uint64_t)w.y << 32), reinterpret_cast<uint64_t*>(p));
}

// One block of the encode pass: lane's 16 values of row `row` at column `col`,
// gamma + c and beta of those columns in registers, r the row's 1/rms.
// (v: the block's 16 inputs, already widened to fp32)
template <bool BIAS, bool SR, int T>
__device__ __forceinline__ void quant_item(const RowArgs& a, float (&v)[16], uint32_t row, uint32_t col, bool ok,
                                           float r, const float (&gv)[16], const float (&bv)[16], GScale g,
                                           const float* rcp_tab, uint32_t cols) {
#pragma unroll
  for (int k = 0; k < 16; ++k) v[k] = v[k] * gv[k];
  if constexpr (BIAS) {
#pragma unroll
    for (int k = 0; k < 16; ++k) v[k] = __builtin_fmaf(v[k], r, bv[k]);
  } else {
#pragma unroll
    for (int k = 0; k < 16; ++k) v[k] = v[k] * r;
  }
  // y rounded in T, stored when asked for; the quantizer takes the rounded values
  if (a.y != nullptr) round_y<T, true>(a, v, row, col, ok);
  else round_y<T, false>(a, v, row, col, ok);
  uint32_t sc;
  const uint2 w = encode_block16<SR>(v, g, rcp_tab, sc, (uint64_t)row * (cols >> 4) + (col >> 4), a.seed, a.offset, 0);
  if (ok) {
    st_nt8(a.codes + (int64_t)row * a.ldc + (col >> 1), w);
    __builtin_nontemporal_store((uint8_t)sc, a.scales + (int64_t)row * a.lds + (col >> 4));
  }
}

// One block of the row-per-wave encode pass (gamma + c and beta from LDS).
template <bool FULL, bool BIAS, bool SR, int T, bool Y>
__device__ __forceinline__ void quant_item_rw(const RowArgs& a, const Raw16<T>& b, const Cursor& pc, float r_lane,
                                           const float* gsh, const float* bsh, GScale g, const float* rcp_tab,
                                           uint32_t cols, int lane) {
  const float r = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, r_lane), (int)pc.k));
  const uint32_t col = pc.sc * kSuper + lane * 16;
  const bool ok = FULL || col < cols;
  const uint32_t lcol = ok ? col : 0;
  float v[16], gv[16];
  widen_raw16<T>(b, v);
  lds16(gsh, lcol, gv);
#pragma unroll
  for (int k = 0; k < 16; ++k) v[k] = v[k] * gv[k];
  if constexpr (BIAS) {
    float bv[16];
    lds16(bsh, lcol, bv);
#pragma unroll
    for (int k = 0; k < 16; ++k) v[k] = __builtin_fmaf(v[k], r, bv[k]);
  } else {
#pragma unroll
    for (int k = 0; k < 16; ++k) v[k] = v[k] * r;
  }
  round_y<T, Y>(a, v, pc.row, col, ok);
  uint32_t sc;
  const uint2 w =
      encode_block16<SR>(v, g, rcp_tab, sc, (uint64_t)pc.row * (cols >> 4) + (col >> 4), a.seed, a.offset, 0);
  if (ok) {
    st_nt8(a.codes + (int64_t)pc.row * a.ldc + (col >> 1), w);
    __builtin_nontemporal_store((uint8_t)sc, a.scales + (int64_t)pc.row * a.lds + (col >> 4));
  }
}

// Encode pass, one row per wave at a time (rows wave, wave + nwaves, ...; at
// most 64 per wave, lane k holding 1/rms of the wave's k-th row): the row's
// superchunks stream through a kDepth ring with gamma + c (and beta) in LDS.
// Used when there are enough rows to give every SIMD several waves.
template <bool FULL, bool BIAS, bool SR, int T>
__global__ __launch_bounds__(kThreads) void k_rms_quant_rowwave(const RowArgs a) {
  extern __shared__ float params[];  // gamma + c [cols], then beta [cols]
  __shared__ float rcp_tab[128];
  const uint32_t rows = (uint32_t)a.rows, cols = (uint32_t)a.cols;
  const int lane = threadIdx.x & 63;
  const uint32_t wave = wave_id(), nwaves = gridDim.x * kWavesPerWG;
  const uint32_t nsc = (cols + kSuper - 1) / kSuper;
  const uint32_t wr = wave_rows(wave, nwaves, rows);  // <= kMaxWaveRows
  const uint32_t n = wr * nsc;
  // the prologue's loads first: loads complete in issue order
  const PartialsPre pm = partials_issue(a.ws, a.nparts, a.amax_in);
  const ParamsPre pp = stage_issue<BIAS, T>(a, cols);
  const float r_lane = (uint32_t)lane < wr ? a.rs[wave + lane * nwaves] : 0.0f;
  // unconditional fill (a wave without rows reads the last row): a fill that
  // may be skipped would make every later wait a wait for all loads
  Raw16<T> ring[kDepth];
  Cursor ld{wave < rows ? wave : rows - 1, 0, 0};
#pragma unroll
  for (int d = 0; d < kDepth; ++d) refill<FULL, T>(a, ring[d], ld, d, n, nsc, nwaves, cols, lane);
  float* gsh = params;
  float* bsh = params + param_floats(cols);
  stage_finish<BIAS, T>(pp, a, cols, gsh, bsh);
  const GScale g = partials_finish(pm, a.ws, a.nparts, a.amax_in, a.amax_out, a.scale_out, rcp_tab);
  Cursor pc{wave, 0, 0};
  // the items, with y stored or not as a compile-time choice
  auto items = [&](auto ytag) {
    constexpr bool Y = decltype(ytag)::value;
    for (uint32_t base = 0; base < n; base += kDepth) {
      if (base + kDepth < n) {
#pragma unroll
        for (int d = 0; d < kDepth; ++d) {
          quant_item_rw<FULL, BIAS, SR, T, Y>(a, ring[d], pc, r_lane, gsh, bsh, g, rcp_tab, cols, lane);
          refill<FULL, T>(a, ring[d], ld, base + kDepth + d, n, nsc, nwaves, cols, lane);
          pc.next(nsc, nwaves);
        }
      } else {
#pragma unroll
        for (int d = 0; d < kDepth; ++d) {
          if (base + d < n) {
            quant_item_rw<FULL, BIAS, SR, T, Y>(a, ring[d], pc, r_lane, gsh, bsh, g, rcp_tab, cols, lane);
            pc.next(nsc, nwaves);
          }
        }
      }
    }
  };
  if (a.y != nullptr) items(std::true_type{});
  else items(std::false_type{});
}

// Encode pass, one superchunk column per wave (for few rows: decode-sized
// calls get nsc times as many waves as rows). Wave w owns one superchunk column, sc = w mod nsc, and the rows
// w / nsc + j * wps, j = 0 .. nr-1 (wps waves per superchunk column, nr <= 64):
// its lanes keep their 16 values of gamma + c (and beta) in registers for the
// whole kernel, and lane j holds 1/rms of the wave's j-th row. D rows in flight.
template <int D, bool FULL, bool BIAS, bool SR, int T>
__global__ __launch_bounds__(kThreads) void k_rms_quant_colwave(const RowArgs a, uint32_t wps) {
  __shared__ float rcp_tab[128];
  const uint32_t rows = (uint32_t)a.rows, cols = (uint32_t)a.cols;
  const int lane = threadIdx.x & 63;
  const uint32_t wave = wave_id();
  const uint32_t nsc = (cols + kSuper - 1) / kSuper;
  const uint32_t sc = wave % nsc, row0 = wave / nsc;
  const uint32_t nr = (row0 < wps && row0 < rows) ? (rows - 1 - row0) / wps + 1 : 0;
  const uint32_t col = sc * kSuper + lane * 16;
  const bool ok = FULL || col < cols;
  // the prologue's loads first: loads complete in issue order
  const PartialsPre pm = partials_issue(a.ws, a.nparts, a.amax_in);
  const Raw16<T> gq = load_raw16<T>(a.gamma, col, ok);
  Raw16<T> bq = {};
  if constexpr (BIAS) bq = load_raw16<T>(a.beta, col, ok);
  const float r_lane = (uint32_t)lane < nr ? a.rs[row0 + lane * wps] : 0.0f;
  // unconditional fill (a wave without rows reads the last row; past the
  // wave's last row the ring re-reads it): a fill that may be skipped would
  // turn every later wait into a wait for all loads
  uint32_t ldr = nr > 0 ? row0 : rows - 1;
  Raw16<T> ring[D];
#pragma unroll
  for (int d = 0; d < D; ++d) {
    ring[d] = load_blk_t<FULL, T>(row_ptr<T>(a, ldr), col, cols);
    if ((uint32_t)d + 1 < nr) ldr += wps;
  }
  const GScale g = partials_finish(pm, a.ws, a.nparts, a.amax_in, a.amax_out, a.scale_out, rcp_tab);
  float gv[16], bv[16];
  widen_raw16<T>(gq, gv);
#pragma unroll
  for (int k = 0; k < 16; ++k) gv[k] = gv[k] + a.woff;
  widen_raw16<T>(bq, bv);
  uint32_t row = row0;
  for (uint32_t base = 0; base < nr; base += D) {
    if (base + D < nr) {
#pragma unroll
      for (int d = 0; d < D; ++d) {
        const float r = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, r_lane), base + d));
        float v[16];
        widen_raw16<T>(ring[d], v);
        // refill before this item's stores: loads and stores share one
        // in-order counter, so a load issued after a store could not be
        // waited for without also waiting for the store
        ring[d] = load_blk_t<FULL, T>(row_ptr<T>(a, ldr), col, cols);
        if (base + D + d + 1 < nr) ldr += wps;
        __builtin_amdgcn_sched_barrier(0);  // keep the refill ahead of the stores
        quant_item<BIAS, SR, T>(a, v, row, col, ok, r, gv, bv, g, rcp_tab, cols);
        row += wps;
      }
    } else {
#pragma unroll
      for (int d = 0; d < D; ++d) {
        if (base + d < nr) {
          const float r =
              __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, r_lane), base + d));
          float v[16];
          widen_raw16<T>(ring[d], v);
          quant_item<BIAS, SR, T>(a, v, row, col, ok, r, gv, bv, g, rcp_tab, cols);
          row += wps;
        }
      }
    }
  }
}

// Workgroups per streaming launch: rows / 4 up to NVFP4Q_RMS_STREAM_WGS
// (default 1024).
int64_t stream_wgs() {
  static int64_t v = [] {
    const char* e = getenv("NVFP4Q_RMS_STREAM_WGS");
    return e ? (int64_t)atoll(e) : (int64_t)1024;
  }();
  return v;
}

// Workgroups of the row-per-wave encode pass: NVFP4Q_RMS_ENCODE_WGS, default
// the same as the amax pass.
int64_t encode_wgs() {
  static int64_t v = [] {
    const char* e = getenv("NVFP4Q_RMS_ENCODE_WGS");
    return e ? (int64_t)atoll(e) : stream_wgs();
  }();
  return v;
}

bool full_cols(int64_t cols) { return cols % kSuper == 0; }

}  // namespace

template <int T>
static void launch_amax_t(const RowArgs& a, hipStream_t s, uint32_t wgs, size_t lds) {
  if (full_cols(a.cols)) hipLaunchKernelGGL((k_rms_amax_stream<true, T>), dim3(wgs), dim3(kThreads), lds, s, a);
  else hipLaunchKernelGGL((k_rms_amax_stream<false, T>), dim3(wgs), dim3(kThreads), lds, s, a);
}

hipError_t launch_rms_stream_amax(const RowArgs& a, hipStream_t s, uint32_t* nparts) {
  const uint32_t wgs = grid_rows(a.rows, stream_wgs() < kRowPartials ? stream_wgs() : kRowPartials);
  *nparts = wgs;
  const size_t lds = (size_t)param_floats((uint32_t)a.cols) * sizeof(float);
  if (a.dtype == kInFP16) launch_amax_t<kInFP16>(a, s, wgs, lds);
  else if (a.dtype == kInFP32) launch_amax_t<kInFP32>(a, s, wgs, lds);
  else launch_amax_t<kInBF16>(a, s, wgs, lds);
  return hipGetLastError();
}

// Encode-pass choice: with at least NVFP4Q_RMS_ROWWAVE_MIN rows (default
// 2048, i.e. two waves per SIMD) one row per wave with up to 1024 workgroups;
// below that one superchunk column per wave and one row per wave.
int64_t rowwave_min() {
  static int64_t v = [] {
    const char* e = getenv("NVFP4Q_RMS_ROWWAVE_MIN");
    return e ? (int64_t)atoll(e) : (int64_t)2048;
  }();
  return v;
}

template <bool FULL, bool BIAS, int T>
static hipError_t launch_qs(const RowArgs& a, hipStream_t s) {
  if (a.rows >= rowwave_min()) {
    // at most kMaxWaveRows rows per wave: lane k holds the k-th row's 1/rms
    const int64_t min_wgs = (a.rows + kMaxWaveRows * kWavesPerWG - 1) / (kMaxWaveRows * kWavesPerWG);
    const uint32_t wgs = grid_rows(a.rows, encode_wgs() > min_wgs ? encode_wgs() : min_wgs);
    const size_t lds = (size_t)param_floats((uint32_t)a.cols) * sizeof(float) * (BIAS ? 2 : 1);
    if (a.sr) hipLaunchKernelGGL((k_rms_quant_rowwave<FULL, BIAS, true, T>), dim3(wgs), dim3(kThreads), lds, s, a);
    else hipLaunchKernelGGL((k_rms_quant_rowwave<FULL, BIAS, false, T>), dim3(wgs), dim3(kThreads), lds, s, a);
    return hipGetLastError();
  }
  const int64_t nsc = (a.cols + kSuper - 1) / kSuper;
  const int64_t wps = a.rows;  // one row per wave
  const int64_t wgs = (wps * nsc + kWavesPerWG - 1) / kWavesPerWG;
  const dim3 grid((uint32_t)wgs), block(kThreads);
  if (a.sr) hipLaunchKernelGGL((k_rms_quant_colwave<2, FULL, BIAS, true, T>), grid, block, 0, s, a, (uint32_t)wps);
  else hipLaunchKernelGGL((k_rms_quant_colwave<2, FULL, BIAS, false, T>), grid, block, 0, s, a, (uint32_t)wps);
  return hipGetLastError();
}

template <int T>
static hipError_t launch_quant_t(const RowArgs& a, hipStream_t s) {
  const bool full = full_cols(a.cols);
  if (a.beta) return full ? launch_qs<true, true, T>(a, s) : launch_qs<false, true, T>(a, s);
  return full ? launch_qs<true, false, T>(a, s) : launch_qs<false, false, T>(a, s);
}

hipError_t launch_rms_stream_quant(const RowArgs& a, hipStream_t s) {
  if (a.dtype == kInFP16) return launch_quant_t<kInFP16>(a, s);
  if (a.dtype == kInFP32) return launch_quant_t<kInFP32>(a, s);
  return launch_quant_t<kInBF16>(a, s);
}

}  // namespace nvfp4q
