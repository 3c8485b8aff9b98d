// Cooperative-row RMSNorm kernels: the amax pass when a bias is present, the
// encode pass when the amax is given (or when there are more rows than the
// workspace keeps 1/rms for), and the y-only normalization.
//
// The four waves of a workgroup share each token row: wave w takes the
// 1024-column superchunks w, w + 4, ... of the row (lane l: the 16-element
// block at columns 16l..16l+15 of each), forms its partial sum of squares,
// and the four partials meet in LDS behind one barrier per row; every wave
// then has 1/rms and normalizes and encodes its own superchunks. A workgroup
// walks its rows (b, b + G, b + 2G, ...) with D rows in flight, so a wave
// holds one superchunk per row and per slot instead of a whole row, and rows
// complete in the order their loads were issued.
//
// Rows of more than 16 superchunks (16384 < hidden <= 32768, 2-byte input
// types) take eight superchunks per wave and one row in flight, with gamma and
// beta read from global memory where they are used (PG) instead of staged in
// LDS: staged as fp32 they would need up to 256 KiB.
//
// "CuTeDSL at Perplexity", QK Norm (the normalization: r = 1/sqrt(mean x^2 +
// eps), y = RN((gamma + c) x r) [+ beta]) and Prefill and decode (one token
// row per thread group, reductions kept inside the group).
#include <type_traits>

#include "rows.hpp"

namespace nvfp4q {

namespace {

enum CoopMode { kCoopAmax = 0, kCoopEncode = 1, kCoopYOnly = 2 };

// The wave's NPW superchunks of one row (zero past the row's end), elements
// of type T (bf16, fp16 or fp32).
template <int NPW, bool FULL, int T>
__device__ __forceinline__ void coop_load(const RowArgs& a, uint32_t row, uint32_t wid, int lane, uint32_t cols,
                                          Raw16<T> (&q)[NPW]) {
  const char* xr = (const char*)a.x + (int64_t)row * a.ld_x * in_size<T>();
#pragma unroll
  for (int j = 0; j < NPW; ++j) {
    const uint32_t col = (wid + 4 * j) * kSuper + lane * 16;
    q[j] = load_raw16<T>(xr, col, FULL || col < cols);
  }
}

// gamma + c (and beta) of the lane's block at column `col`: from the LDS
// stage, or (PG) read from global memory and widened here, with the same
// fp32 arithmetic as the stage.
template <bool PG, bool BIAS, int T>
__device__ __forceinline__ void block_params(const RowArgs& a, const float* gsh, const float* bsh, uint32_t col,
                                             bool ok, float (&gv)[16], float (&bv)[16]) {
  if constexpr (PG) {
    const Raw16<T> gq = load_raw16<T>(a.gamma, col, ok);
    widen_raw16<T>(gq, gv);
#pragma unroll
    for (int i = 0; i < 16; ++i) gv[i] = gv[i] + a.woff;
    if constexpr (BIAS) {
      const Raw16<T> bq = load_raw16<T>(a.beta, col, ok);
      widen_raw16<T>(bq, bv);
    }
  } else {
    const uint32_t lcol = ok ? col : 0;
    lds16(gsh, lcol, gv);
    if constexpr (BIAS) lds16(bsh, lcol, bv);
  }
}

// One row: partial sums of squares, the barrier, 1/rms, then the mode's work.
// Returns the contribution to the amax pass's maximum (kCoopAmax).
// Y: y is stored (a compile-time choice: encode mode when y is asked for,
// y-only mode always).
template <int NPW, bool FULL, bool BIAS, int MODE, bool SR, int T, bool PG, bool Y>
__device__ __forceinline__ float coop_row(const RowArgs& a, uint32_t row, uint32_t k, const Raw16<T> (&q)[NPW],
                                          float (*ssp)[kWavesPerWG], const float* gsh, const float* bsh, GScale g,
                                          const float* rcp_tab, float inv_k, uint32_t wid, int lane, uint32_t cols) {
  float ss = 0.0f;
#pragma unroll
  for (int j = 0; j < NPW; ++j) {
    if constexpr (T == kInBF16) {
      ss = sumsq8(q[j].q[1], sumsq8(q[j].q[0], ss));
    } else {
      float v[16];
      widen_raw16<T>(q[j], v);
#pragma unroll
      for (int i = 0; i < 16; ++i) ss = __builtin_fmaf(v[i], v[i], ss);
    }
  }
  ss = wave_sum(ss);
  if (lane == 0) ssp[k & 1][wid] = ss;
  // Double-buffered partials: a wave writes row k + 1's partial only after
  // every wave has passed row k's barrier and read row k - 1's buffer.
  __syncthreads();
  const float* sp = ssp[k & 1];
  const float r = inv_rms((sp[0] + sp[1]) + (sp[2] + sp[3]), inv_k, a.eps);
  float mrow = 0.0f;
  if constexpr (MODE == kCoopAmax) {
    if (a.rs != nullptr && wid == 0 && lane == 0) a.rs[row] = r;
  }
  const uint32_t nbr = cols >> 4;
#pragma unroll
  for (int j = 0; j < NPW; ++j) {
    const uint32_t col = (wid + 4 * j) * kSuper + lane * 16;
    const bool ok = FULL || col < cols;
    float v[16], gv[16], bv[16];
    block_params<PG, BIAS, T>(a, gsh, bsh, col, ok, gv, bv);
    widen_raw16<T>(q[j], v);
#pragma unroll
    for (int i = 0; i < 16; ++i) v[i] = v[i] * gv[i];
    if constexpr (MODE == kCoopAmax && !BIAS) {
      // y = RN(RN(x * g) * r) is monotone in |RN(x * g)| for this row's r
      mrow = fmaxf(mrow, max16_abs(v));
      continue;
    }
    if constexpr (BIAS) {
#pragma unroll
      for (int i = 0; i < 16; ++i) v[i] = __builtin_fmaf(v[i], r, bv[i]);
    } else {
#pragma unroll
      for (int i = 0; i < 16; ++i) v[i] = v[i] * r;
    }
    if constexpr (MODE == kCoopAmax) {
      mrow = fmaxf(mrow, max16_abs(v));
    } else {
      // y rounded in the input's type, stored when asked for; the quantizer takes the rounded values
      if constexpr (Y) round_store16<T>(v, (char*)a.y + ((int64_t)row * a.ld_y + col) * in_size<T>(), 0u, ok);
      else round16<T>(v);
      if constexpr (MODE == kCoopEncode) {
        uint32_t sc;
        const uint2 w = encode_block16<SR>(v, g, rcp_tab, sc, (uint64_t)row * nbr + (col >> 4), a.seed, a.offset, 0);
        if (ok) {
          // the row's plane addresses kept scalar, the lane's part a 32-bit offset
          const int64_t coff = uniform_i64((int64_t)row * a.ldc), soff = uniform_i64((int64_t)row * a.lds);
          __builtin_nontemporal_store((uint64_t)w.x | ((uint64_t)w.y << 32),
                                      reinterpret_cast<uint64_t*>(a.codes + coff + (col >> 1)));
          __builtin_nontemporal_store((uint8_t)sc, a.scales + soff + (col >> 4));
        }
      }
    }
  }
  if constexpr (MODE == kCoopAmax) return BIAS ? mrow : mrow * r;
  return 0.0f;
}

template <int NPW, int D, bool FULL, bool BIAS, int MODE, bool SR, int T, bool PG>
__global__ __launch_bounds__(kThreads) void k_rms_coop(const RowArgs a) {
  extern __shared__ float params[];  // gamma + c, then beta (param_floats(cols) each); none with PG
  __shared__ float ssp[2][kWavesPerWG];
  __shared__ float rcp_tab[128];
  const uint32_t rows = (uint32_t)a.rows, cols = (uint32_t)a.cols;
  const int lane = threadIdx.x & 63;
  const uint32_t wid = (uint32_t)__builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const uint32_t G = gridDim.x, b = blockIdx.x;
  const uint32_t nr = b < rows ? (rows - 1 - b) / G + 1 : 0;  // this workgroup's rows
  const uint32_t last = nr > 0 ? b + (nr - 1) * G : rows - 1;
  // the prologue's loads first: loads complete in issue order
  PartialsPre pm;
  if constexpr (MODE == kCoopEncode) pm = partials_issue(a.ws, a.nparts, a.amax_in);
  ParamsPre pp;
  if constexpr (T == kInBF16 && !PG) pp = params_issue<BIAS>((const uint16_t*)a.gamma, (const uint16_t*)a.beta, cols);
  // unconditional fill (row index clamped to the workgroup's last row): a
  // fill that may be skipped would turn every later wait into a wait for all
  Raw16<T> ring[D][NPW];
#pragma unroll
  for (int d = 0; d < D; ++d)
    coop_load<NPW, FULL, T>(a, (uint32_t)d < nr ? b + d * G : last, wid, lane, cols, ring[d]);
  float* gsh = params;
  float* bsh = params + param_floats(cols);
  if constexpr (PG) {
  } else if constexpr (T == kInBF16) {
    params_finish<BIAS>(pp, (const uint16_t*)a.gamma, (const uint16_t*)a.beta, a.woff, cols, gsh, bsh);
  } else {
    stage_params_t<BIAS, T>(a.gamma, a.beta, a.woff, cols, gsh, bsh);
  }
  GScale g = {1.0f, 1.0f};
  if constexpr (MODE == kCoopEncode) g = partials_finish(pm, a.ws, a.nparts, a.amax_in, a.amax_out, a.scale_out, rcp_tab);
  else __syncthreads();
  const float inv_k = 1.0f / (float)cols;
  float mloc = 0.0f;
  // the rows, with y stored or not as a compile-time choice (the encode mode
  // takes y only when asked; the y-only mode always stores it)
  auto rows_loop = [&](auto ytag) {
    constexpr bool Y = decltype(ytag)::value;
    for (uint32_t k = 0; k < nr; k += D) {
      if (k + D < nr) {
        // a slot is refilled (row k + D + d, clamped) as soon as its row is done
#pragma unroll
        for (int d = 0; d < D; ++d) {
          const uint32_t kk = k + d;
          mloc = fmaxf(mloc, coop_row<NPW, FULL, BIAS, MODE, SR, T, PG, Y>(a, b + kk * G, kk, ring[d], ssp, gsh, bsh, g,
                                                                        rcp_tab, inv_k, wid, lane, cols));
          coop_load<NPW, FULL, T>(a, kk + D < nr ? b + (kk + D) * G : last, wid, lane, cols, ring[d]);
        }
      } else {
#pragma unroll
        for (int d = 0; d < D; ++d) {
          const uint32_t kk = k + d;
          if (kk < nr)
            mloc = fmaxf(mloc, coop_row<NPW, FULL, BIAS, MODE, SR, T, PG, Y>(a, b + kk * G, kk, ring[d], ssp, gsh, bsh, g,
                                                                          rcp_tab, inv_k, wid, lane, cols));
        }
      }
    }
  };
  if constexpr (MODE == kCoopYOnly) rows_loop(std::true_type{});
  else if constexpr (MODE == kCoopAmax) rows_loop(std::false_type{});
  else if (a.y != nullptr) rows_loop(std::true_type{});
  else rows_loop(std::false_type{});
  if constexpr (MODE == kCoopAmax) {
    // max |bf16(y)| = bf16(max |y|): round-to-nearest-even is monotone.
    publish_partial(a.ws, round_t<T>(mloc));
  }
}

// One launch for a few rows (grid = rows <= kBarrierSlots): workgroup b
// normalizes row b as in coop_row (the four waves' partial sums of squares
// meet in LDS), keeps y (rounded to T, packed) and each block's max |y| in
// registers, takes the tensor's maximum with grid_max, and encodes. The
// amax pass, its kernel boundary and the encode pass's second read of x are
// gone; the price is one device-scope round trip per workgroup.
template <int NPW, bool FULL, bool BIAS, bool SR, int T>
__global__ __launch_bounds__(kThreads) void k_rms_fused(const RowArgs a, uint32_t spin_limit) {
  constexpr int kW = T == kInFP32 ? 16 : 8;  // words of y per block
  extern __shared__ float params[];  // gamma + c, then beta (param_floats(cols) each)
  __shared__ float ssp[kWavesPerWG];
  __shared__ float rcp_tab[128];
  const uint32_t cols = (uint32_t)a.cols, row = blockIdx.x;
  const int lane = threadIdx.x & 63;
  const uint32_t wid = (uint32_t)__builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  // the call counter: only the first wave publishes, polls and advances it
  uint32_t epoch = 0;
  if (wid == 0) epoch = __hip_atomic_load(&a.ws->status[0], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  ParamsPre pp;
  if constexpr (T == kInBF16) pp = params_issue<BIAS>((const uint16_t*)a.gamma, (const uint16_t*)a.beta, cols);
  Raw16<T> q[NPW];
  coop_load<NPW, FULL, T>(a, row, wid, lane, cols, q);
  float* gsh = params;
  float* bsh = params + param_floats(cols);
  if constexpr (T == kInBF16)
    params_finish<BIAS>(pp, (const uint16_t*)a.gamma, (const uint16_t*)a.beta, a.woff, cols, gsh, bsh);
  else
    stage_params_t<BIAS, T>(a.gamma, a.beta, a.woff, cols, gsh, bsh);
  float ss = 0.0f;
#pragma unroll
  for (int j = 0; j < NPW; ++j) {
    if constexpr (T == kInBF16) {
      ss = sumsq8(q[j].q[1], sumsq8(q[j].q[0], ss));
    } else {
      float v[16];
      widen_raw16<T>(q[j], v);
#pragma unroll
      for (int i = 0; i < 16; ++i) ss = __builtin_fmaf(v[i], v[i], ss);
    }
  }
  ss = wave_sum(ss);
  if (lane == 0) ssp[wid] = ss;
  __syncthreads();  // the partial sums, and gamma (and beta) in LDS
  const float r = inv_rms((ssp[0] + ssp[1]) + (ssp[2] + ssp[3]), 1.0f / (float)cols, a.eps);
  // y in T and each block's max |y| (= RN_T(max |v|): the rounding is monotone and odd)
  uint32_t yw[NPW][kW];
  float bm[NPW];
  float mrow = 0.0f;
#pragma unroll
  for (int j = 0; j < NPW; ++j) {
    const uint32_t col = (wid + 4 * j) * kSuper + lane * 16;
    const bool ok = FULL || col < cols;
    const uint32_t lcol = ok ? col : 0;
    float v[16], gv[16];
    widen_raw16<T>(q[j], v);
    lds16(gsh, lcol, gv);
#pragma unroll
    for (int i = 0; i < 16; ++i) v[i] = v[i] * gv[i];
    if constexpr (BIAS) {
      float bv[16];
      lds16(bsh, lcol, bv);
#pragma unroll
      for (int i = 0; i < 16; ++i) v[i] = __builtin_fmaf(v[i], r, bv[i]);
    } else {
#pragma unroll
      for (int i = 0; i < 16; ++i) v[i] = v[i] * r;
    }
    bm[j] = round_t<T>(max16_abs(v));
    mrow = fmaxf(mrow, bm[j]);
#pragma unroll
    for (int k = 0; k < kW; ++k) {
      if constexpr (T == kInFP32)
        yw[j][k] = __float_as_uint(v[k]);
      else if constexpr (T == kInBF16)
        yw[j][k] = pack_bf16(v[2 * k], v[2 * k + 1]);
      else
        yw[j][k] = (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)v[2 * k]) |
                   ((uint32_t)__builtin_bit_cast(uint16_t, (_Float16)v[2 * k + 1]) << 16);
    }
    if (a.y != nullptr && ok) {
      char* yp = (char*)a.y + ((int64_t)row * a.ld_y + col) * in_size<T>();
#pragma unroll
      for (int l = 0; l < kW / 4; ++l)
        *reinterpret_cast<uint4*>(yp + 16 * l) = make_uint4(yw[j][4 * l], yw[j][4 * l + 1], yw[j][4 * l + 2],
                                                            yw[j][4 * l + 3]);
    }
  }
  const float amax = grid_max(a.ws, epoch, mrow, spin_limit);
  const GScale g = scales_from(amax, a.amax_out, a.scale_out, rcp_tab);
  const uint32_t nbr = cols >> 4;
#pragma unroll
  for (int j = 0; j < NPW; ++j) {
    const uint32_t col = (wid + 4 * j) * kSuper + lane * 16;
    float v[16];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      if constexpr (T == kInFP32) {
        v[2 * k] = __uint_as_float(yw[j][2 * k]);
        v[2 * k + 1] = __uint_as_float(yw[j][2 * k + 1]);
      } else {
        v[2 * k] = T == kInBF16 ? bf_lo(yw[j][k]) : h_lo(yw[j][k]);
        v[2 * k + 1] = T == kInBF16 ? bf_hi(yw[j][k]) : h_hi(yw[j][k]);
      }
    }
    const uint32_t sc = block_scale(bm[j], g.enc);
    const uint2 w = encode_with_scale<SR>(v, sc, rcp_tab, (uint64_t)row * nbr + (col >> 4), a.seed, a.offset, 0);
    if (FULL || col < cols) {
      __builtin_nontemporal_store((uint64_t)w.x | ((uint64_t)w.y << 32),
                                  reinterpret_cast<uint64_t*>(a.codes + (int64_t)row * a.ldc + (col >> 1)));
      __builtin_nontemporal_store((uint8_t)sc, a.scales + (int64_t)row * a.lds + (col >> 4));
    }
  }
}

// Bounded waits of the one-launch kernel: 2^20 polls (each a device-scope load
// and a 64-cycle sleep, about a second in all), far past any wait the launch's
// resident workgroups can need.
constexpr uint32_t kFusedSpinLimit = 1u << 20;

template <int NPW, bool BIAS, bool SR, int T>
hipError_t launch_fused_t(const RowArgs& a, hipStream_t s) {
  const size_t lds = (size_t)param_floats((uint32_t)a.cols) * sizeof(float) * (BIAS ? 2 : 1);
  const dim3 grid((uint32_t)a.rows), block(kThreads);
  if (a.cols == (int64_t)NPW * 4 * kSuper)
    hipLaunchKernelGGL((k_rms_fused<NPW, true, BIAS, SR, T>), grid, block, lds, s, a, kFusedSpinLimit);
  else
    hipLaunchKernelGGL((k_rms_fused<NPW, false, BIAS, SR, T>), grid, block, lds, s, a, kFusedSpinLimit);
  return hipGetLastError();
}

template <int NPW, int T>
hipError_t launch_fused_npw_t(const RowArgs& a, hipStream_t s) {
  if (a.beta) return a.sr ? launch_fused_t<NPW, true, true, T>(a, s) : launch_fused_t<NPW, true, false, T>(a, s);
  return a.sr ? launch_fused_t<NPW, false, true, T>(a, s) : launch_fused_t<NPW, false, false, T>(a, s);
}

template <int NPW>
hipError_t launch_fused_npw(const RowArgs& a, hipStream_t s) {
  if (a.dtype == kInFP16) return launch_fused_npw_t<NPW, kInFP16>(a, s);
  if (a.dtype == kInFP32) return launch_fused_npw_t<NPW, kInFP32>(a, s);
  return launch_fused_npw_t<NPW, kInBF16>(a, s);
}

// Workgroups per launch: min(rows, NVFP4Q_RMS_COOP_WGS), default 1024.
int64_t coop_wgs() {
  static int64_t v = [] {
    const char* e = getenv("NVFP4Q_RMS_COOP_WGS");
    return e ? (int64_t)atoll(e) : (int64_t)1024;
  }();
  return v;
}

// Two rows in flight per workgroup: three or four measured slower on the
// 4096 x 4096 prefill (10.7 us at two, 11.3-11.5 us at three or four).
constexpr int kCoopDepth = 2;

// Up to 16 superchunks per row: gamma and beta staged in LDS, two rows in
// flight; more (NPW 8): read where used (PG), one row in flight.
template <int NPW, bool BIAS, int MODE, bool SR, int T>
hipError_t launch_coop_t(const RowArgs& a, uint32_t wgs, hipStream_t s) {
  constexpr bool kPG = NPW > 4;
  constexpr int kD = kPG ? 1 : kCoopDepth;
  const size_t lds = kPG ? 0 : (size_t)param_floats((uint32_t)a.cols) * sizeof(float) * (BIAS ? 2 : 1);
  if (a.cols == (int64_t)NPW * 4 * kSuper)
    hipLaunchKernelGGL((k_rms_coop<NPW, kD, true, BIAS, MODE, SR, T, kPG>), dim3(wgs), dim3(kThreads), lds, s, a);
  else
    hipLaunchKernelGGL((k_rms_coop<NPW, kD, false, BIAS, MODE, SR, T, kPG>), dim3(wgs), dim3(kThreads), lds, s, a);
  return hipGetLastError();
}

template <int NPW, bool BIAS, int T>
hipError_t launch_coop_mode(const RowArgs& a, int mode, uint32_t wgs, hipStream_t s) {
  if (mode == kCoopAmax) return launch_coop_t<NPW, BIAS, kCoopAmax, false, T>(a, wgs, s);
  if (mode == kCoopYOnly) return launch_coop_t<NPW, BIAS, kCoopYOnly, false, T>(a, wgs, s);
  if (a.sr) return launch_coop_t<NPW, BIAS, kCoopEncode, true, T>(a, wgs, s);
  return launch_coop_t<NPW, BIAS, kCoopEncode, false, T>(a, wgs, s);
}

template <int NPW, int T>
hipError_t launch_coop_npw_t(const RowArgs& a, int mode, uint32_t wgs, hipStream_t s) {
  return a.beta ? launch_coop_mode<NPW, true, T>(a, mode, wgs, s) : launch_coop_mode<NPW, false, T>(a, mode, wgs, s);
}

template <int NPW>
hipError_t launch_coop_npw(const RowArgs& a, int mode, uint32_t wgs, hipStream_t s) {
  if (a.dtype == kInFP16) return launch_coop_npw_t<NPW, kInFP16>(a, mode, wgs, s);
  if constexpr (NPW <= 4) {
    if (a.dtype == kInFP32) return launch_coop_npw_t<NPW, kInFP32>(a, mode, wgs, s);
  } else {
    if (a.dtype == kInFP32) return hipErrorInvalidValue;  // rows of 4-byte values stop at 16 superchunks
  }
  return launch_coop_npw_t<NPW, kInBF16>(a, mode, wgs, s);
}

}  // namespace

int rms_max_cols(int dtype) { return (dtype == kInFP32 ? 16 : 32) * kSuper; }
int rms_stage_max_cols() { return 16 * kSuper; }

int rms_fused_max_rows() { return kBarrierSlots; }

hipError_t launch_rms_fused(const RowArgs& a, hipStream_t s) {
  if (a.rows < 1 || a.rows > kBarrierSlots || a.codes == nullptr) return hipErrorInvalidValue;
  const int64_t nsc = (a.cols + kSuper - 1) / kSuper;
  if (nsc <= 4) return launch_fused_npw<1>(a, s);
  if (nsc <= 8) return launch_fused_npw<2>(a, s);
  if (nsc <= 16) return launch_fused_npw<4>(a, s);
  return hipErrorInvalidValue;
}

hipError_t launch_rmsnorm_pass(const RowArgs& a, bool amax_pass, hipStream_t s, uint32_t* nparts) {
  int64_t wgs = a.rows < coop_wgs() ? a.rows : coop_wgs();
  if (amax_pass && wgs > kRowPartials) wgs = kRowPartials;
  if (wgs < 1) wgs = 1;
  if (amax_pass) *nparts = (uint32_t)wgs;
  const int mode = amax_pass ? kCoopAmax : (a.codes != nullptr ? kCoopEncode : kCoopYOnly);
  const int64_t nsc = (a.cols + kSuper - 1) / kSuper;
  if (nsc <= 4) return launch_coop_npw<1>(a, mode, (uint32_t)wgs, s);
  if (nsc <= 8) return launch_coop_npw<2>(a, mode, (uint32_t)wgs, s);
  if (nsc <= 16) return launch_coop_npw<4>(a, mode, (uint32_t)wgs, s);
  if (nsc <= 32) return launch_coop_npw<8>(a, mode, (uint32_t)wgs, s);
  return hipErrorInvalidValue;
}

}  // namespace nvfp4q
