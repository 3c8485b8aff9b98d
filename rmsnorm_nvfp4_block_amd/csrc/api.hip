// C ABI of the library: argument validation and dispatch to the gfx950 kernels.
// Every check happens on the host before anything is enqueued; the only error
// reported after enqueueing is NVFP4Q_E_LAUNCH.
#include "../../include/nvfp4q.h"

#include "device.hpp"
#include "launch.hpp"

#include <cstddef>
#include <cstdlib>
#include <cstring>
#include <mutex>

using namespace nvfp4q;

namespace {

inline bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

// Largest leading dimension accepted (elements or bytes): far beyond any
// device allocation, and small enough that row * ld never overflows int64.
constexpr int64_t kMaxLd = int64_t(1) << 40;

nvfp4q_status check_ws(void* ws, size_t bytes) {
  if (!ws || bytes < sizeof(Workspace) || !aligned(ws, 256)) return NVFP4Q_E_WORKSPACE;
  return NVFP4Q_OK;
}

// Bytes per element of a dtype (0: not a dtype).
int dtype_size(nvfp4q_dtype dt) {
  return dt == NVFP4Q_BF16 || dt == NVFP4Q_FP16 ? 2 : dt == NVFP4Q_FP32 ? 4 : 0;
}

// x: bf16 unless any_dtype (then bf16, fp16 or fp32); rows 16-byte aligned.
nvfp4q_status check_input(const void* x, nvfp4q_dtype dt, int64_t rows, int64_t cols, int64_t ld,
                          bool any_dtype = false) {
  if (any_dtype ? dtype_size(dt) == 0 : dt != NVFP4Q_BF16) return NVFP4Q_E_UNSUPPORTED;
  if (rows < 0 || cols <= 0 || cols % 16 != 0 || ld < cols || ld > kMaxLd) return NVFP4Q_E_SHAPE;
  if (rows > 0x7FFFFFFF || cols > 0x7FFFFFFF) return NVFP4Q_E_SHAPE;
  if (rows > 0 && !x) return NVFP4Q_E_NULLPTR;
  if (!aligned(x, 16) || (ld * dtype_size(dt)) % 16 != 0) return NVFP4Q_E_ALIGN;
  return NVFP4Q_OK;
}

// A plane of `prows` plane rows holding `pcols` elements each (an empty plane,
// no rows or rows of no elements, may have NULL pointers).
nvfp4q_status check_plane(const nvfp4q_plane* p, int64_t prows, int64_t pcols) {
  if (prows == 0 || pcols == 0) return NVFP4Q_OK;  // nothing is written
  if (!p->codes || !p->scales) return NVFP4Q_E_NULLPTR;
  if (p->ld_codes < pcols / 2 || p->ld_scales < pcols / 16) return NVFP4Q_E_SHAPE;
  if (p->ld_codes > kMaxLd || p->ld_scales > kMaxLd) return NVFP4Q_E_SHAPE;
  if (!aligned(p->codes, 16) || p->ld_codes % 8 != 0) return NVFP4Q_E_ALIGN;
  return NVFP4Q_OK;
}

// The rounding mode without option bits.
nvfp4q_rounding base_rounding(nvfp4q_rounding r) { return (nvfp4q_rounding)((int)r & ~NVFP4Q_FAST_MATH); }
bool fast_math(nvfp4q_rounding r) { return ((int)r & NVFP4Q_FAST_MATH) != 0; }

nvfp4q_status check_rounding(nvfp4q_rounding r, const nvfp4q_rng* rng) {
  const nvfp4q_rounding b = base_rounding(r);
  if (b != NVFP4Q_RTNE && b != NVFP4Q_SR) return NVFP4Q_E_UNSUPPORTED;
  if (b == NVFP4Q_SR && !rng) return NVFP4Q_E_NULLPTR;
  return NVFP4Q_OK;
}

nvfp4q_status done(hipError_t e) { return e == hipSuccess ? NVFP4Q_OK : NVFP4Q_E_LAUNCH; }

#define TRY(expr)                             \
  do {                                        \
    nvfp4q_status st_ = (expr);               \
    if (st_ != NVFP4Q_OK) return st_;         \
  } while (0)

const nvfp4q_global kNoGlobal = {nullptr, nullptr, nullptr};

// NVFP4Q_RMS_STREAM=0 selects the cooperative-row RMSNorm encode pass everywhere
// (for comparison; both give identical results).
bool rms_stream_enabled() {
  static const bool on = [] {
    const char* e = getenv("NVFP4Q_RMS_STREAM");
    return !(e && e[0] == '0');
  }();
  return on;
}


// The no-allocation entry point's workspace: a file-scope device array, one
// per GPU (each device that loads the library holds its own copy until the
// process ends). Host code never passes the array's name to a kernel (on the
// host it only stands for the symbol); its device address is looked up once
// per device with hipGetSymbolAddress, with that device current, and kept.
constexpr size_t kScratchBytes = sizeof(Workspace);  // 1 MiB: what every rmsnorm_nvfp4q call needs
__device__ __align__(256) uint8_t scratch[kScratchBytes];
static_assert(kScratchBytes >= sizeof(Workspace), "the static workspace holds one workspace");

constexpr int kMaxDevices = 64;
std::mutex scratch_mu;
void* scratch_ptr[kMaxDevices];

// The current device's copy of `scratch`; NVFP4Q_E_LAUNCH if the device or the
// lookup fails, NVFP4Q_E_UNSUPPORTED for device ordinals past kMaxDevices.
nvfp4q_status static_scratch(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return NVFP4Q_E_LAUNCH;
  if (dev >= kMaxDevices) return NVFP4Q_E_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(scratch_mu);
  if (!scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return NVFP4Q_E_LAUNCH;
    scratch_ptr[dev] = p;
  }
  *out = scratch_ptr[dev];
  return NVFP4Q_OK;
}

// rmsnorm_nvfp4q on the caller's workspace, or (use_static) on the static
// one; either is checked or looked up after the other arguments pass.
nvfp4q_status rmsnorm_impl(const void* x, nvfp4q_dtype dtype, int64_t tokens, int64_t hidden, int64_t ld_x,
                           const void* gamma, const void* beta, float weight_offset, float eps, void* y_out,
                           int64_t ld_y, const nvfp4q_global* g, const nvfp4q_plane* row, nvfp4q_rounding rounding,
                           const nvfp4q_rng* rng, void* workspace, size_t workspace_bytes, bool use_static,
                           void* stream) {
  TRY(check_input(x, dtype, tokens, hidden, ld_x, true));
  const bool one_launch = ((int)rounding & NVFP4Q_ONE_LAUNCH) != 0;
  rounding = (nvfp4q_rounding)((int)rounding & ~NVFP4Q_ONE_LAUNCH);
  if (!gamma) return NVFP4Q_E_NULLPTR;
  if (!aligned(gamma, 16) || !aligned(beta, 16)) return NVFP4Q_E_ALIGN;
  if (weight_offset != 0.0f && weight_offset != 1.0f) return NVFP4Q_E_UNSUPPORTED;
  if (!(eps >= 0.0f)) return NVFP4Q_E_SHAPE;
  if (hidden > rms_max_cols((int)dtype)) return NVFP4Q_E_UNSUPPORTED;
  const bool codes = row && (row->codes || tokens == 0);
  if (!codes && !y_out) return NVFP4Q_E_NULLPTR;
  if (codes) TRY(check_plane(row, tokens, hidden));
  if (y_out) {
    if (ld_y < hidden || ld_y > kMaxLd) return NVFP4Q_E_SHAPE;
    if (!aligned(y_out, 16) || (ld_y * dtype_size(dtype)) % 16 != 0) return NVFP4Q_E_ALIGN;
  }
  TRY(check_rounding(rounding, rng));
  if (use_static) TRY(static_scratch(&workspace));
  else TRY(check_ws(workspace, workspace_bytes));
  const nvfp4q_global& gg = g ? *g : kNoGlobal;
  hipStream_t s = (hipStream_t)stream;
  if (tokens == 0) return codes ? done(launch_empty_scale(gg.amax_out, gg.scale_out, 1, s)) : NVFP4Q_OK;
  RowArgs a = {};
  a.x = x; a.dtype = (int)dtype; a.rows = tokens; a.cols = hidden; a.ld_x = ld_x;
  a.gamma = gamma; a.beta = beta; a.woff = weight_offset; a.eps = eps;
  a.y = y_out; a.ld_y = ld_y;
  a.codes = codes ? row->codes : nullptr; a.ldc = codes ? row->ld_codes : 0;
  a.scales = codes ? row->scales : nullptr; a.lds = codes ? row->ld_scales : 0;
  a.ws = (Workspace*)workspace;
  a.amax_in = gg.amax_in; a.amax_out = gg.amax_out; a.scale_out = gg.scale_out;
  a.sr = base_rounding(rounding) == NVFP4Q_SR;
  a.seed = rng ? rng->seed : 0; a.offset = rng ? rng->offset : 0;
  // NVFP4Q_ONE_LAUNCH, a few rows and no given amax: one launch whose
  // workgroups meet on the amax inside it.
  const bool staged = hidden <= rms_stage_max_cols();  // gamma and beta fit the LDS stage
  if (one_launch && codes && !a.amax_in && tokens <= rms_fused_max_rows() && staged)
    return done(launch_rms_fused(a, s));
  // With the amax pass and a row count that fits the workspace's row-scale
  // slots, the encode pass streams rows using the 1/rms the amax pass stored.
  const bool streamed = codes && !a.amax_in && tokens <= kRowScaleCap && staged && rms_stream_enabled();
  if (streamed) a.rs = reinterpret_cast<float*>(static_cast<char*>(workspace) + offsetof(Workspace, partial)) + kRowPartials;
  if (codes && !a.amax_in) {
    const hipError_t e = (streamed && !beta) ? launch_rms_stream_amax(a, s, &a.nparts)
                                           : launch_rmsnorm_pass(a, true, s, &a.nparts);
    if (e != hipSuccess) return NVFP4Q_E_LAUNCH;
  }
  return done(streamed ? launch_rms_stream_quant(a, s) : launch_rmsnorm_pass(a, false, s, nullptr));
}

}  // namespace

namespace nvfp4q {
static bool xcd_order() {
  static const bool on = [] {
    const char* e = getenv("NVFP4Q_XCD_ORDER");
    return !(e && e[0] == '0');
  }();
  return on;
}
uint32_t xcd_chunk(uint64_t items) { return xcd_order() ? (uint32_t)((items + kXcds - 1) / kXcds) : 0u; }
uint32_t xcd_grid(uint64_t items) { return xcd_order() ? kXcds * xcd_chunk(items) : (uint32_t)items; }
}  // namespace nvfp4q

extern "C" {

size_t nvfp4q_workspace_bytes(void) { return sizeof(Workspace); }

int nvfp4q_version(void) { return 1; }

// The build passes the sha256 of the sources (every file of csrc/ and
// include/); a library built any other way says so.
#ifndef NVFP4Q_SOURCE_SHA256
#define NVFP4Q_SOURCE_SHA256 "unknown"
#endif
const char* nvfp4q_source_sha256(void) { return NVFP4Q_SOURCE_SHA256; }

const char* nvfp4q_status_string(nvfp4q_status s) {
  int v;  // read as an int: a caller may pass any code
  std::memcpy(&v, &s, sizeof v);
  switch (v) {
    case NVFP4Q_OK: return "ok";
    case NVFP4Q_E_NULLPTR: return "a required pointer is NULL";
    case NVFP4Q_E_SHAPE: return "a size or leading dimension breaks the shape rules";
    case NVFP4Q_E_ALIGN: return "a pointer or leading dimension breaks the alignment rules";
    case NVFP4Q_E_UNSUPPORTED: return "dtype, rounding mode or option not supported";
    case NVFP4Q_E_LAUNCH: return "a kernel launch failed";
    case NVFP4Q_E_WORKSPACE: return "workspace missing, misaligned or too small";
  }
  return "unknown status";
}

nvfp4q_status nvfp4q_quantize(const void* x, nvfp4q_dtype dtype, int64_t rows, int64_t cols, int64_t ld_x,
                              const nvfp4q_global* g, const nvfp4q_plane* row, nvfp4q_rounding rounding,
                              const nvfp4q_rng* rng, void* workspace, size_t workspace_bytes, void* stream) {
  TRY(check_input(x, dtype, rows, cols, ld_x, true));
  if (!row) return NVFP4Q_E_NULLPTR;
  TRY(check_plane(row, rows, cols));
  TRY(check_rounding(rounding, rng));
  TRY(check_ws(workspace, workspace_bytes));
  const nvfp4q_global& gg = g ? *g : kNoGlobal;
  hipStream_t s = (hipStream_t)stream;
  if (rows == 0) return done(launch_empty_scale(gg.amax_out, gg.scale_out, 1, s));
  RowArgs a = {};
  a.x = x; a.dtype = (int)dtype; a.rows = rows; a.cols = cols; a.ld_x = ld_x;
  a.codes = row->codes; a.ldc = row->ld_codes; a.scales = row->scales; a.lds = row->ld_scales;
  a.ws = (Workspace*)workspace;
  a.amax_in = gg.amax_in; a.amax_out = gg.amax_out; a.scale_out = gg.scale_out;
  a.sr = base_rounding(rounding) == NVFP4Q_SR;
  a.seed = rng ? rng->seed : 0; a.offset = rng ? rng->offset : 0;
  if (!a.amax_in) {
    hipError_t e = launch_amax_rows(a, s, &a.nparts);
    if (e != hipSuccess) return NVFP4Q_E_LAUNCH;
  }
  return done(launch_quant_rows(a, s));
}

nvfp4q_status rmsnorm_nvfp4q(const void* x, nvfp4q_dtype dtype, int64_t tokens, int64_t hidden, int64_t ld_x,
                             const void* gamma, const void* beta, float weight_offset, float eps, void* y_out,
                             int64_t ld_y, const nvfp4q_global* g, const nvfp4q_plane* row,
                             nvfp4q_rounding rounding, const nvfp4q_rng* rng, void* workspace,
                             size_t workspace_bytes, void* stream) {
  return rmsnorm_impl(x, dtype, tokens, hidden, ld_x, gamma, beta, weight_offset, eps, y_out, ld_y, g, row,
                      rounding, rng, workspace, workspace_bytes, false, stream);
}

nvfp4q_status rmsnorm_nvfp4q_noalloc(const void* x, nvfp4q_dtype dtype, int64_t tokens, int64_t hidden,
                                     int64_t ld_x, const void* gamma, const void* beta, float weight_offset,
                                     float eps, void* y_out, int64_t ld_y, const nvfp4q_global* g,
                                     const nvfp4q_plane* row, nvfp4q_rounding rounding, const nvfp4q_rng* rng,
                                     void* stream) {
  return rmsnorm_impl(x, dtype, tokens, hidden, ld_x, gamma, beta, weight_offset, eps, y_out, ld_y, g, row,
                      rounding, rng, nullptr, 0, true, stream);
}

}  // extern "C"

namespace {

// nvfp4q_quantize_2d over `experts` stacked weights of `rows` rows each.
nvfp4q_status quantize_2d_impl(const void* x, nvfp4q_dtype dtype, int experts, int64_t rows, int64_t cols,
                               int64_t ld_x, const nvfp4q_global* g, const nvfp4q_plane* row,
                               const nvfp4q_plane* col, nvfp4q_rounding rounding, const nvfp4q_rng* rng,
                               void* workspace, size_t workspace_bytes, void* stream) {
  if (rows < 0) return NVFP4Q_E_SHAPE;
  TRY(check_input(x, dtype, experts * rows, cols, ld_x, true));
  // planes of an empty input hold no bytes and may come with NULL pointers
  const bool has_row = row && (row->codes || rows == 0), has_col = col && (col->codes || rows == 0);
  if (!has_row && !has_col) return NVFP4Q_E_NULLPTR;
  const bool tile16 = ((int)rounding & NVFP4Q_SCALE_16X16) != 0;
  rounding = (nvfp4q_rounding)((int)rounding & ~NVFP4Q_SCALE_16X16);
  if (has_row) TRY(check_plane(row, experts * rows, cols));
  if ((has_col || tile16) && rows % 16 != 0) return NVFP4Q_E_SHAPE;
  if (has_col) {
    if (experts * cols > 0x7FFFFFFF) return NVFP4Q_E_SHAPE;
    TRY(check_plane(col, experts * cols, rows));
  }
  TRY(check_rounding(rounding, rng));
  TRY(check_ws(workspace, workspace_bytes));
  const nvfp4q_global& gg = g ? *g : kNoGlobal;
  hipStream_t s = (hipStream_t)stream;
  if (rows == 0) return done(launch_empty_scale(gg.amax_out, gg.scale_out, experts, s));
  uint32_t nparts = 0;
  if (!gg.amax_in) {
    RowArgs r = {};
    r.x = x; r.dtype = (int)dtype; r.rows = rows; r.cols = cols; r.ld_x = ld_x;
    r.ws = (Workspace*)workspace;
    hipError_t e = launch_amax_rows(r, s, &nparts, experts);
    if (e != hipSuccess) return NVFP4Q_E_LAUNCH;
  }
  TwoDArgs a = {};
  a.nparts = nparts;
  a.x = x; a.rows = rows; a.cols = cols; a.ld_x = ld_x;
  a.experts = experts;
  a.dtype = (int)dtype;
  if (has_row) { a.rcodes = row->codes; a.rldc = row->ld_codes; a.rscales = row->scales; a.rlds = row->ld_scales; }
  if (has_col) { a.ccodes = col->codes; a.cldc = col->ld_codes; a.cscales = col->scales; a.clds = col->ld_scales; }
  a.tile16 = tile16;
  a.ws = (Workspace*)workspace;
  a.amax_in = gg.amax_in; a.amax_out = gg.amax_out; a.scale_out = gg.scale_out;
  a.sr = base_rounding(rounding) == NVFP4Q_SR;
  a.seed = rng ? rng->seed : 0; a.offset = rng ? rng->offset : 0;
  return done(launch_quant_2d(a, s));
}

}  // namespace

extern "C" {

nvfp4q_status nvfp4q_quantize_2d(const void* x, nvfp4q_dtype dtype, int64_t rows, int64_t cols, int64_t ld_x,
                                 const nvfp4q_global* g, const nvfp4q_plane* row, const nvfp4q_plane* col,
                                 nvfp4q_rounding rounding, const nvfp4q_rng* rng, void* workspace,
                                 size_t workspace_bytes, void* stream) {
  return quantize_2d_impl(x, dtype, 1, rows, cols, ld_x, g, row, col, rounding, rng, workspace, workspace_bytes,
                          stream);
}

nvfp4q_status nvfp4q_quantize_2d_grouped(const void* x, nvfp4q_dtype dtype, int32_t experts, int64_t rows,
                                         int64_t cols, int64_t ld_x, const nvfp4q_global* g,
                                         const nvfp4q_plane* row, const nvfp4q_plane* col,
                                         nvfp4q_rounding rounding, const nvfp4q_rng* rng, void* workspace,
                                         size_t workspace_bytes, void* stream) {
  if (experts < 1 || experts > 64) return NVFP4Q_E_SHAPE;
  return quantize_2d_impl(x, dtype, experts, rows, cols, ld_x, g, row, col, rounding, rng, workspace,
                          workspace_bytes, stream);
}

nvfp4q_status nvfp4q_qk_norm(void* q, void* k, nvfp4q_dtype dtype, int64_t tokens, int32_t q_heads,
                             int32_t k_heads, int32_t head_dim, int64_t ld_q, int64_t ld_k, const void* q_weight,
                             const void* k_weight, float weight_offset, float eps, void* stream) {
  if (dtype_size(dtype) == 0) return NVFP4Q_E_UNSUPPORTED;
  if (head_dim != 64 && head_dim != 128 && head_dim != 256) return NVFP4Q_E_UNSUPPORTED;
  if (tokens < 0 || q_heads < 0 || k_heads < 0 || q_heads + k_heads < 1) return NVFP4Q_E_SHAPE;
  if (tokens > 0x7FFFFFFF || (int64_t)q_heads + k_heads > 65536) return NVFP4Q_E_SHAPE;
  if (q_heads > 0 && ld_q < (int64_t)q_heads * head_dim) return NVFP4Q_E_SHAPE;
  if (k_heads > 0 && ld_k < (int64_t)k_heads * head_dim) return NVFP4Q_E_SHAPE;
  if (ld_q > kMaxLd || ld_k > kMaxLd) return NVFP4Q_E_SHAPE;
  if (weight_offset != 0.0f && weight_offset != 1.0f) return NVFP4Q_E_UNSUPPORTED;
  if (!(eps >= 0.0f)) return NVFP4Q_E_SHAPE;
  if (tokens > 0 && q_heads > 0 && (!q || !q_weight)) return NVFP4Q_E_NULLPTR;
  if (tokens > 0 && k_heads > 0 && (!k || !k_weight)) return NVFP4Q_E_NULLPTR;
  const int es = dtype_size(dtype);
  if (q_heads > 0 && (!aligned(q, 16) || !aligned(q_weight, 16) || (ld_q * es) % 16 != 0)) return NVFP4Q_E_ALIGN;
  if (k_heads > 0 && (!aligned(k, 16) || !aligned(k_weight, 16) || (ld_k * es) % 16 != 0)) return NVFP4Q_E_ALIGN;
  QkArgs a = {};
  a.q = q; a.k = k; a.wq = q_weight; a.wk = k_weight;
  a.tokens = tokens; a.ldq = ld_q; a.ldk = ld_k;
  a.hq = q_heads; a.hk = k_heads; a.d = head_dim;
  a.woff = weight_offset; a.eps = eps;
  a.dtype = (int)dtype;
  return done(launch_qk_norm(a, (hipStream_t)stream));
}

nvfp4q_status nvfp4q_grouped(const void* x, nvfp4q_dtype dtype, int64_t total_rows, int64_t cols, int64_t ld_x,
                             const int32_t* offsets, int32_t num_groups, int32_t* padded_offsets_out,
                             int apply_rht, uint32_t rht_sign_mask, const nvfp4q_global* g,
                             const nvfp4q_plane* col, const nvfp4q_global* g_row, const nvfp4q_plane* row,
                             nvfp4q_rounding rounding, const nvfp4q_rng* rng, void* workspace,
                             size_t workspace_bytes, void* stream) {
  TRY(check_input(x, dtype, total_rows, cols, ld_x, true));
  // an empty rowwise plane (no rows) may come with NULL pointers
  const bool want_col = col && col->codes, want_row = row && (row->codes || total_rows == 0);
  if (!offsets || (!want_col && !want_row)) return NVFP4Q_E_NULLPTR;
  if (num_groups < 1 || num_groups > 64) return NVFP4Q_E_SHAPE;
  if (apply_rht != 0 && apply_rht != 1) return NVFP4Q_E_UNSUPPORTED;
  if (rht_sign_mask > 0xFFFFu) return NVFP4Q_E_UNSUPPORTED;
  if (ld_x * dtype_size(dtype) > 2 * kGroupedMaxLd) return NVFP4Q_E_SHAPE;
  const int64_t cap = total_rows + 15 * (int64_t)num_groups;
  if (want_col) {
    TRY(check_plane(col, cols, cap));  // codes and scales present (cap >= 15 > 0), alignment
    if (col->ld_codes * 2 < cap || col->ld_scales * 16 < cap) return NVFP4Q_E_SHAPE;
  }
  if (want_row) TRY(check_plane(row, total_rows, cols));
  TRY(check_rounding(rounding, rng));
  TRY(check_ws(workspace, workspace_bytes));
  const nvfp4q_global& gg = g ? *g : kNoGlobal;
  const nvfp4q_global& gr = g_row ? *g_row : kNoGlobal;
  GroupArgs a = {};
  a.x = x; a.dtype = (int)dtype; a.rows = total_rows; a.cols = cols; a.ld_x = ld_x;
  a.offsets = offsets; a.groups = num_groups; a.poff_out = padded_offsets_out;
  a.rht = apply_rht != 0; a.mask = rht_sign_mask;
  a.col = want_col;
  if (want_col) { a.codes = col->codes; a.ldc = col->ld_codes; a.scales = col->scales; a.lds = col->ld_scales; }
  a.amax_in = gg.amax_in; a.amax_out = gg.amax_out; a.scale_out = gg.scale_out;
  a.row = want_row;
  if (want_row) { a.rcodes = row->codes; a.rldc = row->ld_codes; a.rscales = row->scales; a.rlds = row->ld_scales; }
  a.ramax_in = gr.amax_in; a.ramax_out = gr.amax_out; a.rscale_out = gr.scale_out;
  a.ws = (Workspace*)workspace;
  a.sr = base_rounding(rounding) == NVFP4Q_SR;
  a.fast = fast_math(rounding);
  a.seed = rng ? rng->seed : 0; a.offset = rng ? rng->offset : 0;
  return done(launch_grouped(a, (hipStream_t)stream));
}

}  // extern "C"
