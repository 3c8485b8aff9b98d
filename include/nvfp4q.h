/*
 * nvfp4q.h -- C ABI of an MI355X (gfx950) library for per-token RMSNorm and
 * NVFP4 block quantization.
 *
 * Sources (cited by page title and section):
 *   [PR]   "[nvfp4_training] Optimize CuteDSL kernels for NVFP4 training"
 *          (pytorch/ao pull request 4798): Optimization items 1-7, Fast math,
 *          Grouped allocation tail, Config surface and AUTO, Correctness.
 *   [Blog] "CuTeDSL at Perplexity": QK Norm, Blackwell support, prefill and
 *          decode specialization, grid synchronization.
 *
 * What is computed (NVFP4):
 *   amax  = max |x| over the tensor, or over one group in grouped mode;
 *   S_enc = 2688 / amax, S_dec = amax / 2688 (2688 = 6 * 448; both 1 when
 *           amax is 0 or S_enc would not be finite);
 *   per block of 16 elements (16 consecutive elements of a row, or 16
 *   consecutive rows of one column for the columnwise plane):
 *     scale = E4M3 round-to-nearest-even, saturating, of (bmax / 6) * S_enc,
 *     each element x -> E2M1 code of x * (1 / (f32(scale) * S_dec)),
 *     rounded to nearest even (RTNE) or stochastically (SR); codes are packed
 *     two per byte with the even element in the low nibble.
 *   [Blog, Blackwell support] (16-element amax), [PR, Optimization 1 and 3]
 *   (encode multiply and saturating conversion), [PR, Fast math] (the encode
 *   reciprocal is 1 / (decoded block scale * global decode scale), computed
 *   exactly; this library has only the exact path).
 *
 * Stochastic rounding [PR, Optimization 3; Correctness]: one Philox4x32-10
 * evaluation per 16-element block, key = (seed lo32, seed hi32), counter =
 * (block index lo32, block index hi32, tag, offset); tag 0 for a rowwise plane
 * and 1 for a columnwise plane; the block index is the position of the block's
 * scale byte in a packed scale plane. Element j of a block uses byte (j & 3) of
 * output word (j >> 2) and rounds up iff byte + floor(256 * frac) >= 256, frac
 * being its position between the two neighbouring E2M1 magnitudes. Scales are
 * always round-to-nearest-even. Output is a pure function of (inputs, seed,
 * offset), independent of launch geometry.
 *
 * Conventions for every entry point:
 *   - Pointers marked "device" are caller-owned device memory on the current
 *     HIP device; struct pointers (nvfp4q_plane*, ...) are host memory read
 *     only during the call. The library never allocates, frees or
 *     synchronizes; all work is enqueued on `stream` (a hipStream_t; NULL is
 *     the default stream), so calls may be captured in a HIP graph.
 *   - `workspace` is device scratch memory of at least nvfp4q_workspace_bytes()
 *     bytes (1 MiB), 256-byte aligned, owned by the caller. Its first 640
 *     bytes hold the state of NVFP4Q_ONE_LAUNCH calls: before the first such
 *     call they must hold zeros (any one 32-bit value repeated also works),
 *     and from then on only the library writes them. The rest needs no
 *     initialization and carries nothing from one call to the next (an amax
 *     pass writes per-workgroup partial maxima there, and for RMSNorm each
 *     row's 1/rms, and the encode pass of the same call reads them; every such
 *     slot read is written earlier in the same call). One workspace serves any
 *     number of calls that are ordered on one stream; calls that can run at
 *     the same time (different streams) need different workspaces.
 *   - Errors are returned synchronously, before anything is enqueued, except
 *     NVFP4Q_E_LAUNCH. Device-side data that break a stated rule (for example
 *     decreasing group offsets) give unspecified output but no out-of-bounds
 *     access.
 *   - Shapes: elements per row (`cols`, `hidden`) must be a multiple of 16;
 *     a columnwise plane needs rows % 16 == 0 (except grouped mode, which pads
 *     each group). Leading dimensions are in elements for input and output
 *     tensors (x, y, q, k) and in bytes for code and scale planes. Input and
 *     output tensors start 16-byte aligned and their rows stay so (leading
 *     dimension times element size a multiple of 16); code planes are 16-byte
 *     aligned with ld_codes a multiple of 8 bytes. Scale planes have no
 *     alignment rule.
 *   - Element types: every entry point takes bfloat16, float16 and float32
 *     input (nvfp4q_dtype); any other value returns NVFP4Q_E_UNSUPPORTED.
 */
#ifndef NVFP4Q_H
#define NVFP4Q_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  NVFP4Q_OK = 0,
  NVFP4Q_E_NULLPTR = 1,     /* a required pointer is NULL */
  NVFP4Q_E_SHAPE = 2,       /* a size or leading dimension breaks the shape rules
                               (every leading dimension is at most 2^40) */
  NVFP4Q_E_ALIGN = 3,       /* a pointer or leading dimension breaks the alignment rules */
  NVFP4Q_E_UNSUPPORTED = 4, /* dtype, rounding mode or option not built */
  NVFP4Q_E_LAUNCH = 5,      /* a kernel launch failed on the HIP side */
  NVFP4Q_E_WORKSPACE = 6,   /* workspace missing, misaligned or too small */
  NVFP4Q_STATUS_MAX_ENUM = 0x7FFFFFFF /* not a status: every enum here is a 32-bit
                                         type that holds any non-negative int */
} nvfp4q_status;

/* Element type of the input; every entry point takes all three. The
 * quantizers (rowwise, 2D, grouped) read the values exactly as given; the
 * grouped transform rounds its output through the input's type (bf16, fp16;
 * fp32: not at all). The norms take gamma (and beta) in the input's type and
 * round their output y to nearest even in that type (fp32: not rounded
 * further); rmsnorm_nvfp4q quantizes that y. Rows of x (and y) start 16-byte
 * aligned: leading dimension * element size is a multiple of 16. */
typedef enum { NVFP4Q_BF16 = 0, NVFP4Q_FP16 = 1, NVFP4Q_FP32 = 2, NVFP4Q_DTYPE_MAX_ENUM = 0x7FFFFFFF } nvfp4q_dtype;

/* Rounding of the E2M1 codes. NVFP4Q_FAST_MATH may be OR-ed into the value
 * passed as `rounding` ([PR, Fast math]): with the grouped transform on, the
 * transform's fp32 output is quantized (and enters the group amax) without
 * its bf16 round-through; the encode reciprocal stays correctly rounded (it
 * comes from a 127-entry table per workgroup, so an approximate reciprocal
 * would save nothing). On paths without the transform the flag changes
 * nothing. Other bits: NVFP4Q_E_UNSUPPORTED. */
typedef enum { NVFP4Q_RTNE = 0, NVFP4Q_SR = 1, NVFP4Q_ROUNDING_MAX_ENUM = 0x7FFFFFFF } nvfp4q_rounding;
#define NVFP4Q_FAST_MATH 0x100
/* nvfp4q_quantize_2d only (other entry points: NVFP4Q_E_UNSUPPORTED): one
 * E4M3 scale per 16 x 16 tile of x, used by both planes, so that a weight and
 * its transpose decode to the same values. */
#define NVFP4Q_SCALE_16X16 0x200
/* rmsnorm_nvfp4q and rmsnorm_nvfp4q_noalloc only (other entry points:
 * NVFP4Q_E_UNSUPPORTED): with codes, at most 64 tokens, hidden <= 16384 and
 * no given amax, one launch (one workgroup per token) whose workgroups meet on the amax inside
 * it ([Blog] Grid synchronization) instead of an amax pass and an encode pass;
 * same results. It keeps state in the workspace's first 640 bytes (see the
 * workspace convention). Measured on MI355X it is not faster than the two
 * launches (8 x 7168 with a bias, graph replay: 6.87 us per call against
 * 6.86 us; the wait for every workgroup's maximum costs what the second
 * launch does), so it is an option, not the default; otherwise it changes
 * nothing. */
#define NVFP4Q_ONE_LAUNCH 0x400

/* One quantized plane. codes: device, [plane_rows][ld_codes] bytes, two E2M1
 * codes per byte, even element in the low nibble. scales: device,
 * [plane_rows][ld_scales] E4M3 bytes, one per 16 elements. A rowwise plane of
 * an [R, C] input has R plane rows of C/2 code bytes and C/16 scale bytes; a
 * columnwise plane has C plane rows of R/2 code bytes and R/16 scale bytes
 * (plane row c holds input column c). */
typedef struct {
  uint8_t *codes;
  int64_t ld_codes;
  uint8_t *scales;
  int64_t ld_scales;
} nvfp4q_plane;

/* Per-tensor (or per-group) scale. All device pointers, each 1 float (G floats
 * in grouped mode). amax_in: nullable; when given it is used as amax and the
 * amax pass is skipped ("precomputed amax"). amax_out, scale_out: nullable;
 * receive the amax used and S_dec = amax / 2688 (1 when amax is 0). */
typedef struct {
  const float *amax_in;
  float *amax_out;
  float *scale_out;
} nvfp4q_global;

/* Stochastic-rounding state; ignored under NVFP4Q_RTNE. */
typedef struct {
  uint64_t seed;
  uint32_t offset;
} nvfp4q_rng;

/* Bytes of workspace every entry point needs (a constant, 1 MiB). */
size_t nvfp4q_workspace_bytes(void);

/* Static description of a status code (any int value; unknown ones get
 * "unknown status"); never NULL. */
const char *nvfp4q_status_string(nvfp4q_status s);

/* ABI version: 1. */
int nvfp4q_version(void);

/* The sha256 (64 lowercase hex digits) of the sources this library was built
 * from: every file of the package's csrc/ directory and of include/, in name
 * order, as rmsnorm_nvfp4_block_amd/build.py computes it; "unknown" when the
 * library was built without it. Lets a caller check that a prebuilt library
 * matches the sources beside it. A static string, never NULL. */
const char *nvfp4q_source_sha256(void);

/*
 * nvfp4q_quantize -- rowwise NVFP4 of a [rows, cols] bf16, fp16 or fp32 tensor.
 *   x: device, rows x cols of dtype, row stride ld_x elements.
 *   g: per-tensor scale (amax computed from x unless g->amax_in is given).
 *   row: the rowwise plane [rows][cols/2] codes, [rows][cols/16] scales.
 *   rounding: NVFP4Q_RTNE or NVFP4Q_SR (rng used, tag 0,
 *             block index = row * (cols/16) + col/16).
 * rows == 0 writes amax_out = 0 and scale_out = 1 and nothing else.
 * [PR, Optimization 1, 4, 6, 7; Blog, Blackwell support]
 */
nvfp4q_status nvfp4q_quantize(const void *x, nvfp4q_dtype dtype, int64_t rows, int64_t cols,
                              int64_t ld_x, const nvfp4q_global *g, const nvfp4q_plane *row,
                              nvfp4q_rounding rounding, const nvfp4q_rng *rng, void *workspace,
                              size_t workspace_bytes, void *stream);

/*
 * rmsnorm_nvfp4q -- per-token RMSNorm feeding rowwise NVFP4.
 *   y = RN_T((gamma + weight_offset) * (x * r) [+ beta]),
 *   r = 1 / sqrt(sum_k x_k^2 / hidden + eps),
 *   T the input's element type (bf16, fp16; for fp32 input y is the fp32
 *   result); the quantizer consumes that y and amax = max |y|.
 *   fp32 evaluation: g = RN(gamma + weight_offset) per column, the sum of
 *   squares ss in fp32, r = v_rsq_f32(RN(RN(ss * RN(1 / hidden)) + eps))
 *   (within 1 ulp),
 *   then y = RN_T(RN(RN(x * g) * r)), or with beta
 *   y = RN_T(fma(RN(x * g), r, beta)) (one rounding for the product and the
 *   sum). The order of the sum of squares is not fixed: y may differ from the
 *   exactly rounded value by one step of T where the exact value lies next to
 *   a rounding boundary.
 *   [Blog, QK Norm: rsqrt of the mean square plus EPS, weight plus a
 *   compile-time WEIGHT_BIAS, cast back to the element type; Configuration
 *   space: the input and output type is a knob]
 *   x: device [tokens, hidden] of `dtype`, row stride ld_x.
 *   gamma: device [hidden] of `dtype` (required). beta: device [hidden] of
 *     `dtype`, or NULL (no-bias variant, compiled separately).
 *   weight_offset: added to gamma (the page's WEIGHT_BIAS); must be 0 or 1.
 *   eps: added to the mean square.
 *   y_out: device [tokens, hidden] of `dtype` with row stride ld_y, or NULL.
 *   row: the rowwise plane, or row->codes == NULL to produce only y_out.
 *   rounding / rng as for nvfp4q_quantize.
 *   g: as for nvfp4q_quantize; with g->amax_in the call is one pass over x
 *     (the amax is not computed), otherwise an amax pass precedes the encode
 *     pass (or, with NVFP4Q_ONE_LAUNCH and at most 64 tokens, one launch).
 *     hidden <= 32768 for bf16 and fp16, <= 16384 for fp32
 *     (NVFP4Q_E_UNSUPPORTED above that); rows wider than 16384 take the
 *     cooperative-row passes with gamma and beta read where they are used.
 */
nvfp4q_status rmsnorm_nvfp4q(const void *x, nvfp4q_dtype dtype, int64_t tokens, int64_t hidden,
                             int64_t ld_x, const void *gamma, const void *beta, float weight_offset,
                             float eps, void *y_out, int64_t ld_y, const nvfp4q_global *g,
                             const nvfp4q_plane *row, nvfp4q_rounding rounding,
                             const nvfp4q_rng *rng, void *workspace, size_t workspace_bytes,
                             void *stream);

/*
 * rmsnorm_nvfp4q_noalloc -- rmsnorm_nvfp4q without a workspace argument, for
 * callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid allocation): the library's own
 * static 1 MiB device array stands in for the workspace. Arguments, results
 * and errors are those of rmsnorm_nvfp4q (the same kernels run); nothing is
 * allocated or freed, and every shape rmsnorm_nvfp4q accepts fits the array
 * (that path needs a constant 1 MiB). The array exists once per GPU, is held
 * until the process ends, starts as zeros, and keeps the last call's contents
 * (its first 640 bytes the NVFP4Q_ONE_LAUNCH state, as for a workspace; no
 * call reads the rest before writing it); calls that can overlap on one GPU (different
 * streams, or different host threads on one device) race on it and must not
 * be issued. NVFP4Q_E_LAUNCH if the array's device address cannot be looked
 * up on the current device.
 */
nvfp4q_status rmsnorm_nvfp4q_noalloc(const void *x, nvfp4q_dtype dtype, int64_t tokens, int64_t hidden,
                                     int64_t ld_x, const void *gamma, const void *beta, float weight_offset,
                                     float eps, void *y_out, int64_t ld_y, const nvfp4q_global *g,
                                     const nvfp4q_plane *row, nvfp4q_rounding rounding,
                                     const nvfp4q_rng *rng, void *stream);

/*
 * nvfp4q_quantize_2d -- rowwise and columnwise (transposed) planes of one
 * [rows, cols] tensor (bf16, fp16 or fp32) under one shared per-tensor scale
 * (weights).
 *   row: rowwise plane or row->codes == NULL; col: columnwise plane
 *   [cols][rows/2] codes, [cols][rows/16] scales, or col->codes == NULL
 *   (with rows == 0 a given plane may have NULL pointers).
 *   rows % 16 == 0 when the columnwise plane is requested.
 *   SR: rowwise blocks use tag 0 and index row * (cols/16) + col/16;
 *   columnwise blocks use tag 1 and index col * (rows/16) + row/16.
 *   NVFP4Q_SCALE_16X16 in `rounding`: the block amax is taken over the 16 x 16
 *   tile (rows 16i.., columns 16j..) and every element of the tile is encoded
 *   with that tile's scale in both planes; the scale arrays keep their layout
 *   (the tile's code on each of its 16 rows, resp. 16 columns); rows % 16 == 0
 *   also for a rowwise-only call. The pages measure "2D weights" and describe
 *   columnwise reads sharing one amax and reciprocal without defining the
 *   tile; this is the reading taken.
 *   [PR, Optimization 2 (2D weight kernel, staged columnwise reads);
 *    Performance (2D weights against a precomputed amax)]
 */
nvfp4q_status nvfp4q_quantize_2d(const void *x, nvfp4q_dtype dtype, int64_t rows, int64_t cols,
                                 int64_t ld_x, const nvfp4q_global *g, const nvfp4q_plane *row,
                                 const nvfp4q_plane *col, nvfp4q_rounding rounding,
                                 const nvfp4q_rng *rng, void *workspace, size_t workspace_bytes,
                                 void *stream);

/*
 * nvfp4q_quantize_2d_grouped -- nvfp4q_quantize_2d of `experts` weights of
 * [rows, cols] each, stacked in x as [experts * rows, cols] (expert e in rows
 * e * rows ..), in one launch per pass, each weight under its own amax.
 *   g: amax_in / amax_out / scale_out hold `experts` floats each.
 *   row: rowwise plane of the stacked x ([experts * rows] plane rows).
 *   col: the experts' columnwise planes stacked: [experts * cols] plane rows,
 *     expert e's transposed plane in plane rows e * cols ..
 *   SR: expert e uses tag 2e (rowwise) and 2e + 1 (columnwise) with the block
 *   indices of nvfp4q_quantize_2d of its own weight, so expert 0 matches that
 *   call and no two experts share a random stream. NVFP4Q_SCALE_16X16 as there.
 *   1 <= experts <= 64, else NVFP4Q_E_SHAPE.
 *   [PR, Performance (grouped 2D weights, E = 4 experts, against a
 *    precomputed amax)]
 */
nvfp4q_status nvfp4q_quantize_2d_grouped(const void *x, nvfp4q_dtype dtype, int32_t experts, int64_t rows,
                                         int64_t cols, int64_t ld_x, const nvfp4q_global *g,
                                         const nvfp4q_plane *row, const nvfp4q_plane *col,
                                         nvfp4q_rounding rounding, const nvfp4q_rng *rng, void *workspace,
                                         size_t workspace_bytes, void *stream);

/*
 * nvfp4q_qk_norm -- per-head RMSNorm of the attention heads of q and k, in
 * place, one launch for both ("CuTeDSL at Perplexity", QK Norm):
 *   y = RN((w + c) * (x * r)),  r = 1 / sqrt(sum x^2 / head_dim + eps)
 * over each head of head_dim (64, 128 or 256; else NVFP4Q_E_UNSUPPORTED)
 * consecutive elements, fp32 arithmetic, rounded to nearest even in the
 * input's type (fp32: not rounded further) and written over x.
 *   q: device bf16, fp16 or fp32 (dtype), `tokens` rows of q_heads *
 *     head_dim elements, row stride ld_q elements (16-byte aligned rows); k
 *     likewise with k_heads and ld_k. Either head count may be 0 (its pointers then unused), not
 *     both.
 *   q_weight, k_weight: device [head_dim] of the same dtype, 16-byte aligned.
 *   weight_offset: c, 0 or 1; eps >= 0 (float32).
 *   No workspace; no output besides q and k. The pages fix no reduction
 *   order: the sum of squares is an fp32 sum in DPP steps, r comes from
 *   v_rsq_f32 (within 1 ulp), so y can differ from the exactly rounded value
 *   by about one bf16 step.
 */
nvfp4q_status nvfp4q_qk_norm(void *q, void *k, nvfp4q_dtype dtype, int64_t tokens, int32_t q_heads,
                             int32_t k_heads, int32_t head_dim, int64_t ld_q, int64_t ld_k,
                             const void *q_weight, const void *k_weight, float weight_offset, float eps,
                             void *stream);

/*
 * nvfp4q_grouped -- per-group NVFP4 of a packed [total_rows, cols] tensor
 * (bf16, fp16 or fp32): the columnwise plane, optionally after a 16-point random Hadamard
 * transform along the rows of each 16-row block, and/or the rowwise plane,
 * each with one global scale per group, from one read of x.
 *   offsets: device int32 [num_groups + 1]; offsets[0] = 0, non-decreasing,
 *     offsets[num_groups] = total_rows; group g is rows offsets[g] ..
 *     offsets[g+1] - 1. 1 <= num_groups <= 64.
 *   Columnwise: each group is zero-padded to P_g = 16 * ceil(n_g / 16) rows;
 *   padded groups are laid out back to back: group g owns plane columns
 *   Poff[g] .. Poff[g] + P_g - 1, Poff = exclusive prefix sum of P_g.
 *   padded_offsets_out: device int32 [num_groups + 1] receives Poff (nullable).
 *   apply_rht: 0 or 1. With 1, each 16-row block of one column becomes
 *     bf16_rne(0.25 * H16 * D * v): D = diag(d), d_i = -1 iff bit i of
 *     rht_sign_mask is set, H16 the Sylvester Hadamard matrix evaluated as
 *     four butterfly stages (h = 1, 2, 4, 8) of fp32 (a + b, a - b).
 *     The transform and the columnwise amax see the zero-padded rows. With
 *     NVFP4Q_FAST_MATH in `rounding` the bf16 rounding is left out.
 *   g, col: the columnwise scales (G floats each: amax_in optional, amax_out,
 *     scale_out; g nullable) and plane, `cols` plane rows; ld_codes * 2 and
 *     ld_scales * 16 must be >= total_rows + 15 * num_groups (the largest
 *     possible padded length). Plane columns at and past Poff[G] are never
 *     written [PR, Grouped allocation tail]. col NULL (or col->codes NULL):
 *     no columnwise plane.
 *   g_row, row: the rowwise scales (G floats each, nullable) and plane
 *     ([total_rows, cols/2] codes, [total_rows, cols/16] scales), as
 *     nvfp4q_quantize of each group's rows under the group's own amax
 *     max|x| (no transform) [PR, Performance (grouped rowwise + columnwise
 *     in one pass)]. row NULL (or row->codes NULL while total_rows > 0):
 *     no rowwise plane. At least one plane must be given.
 *   SR: columnwise tag 1, block index = plane_row * (Poff[G] / 16) +
 *   plane_col / 16; rowwise tag 0, block index = row * (cols / 16) + col / 16.
 *   Without amax_in (for a requested plane) the amax pass keeps one maximum
 *   per group for each of its workgroups (at most 1024) in the workspace, so
 *   the workspace bounds no input size.
 *   A row stride above 2^25 bytes (ld_x above 2^24 for bf16 / fp16, 2^23 for
 *   fp32) returns NVFP4Q_E_SHAPE (the kernels address 32 rows of x with
 *   32-bit byte offsets). fp16 / fp32 input: the transform's output is
 *   rounded through the input's type (fp16), or not at all (fp32).
 *   [PR, Optimization 2, 3, 5; Fast math (bf16 round-through of the
 *    transform); Config surface and AUTO (64 groups, device offsets)]
 */
nvfp4q_status nvfp4q_grouped(const void *x, nvfp4q_dtype dtype, int64_t total_rows, int64_t cols,
                             int64_t ld_x, const int32_t *offsets, int32_t num_groups,
                             int32_t *padded_offsets_out, int apply_rht, uint32_t rht_sign_mask,
                             const nvfp4q_global *g, const nvfp4q_plane *col,
                             const nvfp4q_global *g_row, const nvfp4q_plane *row,
                             nvfp4q_rounding rounding, const nvfp4q_rng *rng, void *workspace,
                             size_t workspace_bytes, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* NVFP4Q_H */
