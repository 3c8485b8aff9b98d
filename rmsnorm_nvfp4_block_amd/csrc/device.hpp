// Device helpers shared by the gfx950 kernels: bf16 widening and rounding,
// E4M3/E2M1 conversions, per-tensor and per-block scales, Philox4x32-10,
// stochastic rounding, wave reductions and the workspace layout.
//
// Sources: "[nvfp4_training] Optimize CuteDSL kernels for NVFP4 training"
// (pytorch/ao PR 4798), Optimization items 1, 3, 6, 7 and Fast math;
// "CuTeDSL at Perplexity", QK Norm and Blackwell support.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nvfp4q {

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;
constexpr float kFltMax = 3.40282347e+38f;

// ---------------------------------------------------------------- workspace
// Device memory shared by the kernels of one call, in a caller-owned buffer.
// An amax pass writes one partial maximum per workgroup into `partial` with a
// plain store; the encode pass that follows reduces the partials it needs at its
// start (the kernel boundary orders the two). Every slot an encode pass reads is
// written earlier in the same call, so `partial` carries no state between
// calls and needs no reset.
//
// The rowwise RMSNorm amax pass launches at most kRowPartials workgroups and
// also leaves each row's 1/rms in partial[kRowPartials + row] (rows up to
// kRowScaleCap), so that the encode pass can stream the row in pieces.
//
// The one-launch RMSNorm for a few rows (at most kBarrierSlots workgroups, all
// resident at once) meets inside the kernel instead (grid_max below): status[0]
// counts its completed calls, slot[w] holds (that count + 1, workgroup w's
// maximum), status[1] is set if a wait ever gave up. These words carry state
// from call to call: they must start equal (zeros) and only that kernel
// writes them.
constexpr int kBarrierSlots = 64;
constexpr int kPartials = 262144 - 32 - 2 * kBarrierSlots;
constexpr int kRowPartials = 4096;
constexpr int kRowScaleCap = kPartials - kRowPartials;
struct Workspace {
  uint32_t status[32];             // [0] one-launch calls completed, [1] a wait gave up; the rest reserved
  uint64_t slot[kBarrierSlots];    // one-launch: (calls completed + 1) << 32 | the workgroup's maximum
  float partial[kPartials];        // per-workgroup partial maxima of the last amax pass
};
static_assert(sizeof(Workspace) == 1 << 20, "workspace layout");

// ---------------------------------------------------------------- bf16
// bfloat16 -> float32 is a 16-bit shift (PR, Optimization item 6).
__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Two float32 -> packed bf16x2 with round-to-nearest-even (v_cvt_pk_bf16_f32;
// checked bit-exact against the definition over every finite float32).
__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  f32x2 v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

// float32 rounded to nearest even in bf16, returned as float32: the same
// conversion with +0 in the low half leaves exactly the bf16 value's float32
// bits (one instruction, where packing a pair and widening both halves takes
// three for two values).
__device__ __forceinline__ float bf16_round(float a) {
  f32x2 v = {0.0f, a};
  return __builtin_bit_cast(float, __builtin_convertvector(v, bf16x2));
}

// A 64-bit value that is the same for every lane, kept in scalar registers
// (the compiler otherwise folds a row's offset into per-lane 64-bit address
// math).
__device__ __forceinline__ int64_t uniform_i64(int64_t v) {
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)v);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)((uint64_t)v >> 32));
  return (int64_t)(((uint64_t)hi << 32) | lo);
}

// ---------------------------------------------------------------- FP8 / FP4
// E4M3 code of a non-negative float: round to nearest even, saturating at 448.
// v_cvt_pk_fp8_f32 rounds to nearest even over [0, 448] including subnormals
// (checked exhaustively); the clamp supplies the saturation.
__device__ __forceinline__ uint32_t e4m3_code(float s) {
  s = fminf(s, 448.0f);
  // both halves of the destination word are written: any `old` value serves (s's bits: no zero to copy)
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(s, s, __float_as_int(s), false) & 0xFFu;
}
__device__ __forceinline__ float e4m3_value(uint32_t code) {
  return __builtin_amdgcn_cvt_f32_fp8((int)code, 0);
}

// Two float32 -> two E2M1 codes (round to nearest even, saturating to 6, sign
// kept) written into byte SEL of `old`, first value in the low nibble. With a
// unit scale v_cvt_scalef32_pk_fp4_f32 matches that definition on every
// float32 input.
template <int SEL>
__device__ __forceinline__ uint32_t e2m1x2(uint32_t old, float a, float b) {
  return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(old, a, b, 1.0f, SEL);
}

// ---------------------------------------------------------------- scales
// Per-tensor scales from amax: S_enc = 2688 / amax, S_dec = amax / 2688, each a
// correctly rounded fp32 division; 1 and 1 when amax is 0 or S_enc overflows.
struct GScale {
  float enc, dec;
};
__device__ __forceinline__ GScale global_scale(float amax) {
  float enc = 2688.0f / amax;
  float dec = amax / 2688.0f;
  bool bad = !(amax > 0.0f) || !(enc <= kFltMax);
  GScale g;
  g.enc = bad ? 1.0f : enc;
  g.dec = bad ? 1.0f : dec;
  return g;
}

// RN(b / 6) for b >= 0. For normal b, q0 = RN(b * RN(1/6)) is corrected once
// with the exact remainder fma(-q0, 6, b) (Markstein's correction); this equals
// the correctly rounded quotient for every normal float32 (checked
// exhaustively). Subnormal b takes the division.
__device__ __forceinline__ float div6(float b) {
  const float y = 0.166666672f;  // RN(1/6)
  const float q0 = b * y;
  const float r = __builtin_fmaf(-q0, 6.0f, b);
  const float q1 = __builtin_fmaf(r, y, q0);
  if (__builtin_expect(b < 1.17549435e-38f, 0)) return b / 6.0f;
  return q1;
}

// Block scale code: E4M3(RN(RN(bmax / 6) * S_enc)).
__device__ __forceinline__ uint32_t block_scale(float bmax, float s_enc) {
  return e4m3_code(div6(bmax) * s_enc);
}

// Encode multiplier for a block scale code: RN(1 / RN(f32(s) * S_dec)),
// 0 for a zero scale, clamped to the largest finite float (PR, Fast math:
// the exact path takes the correctly rounded reciprocal of this product).
__device__ __forceinline__ float encode_mult(uint32_t scode, float s_dec) {
  float p = e4m3_value(scode) * s_dec;
  float r = fminf(1.0f / p, kFltMax);
  return scode ? r : 0.0f;
}

// ---------------------------------------------------------------- Philox
// Philox4x32-10 (Salmon, Moraes, Dror and Shaw, SC'11): ten rounds of two
// 32x32->64-bit products of counter words 0 and 2 mixed into the other words
// and the key by XOR, with Weyl key increments between rounds.
struct U4 {
  uint32_t x, y, z, w;
};
// a ^ b ^ k in one v_bitop3_b32 (truth table 0x96 = three-input XOR; the
// compiler emits two XORs for the plain expression).
__device__ __forceinline__ uint32_t xor3_key(uint32_t a, uint32_t b, uint32_t k) {
  return __builtin_amdgcn_bitop3_b32(a, b, k, 0x96);
}

// The key (the seed) must be the same for every lane of the wave.
__device__ __forceinline__ U4 philox10(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3,
                                       uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    uint64_t p0 = (uint64_t)0xD2511F53u * c0;
    uint64_t p1 = (uint64_t)0xCD9E8D57u * c2;
    uint32_t n0 = xor3_key((uint32_t)(p1 >> 32), c1, k0);
    uint32_t n2 = xor3_key((uint32_t)(p0 >> 32), c3, k1);
    c1 = (uint32_t)p1;
    c3 = (uint32_t)p0;
    c0 = n0;
    c2 = n2;
    k0 += 0x9E3779B9u;
    k1 += 0xBB67AE85u;
  }
  return U4{c0, c1, c2, c3};
}

// The four random words of one 16-element block: key = seed, counter =
// (block lo32, block hi32, tag, offset). Tag 0 rowwise, 1 columnwise.
__device__ __forceinline__ U4 block_random(uint64_t blk, uint32_t tag, uint64_t seed, uint32_t offset) {
  return philox10((uint32_t)blk, (uint32_t)(blk >> 32), tag, offset, (uint32_t)seed,
                  (uint32_t)(seed >> 32));
}

// Stochastic rounding onto the signed E2M1 grid. The definition: with
// lo <= |v| < hi the neighbouring magnitudes (|v| clamped to 6) and frac the
// position of |v| between them, the magnitude becomes hi iff
// r + floor(256 * frac) >= 256 for the element's random byte r; the sign is
// kept as in round-to-nearest.
//
// v_cvt_scalef32_sr_pk_fp4_f32 converts a pair (a, b) with one 32-bit random
// operand R: for a it adds R to the bits below the E2M1 step and keeps the
// carry, for b it does the same with R << 1 (measured: b follows the rule with
// byte r exactly when R = r << 23, a when R = r << 24, zeros below; checked
// against the definition on 4096 values x 256 bytes). Each element has its own
// byte, so a pair is converted twice: once with a's byte in bits 31..24 (the
// low nibble, a's code, is kept) and once with b's byte in bits 30..23 (the
// high nibble, b's code, is kept).
//
// The instruction writes only the byte of its destination that op_sel[3:2]
// selects, so four conversions fill one register; the compiler's builtin does
// not tie the destination's other bytes to its `old` operand, so bytes 1..3
// are written through inline assembly with the register as an in-out operand
// (byte 0 by the builtin, whose other bytes are then overwritten).
template <int SEL>
__device__ __forceinline__ uint32_t sr_byte(uint32_t acc, f32x2 ab, uint32_t r) {
  if constexpr (SEL == 0) {
    return __builtin_amdgcn_cvt_scalef32_sr_pk_fp4_f32(acc, ab, r, 1.0f, 0);
  } else if constexpr (SEL == 1) {
    asm("v_cvt_scalef32_sr_pk_fp4_f32 %0, %1, %2, 1.0 op_sel:[0,0,1,0]" : "+v"(acc) : "v"(ab), "v"(r));
  } else if constexpr (SEL == 2) {
    asm("v_cvt_scalef32_sr_pk_fp4_f32 %0, %1, %2, 1.0 op_sel:[0,0,0,1]" : "+v"(acc) : "v"(ab), "v"(r));
  } else {
    asm("v_cvt_scalef32_sr_pk_fp4_f32 %0, %1, %2, 1.0 op_sel:[0,0,1,1]" : "+v"(acc) : "v"(ab), "v"(r));
  }
  return acc;
}

// Byte K of w in bits 31..24, zeros below (the random operand of a pair's
// first element).
template <int K>
__device__ __forceinline__ uint32_t rand_first(uint32_t w) {
  if constexpr (K == 0) return w << 24;
  else if constexpr (K == 3) return w & 0xFF000000u;
  else return __builtin_amdgcn_perm(0u, w, (uint32_t)(K << 24) | 0x000C0C0Cu);  // 0x0C: a zero byte
}
// Byte K of w in bits 30..23, zeros below (the operand of a pair's second
// element, which the instruction shifts left by one).
template <int K>
__device__ __forceinline__ uint32_t rand_second(uint32_t w) {
  if constexpr (K == 1) {
    // one shift with the byte selected as its source operand (SDWA)
    uint32_t r;
    asm("v_lshlrev_b32_sdwa %0, %1, %2 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:DWORD src1_sel:BYTE_1"
        : "=v"(r) : "v"(23u), "v"(w));
    return r;
  }
  return ((w >> (8 * K)) & 0xFFu) << 23;
}

// Eight SR codes packed in a word (element 2i in the low nibble of byte i).
// Element e takes byte (e & 3) of w0 (e < 4) or of w1 (e >= 4). Register a
// collects the conversions for the first elements (low nibbles kept), b those
// for the second elements (high nibbles kept).
__device__ __forceinline__ uint32_t sr_pack8(const float v[8], uint32_t w0, uint32_t w1) {
  const f32x2 p0 = {v[0], v[1]}, p1 = {v[2], v[3]}, p2 = {v[4], v[5]}, p3 = {v[6], v[7]};
  // every byte of a and b is written below, so their first `old` can be any
  // value: the random operand itself, which is dead afterwards (no copy of a zero)
  const uint32_t ra = rand_first<0>(w0), rb = rand_second<1>(w0);
  uint32_t a = sr_byte<0>(ra, p0, ra);
  uint32_t b = sr_byte<0>(rb, p0, rb);
  a = sr_byte<1>(a, p1, rand_first<2>(w0));
  b = sr_byte<1>(b, p1, rand_second<3>(w0));
  a = sr_byte<2>(a, p2, rand_first<0>(w1));
  b = sr_byte<2>(b, p2, rand_second<1>(w1));
  a = sr_byte<3>(a, p3, rand_first<2>(w1));
  b = sr_byte<3>(b, p3, rand_second<3>(w1));
  return (a & 0x0F0F0F0Fu) | (b & 0xF0F0F0F0u);  // v_bfi_b32
}

// Eight RTNE codes packed in a word.
__device__ __forceinline__ uint32_t rtne_pack8(const float v[8]) {
  // every byte is written, so the first `old` can be any value: v[0]'s bits
  uint32_t out = __float_as_uint(v[0]);
  out = e2m1x2<0>(out, v[0], v[1]);
  out = e2m1x2<1>(out, v[2], v[3]);
  out = e2m1x2<2>(out, v[4], v[5]);
  out = e2m1x2<3>(out, v[6], v[7]);
  return out;
}

// ---------------------------------------------------------------- lanes
// Value from the neighbouring lane (lane ^ 1) through DPP quad_perm [1,0,3,2].
__device__ __forceinline__ float swap_pair(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0xB1, 0xF, 0xF, false));
}
__device__ __forceinline__ uint32_t swap_pair_u(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, false);
}

// DPP lane moves (row = 16 lanes). bound_ctrl keeps the source value for
// lanes whose source is outside the row mask.
template <int CTRL, int ROWMASK = 0xF>
__device__ __forceinline__ float dpp_f(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, ROWMASK, 0xF, false));
}
constexpr int kDppXor1 = 0xB1;          // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;          // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141;   // reverse within 8 lanes
constexpr int kDppMirror = 0x140;       // reverse within 16 lanes
constexpr int kDppBcast15 = 0x142;      // lane 15 of each row to the next row
constexpr int kDppBcast31 = 0x143;      // lane 31 to rows 2 and 3

// Sum / max over the 64 lanes, returned as a wave-uniform value: reductions
// within each 16-lane row by DPP, then across rows with the row broadcasts;
// lane 63 holds the total.
__device__ __forceinline__ float wave_sum(float v) {
  v += dpp_f<kDppXor1>(v);
  v += dpp_f<kDppXor2>(v);
  v += dpp_f<kDppHalfMirror>(v);
  v += dpp_f<kDppMirror>(v);
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), kDppBcast15, 0xA, 0xF, false));
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), kDppBcast31, 0xC, 0xF, false));
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 63));
}
__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, dpp_f<kDppXor1>(v));
  v = fmaxf(v, dpp_f<kDppXor2>(v));
  v = fmaxf(v, dpp_f<kDppHalfMirror>(v));
  v = fmaxf(v, dpp_f<kDppMirror>(v));
  v = fmaxf(v, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), kDppBcast15, 0xA, 0xF, false)));
  v = fmaxf(v, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), kDppBcast31, 0xC, 0xF, false)));
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 63));
}

// Maxima of magnitudes with v_max3_f32 and absolute-value source modifiers:
// 16 values in 7 three-input maxima and one two-input maximum (the compiler,
// left to fmaxf, adds a canonicalizing max per value, and every max is a
// slow VALU instruction on gfx950). For finite inputs the result equals the
// fmaxf form; non-finite inputs are outside the method's definition.
__device__ __forceinline__ float max3_abs(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, |%1|, |%2|, |%3|" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}
// max(m, |a|, |b|) for m >= 0
__device__ __forceinline__ float max3_m_abs(float m, float a, float b) {
  float r;
  asm("v_max3_f32 %0, %1, |%2|, |%3|" : "=v"(r) : "v"(m), "v"(a), "v"(b));
  return r;
}
__device__ __forceinline__ float max3_pos(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}
__device__ __forceinline__ float max8_abs(const float v[8]) {
  const float a = max3_abs(v[0], v[1], v[2]);
  const float b = max3_abs(v[3], v[4], v[5]);
  return fmaxf(b, max3_m_abs(a, v[6], v[7]));
}
__device__ __forceinline__ float max16_abs(const float v[16]) {
  const float a = max3_abs(v[0], v[1], v[2]);
  const float b = max3_abs(v[3], v[4], v[5]);
  const float c = max3_abs(v[6], v[7], v[8]);
  const float d = max3_abs(v[9], v[10], v[11]);
  const float e = max3_abs(v[12], v[13], v[14]);
  return fmaxf(max3_pos(a, b, c), max3_m_abs(d, e, v[15]));
}

__device__ __forceinline__ void widen8(const uint4 q, float v[8]) {
  v[0] = bf_lo(q.x); v[1] = bf_hi(q.x);
  v[2] = bf_lo(q.y); v[3] = bf_hi(q.y);
  v[4] = bf_lo(q.z); v[5] = bf_hi(q.z);
  v[6] = bf_lo(q.w); v[7] = bf_hi(q.w);
}

// ---------------------------------------------------------------- loads
// 16-byte load of 8 bf16 values, zero when !ok. The if-form keeps the access a
// single global_load_dwordx4 (a select between the load and a zero vector is
// split into four dword loads by the compiler).
__device__ __forceinline__ uint4 ld16(const void* p, bool ok) {
  uint4 q = make_uint4(0u, 0u, 0u, 0u);
  if (ok) q = *reinterpret_cast<const uint4*>(p);
  return q;
}

// Encode-reciprocal table for the 127 finite non-negative E4M3 codes (index
// 127 is never produced), filled by threads 0..127 of a workgroup.
__device__ __forceinline__ void fill_rcp_table(float* tab, float s_dec) {
  if (threadIdx.x < 128) tab[threadIdx.x] = encode_mult(threadIdx.x, s_dec);
}

constexpr int kWGThreads = 256;  // the usual workgroup; kernels of other sizes pass their wave count
constexpr int kWavesPerWG = kWGThreads / kWave;

// ---------------------------------------------------------------- consumers
// Workgroup-wide max of a per-lane value over NW waves (all threads must call).
template <int NW = kWavesPerWG>
__device__ __forceinline__ float wg_max(float m) {
  __shared__ float red[NW];
  m = wave_max(m);
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  __syncthreads();
  if (lane == 0) red[wid] = m;
  __syncthreads();
  float t = red[0];
#pragma unroll
  for (int i = 1; i < NW; ++i) t = fmaxf(t, red[i]);
  return t;
}

// Max over partial[first .. first + n) with all threads of the workgroup.
// (NW: the waves of the calling workgroup.)
template <int NW = kWavesPerWG>
__device__ __forceinline__ float reduce_partials(const Workspace* ws, uint32_t first, uint32_t n) {
  float m = 0.0f;
  for (uint32_t i = threadIdx.x; i < n; i += 64 * NW) m = fmaxf(m, ws->partial[first + i]);
  return wg_max<NW>(m);
}

// Per-tensor scales for an encode kernel, into every thread, and the encode
// reciprocal table into LDS: from amax_in when given, otherwise the max of the
// `nparts` partials of the amax pass. Workgroup 0 of the tensor (blockIdx.x 0;
// a launch over several tensors has one per blockIdx.y, and passes that
// tensor's amax_out / scale_out) reports amax and S_dec.
__device__ __forceinline__ GScale scales_from(float a, float* amax_out, float* scale_out, float* rcp_tab) {
  const GScale g = global_scale(a);
  if (threadIdx.x == 0 && blockIdx.x == 0) {
    if (amax_out) *amax_out = a;
    if (scale_out) *scale_out = g.dec;
  }
  fill_rcp_table(rcp_tab, g.dec);
  __syncthreads();
  return g;
}

template <int NW = kWavesPerWG>
__device__ __forceinline__ GScale consume_scales(const Workspace* ws, uint32_t nparts, const float* amax_in,
                                                 float* amax_out, float* scale_out, float* rcp_tab,
                                                 uint32_t first = 0) {
  return scales_from(amax_in ? *amax_in : reduce_partials<NW>(ws, first, nparts), amax_out, scale_out, rcp_tab);
}

// The same in two steps, so that a kernel can issue these loads before its
// bulk loads (loads complete in issue order, so a wait for a later load also
// waits for every earlier one): the first 4 partials of this thread ...
struct PartialsPre {
  float m[4];
};
__device__ __forceinline__ PartialsPre partials_issue(const Workspace* ws, uint32_t nparts, const float* amax_in) {
  PartialsPre p;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const uint32_t i = threadIdx.x + k * kWGThreads;
    p.m[k] = 0.0f;
    if (amax_in == nullptr && i < nparts) p.m[k] = ws->partial[i];
  }
  return p;
}
// ... then the rest, the workgroup maximum and the scales.
__device__ __forceinline__ GScale partials_finish(const PartialsPre& p, const Workspace* ws, uint32_t nparts,
                                                  const float* amax_in, float* amax_out, float* scale_out,
                                                  float* rcp_tab) {
  float a;
  if (amax_in) {
    a = *amax_in;
  } else {
    float m = fmaxf(fmaxf(p.m[0], p.m[1]), fmaxf(p.m[2], p.m[3]));
    for (uint32_t i = threadIdx.x + 4 * kWGThreads; i < nparts; i += kWGThreads) m = fmaxf(m, ws->partial[i]);
    a = wg_max(m);
  }
  return scales_from(a, amax_out, scale_out, rcp_tab);
}

// Amax pass epilogue: the workgroup's maximum into its partial slot (by
// default the workgroup's linear index).
__device__ __forceinline__ void publish_partial(Workspace* ws, float m) {
  m = wg_max(m);
  if (threadIdx.x == 0) ws->partial[blockIdx.y * gridDim.x + blockIdx.x] = m;
}
__device__ __forceinline__ void publish_partial_at(Workspace* ws, float m, uint32_t slot) {
  m = wg_max(m);
  if (threadIdx.x == 0) ws->partial[slot] = m;
}

// ---------------------------------------------------------------- one launch
// The maximum of m over all workgroups of a launch, inside the launch ("CuTeDSL
// at Perplexity", Grid synchronization), for launches of at most kBarrierSlots
// workgroups that are all resident at once. Every workgroup read `epoch` =
// status[0] at its start; it publishes (epoch + 1, its maximum) in its slot
// with one device-scope atomic store, and its first wave polls every slot with
// device-scope atomic loads until all carry epoch + 1 (non-negative floats
// compare like their bit patterns). Workgroup 0 then advances status[0]: every
// workgroup has read the old value before any slot can show the new one. A
// wait is bounded by spin_limit polls; past it status[1] is set and the
// maximum of the slots seen is used (the output is then unspecified, but every
// wave ends). All threads call; m >= 0.
__device__ __forceinline__ float grid_max(Workspace* ws, uint32_t epoch, float m, uint32_t spin_limit) {
  __shared__ float gm;
  m = wg_max(m);
  const uint32_t tag = epoch + 1u;
  if (threadIdx.x == 0)
    __hip_atomic_store(&ws->slot[blockIdx.x], ((uint64_t)tag << 32) | __float_as_uint(m), __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
  if (threadIdx.x < 64) {
    const uint32_t lane = threadIdx.x;
    bool done = lane >= gridDim.x;
    uint64_t v = 0;
    for (uint32_t spins = 0;; ++spins) {
      if (!done) {
        v = __hip_atomic_load(&ws->slot[lane], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        done = (uint32_t)(v >> 32) == tag;
      }
      if (__all(done)) break;
      if (spins >= spin_limit) {
        if (lane == 0) __hip_atomic_store(&ws->status[1], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        break;
      }
      __builtin_amdgcn_s_sleep(1);
    }
    const float x = wave_max(lane < gridDim.x ? __uint_as_float((uint32_t)v) : 0.0f);
    if (lane == 0) gm = x;
  }
  __syncthreads();
  if (blockIdx.x == 0 && threadIdx.x == 0)
    __hip_atomic_store(&ws->status[0], tag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return gm;
}

// ---------------------------------------------------------------- XCD order
// The GPU dispatches the workgroups of a launch round-robin over its 8 XCDs
// (workgroup b to XCD b mod 8), and each XCD has its own L2. Tiles that are
// neighbours in a plane share partially written cache lines (a 128-token tile
// writes half a line of columnwise codes and 8 bytes of a scale line);
// written through different L2s those lines reach memory in pieces. Giving
// XCD x the contiguous work items x * chunk .. x * chunk + chunk - 1 keeps
// neighbours on one L2, where the pieces merge. The grid has kXcds * chunk
// workgroups; items past the end are idle.
// (chunk 0: plain order, work item = workgroup index; NVFP4Q_XCD_ORDER=0
// selects it, for comparison.)
constexpr uint32_t kXcds = 8;
__device__ __forceinline__ uint32_t xcd_work_item(uint32_t chunk) {
  return chunk ? (blockIdx.x % kXcds) * chunk + blockIdx.x / kXcds : blockIdx.x;
}
uint32_t xcd_chunk(uint64_t items);     // 0 when the plain order is selected
uint32_t xcd_grid(uint64_t items);      // workgroups to launch for `items` work items


// The codes of one 16-element block held by one lane (fp32 values that are
// bf16 values) under scale code sc: encode multiplier from the table, 16 codes
// in two words (element 2i in the low nibble of byte i). SR draws one Philox
// evaluation for the block: elements 0-3 take word 0, 4-7 word 1, 8-11 word 2,
// 12-15 word 3.
template <bool SR>
__device__ __forceinline__ uint2 encode_with_scale(float v[16], uint32_t sc, const float* rcp_tab, uint64_t blk,
                                                   uint64_t seed, uint32_t offset, uint32_t tag) {
  const float rc = rcp_tab[sc];
#pragma unroll
  for (int i = 0; i < 16; ++i) v[i] = v[i] * rc;
  uint2 out;
  if constexpr (SR) {
    const U4 w = block_random(blk, tag, seed, offset);
    out.x = sr_pack8(v, w.x, w.y);
    out.y = sr_pack8(v + 8, w.z, w.w);
  } else {
    out.x = rtne_pack8(v);
    out.y = rtne_pack8(v + 8);
  }
  return out;
}

// Encode with the block's own scale (from its maximum).
template <bool SR>
__device__ __forceinline__ uint2 encode_block16(float v[16], GScale g, const float* rcp_tab, uint32_t& sc,
                                                uint64_t blk, uint64_t seed, uint32_t offset, uint32_t tag) {
  sc = block_scale(max16_abs(v), g.enc);
  return encode_with_scale<SR>(v, sc, rcp_tab, blk, seed, offset, tag);
}

}  // namespace nvfp4q
