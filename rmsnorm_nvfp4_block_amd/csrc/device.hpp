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
// Self-resetting device state. Every counter and accumulator is zero between
// calls: the last workgroup of a reduction returns it to zero. Result slots are
// written before they are read within a call and carry no state across calls.
struct Workspace {
  uint32_t count;          // arrival counter of the last-workgroup reduction
  uint32_t bar_count;      // grid-barrier arrival counter
  uint32_t bar_gen;        // grid-barrier generation (monotone, wraps)
  uint32_t status;         // sticky device-side error flags (bit 0: barrier timeout)
  uint32_t amax_bits[64];  // per-tensor / per-group amax accumulators (fp32 bits, >= 0)
  float enc[64];           // S_enc per tensor / group (result slot)
  float dec[64];           // S_dec per tensor / group (result slot)
  float amax[64];          // amax used per tensor / group (result slot)
  int32_t poff[72];        // padded group offsets (result slot)
  uint32_t rsv[1024 - 4 - 64 * 4 - 72];
};
static_assert(sizeof(Workspace) == 4096, "workspace layout");

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

// ---------------------------------------------------------------- FP8 / FP4
// E4M3 code of a non-negative float: round to nearest even, saturating at 448.
// v_cvt_pk_fp8_f32 rounds to nearest even over [0, 448] including subnormals
// (checked exhaustively); the clamp supplies the saturation.
__device__ __forceinline__ uint32_t e4m3_code(float s) {
  s = fminf(s, 448.0f);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(s, s, 0, false) & 0xFFu;
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

// Block scale code: E4M3(RN(RN(bmax / 6) * S_enc)).
__device__ __forceinline__ uint32_t block_scale(float bmax, float s_enc) {
  float q = bmax / 6.0f;
  return e4m3_code(q * s_enc);
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
__device__ __forceinline__ U4 philox10(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3,
                                       uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    uint64_t p0 = (uint64_t)0xD2511F53u * c0;
    uint64_t p1 = (uint64_t)0xCD9E8D57u * c2;
    uint32_t n0 = (uint32_t)(p1 >> 32) ^ c1 ^ k0;
    uint32_t n2 = (uint32_t)(p0 >> 32) ^ c3 ^ k1;
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
// kept as in round-to-nearest. v_cvt_scalef32_sr_pk_fp4_f32 adds its 32-bit
// random operand to the bits below the E2M1 step and keeps the carry; with the
// byte in bits 31..24 and zeros below, that is exactly the rule above (checked
// against the definition on every float32 input and every byte). Its second
// source reuses the same random bits, so each element gets its own instruction
// with a zero partner. The instruction writes only the selected byte of its
// destination, while the compiler treats the whole register as written, so
// only byte 0 of the result is meaningful: the element's code in the low
// nibble and the zero partner's code (0) in the high nibble. Bytes are gathered
// with v_perm_b32, which reads byte 0 alone.
__device__ __forceinline__ uint32_t e2m1_sr(float v, uint32_t rand_top) {
  f32x2 ab = {v, 0.0f};
  return __builtin_amdgcn_cvt_scalef32_sr_pk_fp4_f32(0u, ab, rand_top, 1.0f, 0);
}

// Byte b of w moved to bits 31..24, zeros below (v_perm_b32 selects bytes of
// its second operand with indices 0..3, of its first with 4..7; 0x0C yields a
// zero byte).
template <int B>
__device__ __forceinline__ uint32_t byte_to_top(uint32_t w) {
  return __builtin_amdgcn_perm(0u, w, ((uint32_t)B << 24) | 0x000C0C0Cu);
}

// Byte 0 of a, b, c, d gathered into bytes 0..3.
__device__ __forceinline__ uint32_t gather_b0(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
  const uint32_t ab = __builtin_amdgcn_perm(b, a, 0x0C0C0400u);
  const uint32_t cd = __builtin_amdgcn_perm(d, c, 0x0C0C0400u);
  return __builtin_amdgcn_perm(cd, ab, 0x05040100u);
}

// Eight SR codes packed in a word (element 2i in the low nibble of byte i).
// Element e takes byte (e & 3) of w0 (e < 4) or of w1 (e >= 4).
__device__ __forceinline__ uint32_t sr_pack8(const float v[8], uint32_t w0, uint32_t w1) {
  const uint32_t ev = gather_b0(e2m1_sr(v[0], byte_to_top<0>(w0)), e2m1_sr(v[2], byte_to_top<2>(w0)),
                                e2m1_sr(v[4], byte_to_top<0>(w1)), e2m1_sr(v[6], byte_to_top<2>(w1)));
  const uint32_t od = gather_b0(e2m1_sr(v[1], byte_to_top<1>(w0)), e2m1_sr(v[3], byte_to_top<3>(w0)),
                                e2m1_sr(v[5], byte_to_top<1>(w1)), e2m1_sr(v[7], byte_to_top<3>(w1)));
  return ev | (od << 4);
}

// Eight RTNE codes packed in a word.
__device__ __forceinline__ uint32_t rtne_pack8(const float v[8]) {
  uint32_t out = 0;
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

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}

__device__ __forceinline__ float max8_abs(const float v[8]) {
  float a = fmaxf(fabsf(v[0]), fabsf(v[1]));
  float b = fmaxf(fabsf(v[2]), fabsf(v[3]));
  float c = fmaxf(fabsf(v[4]), fabsf(v[5]));
  float d = fmaxf(fabsf(v[6]), fabsf(v[7]));
  return fmaxf(fmaxf(a, b), fmaxf(c, d));
}

__device__ __forceinline__ void widen8(const uint4 q, float v[8]) {
  v[0] = bf_lo(q.x); v[1] = bf_hi(q.x);
  v[2] = bf_lo(q.y); v[3] = bf_hi(q.y);
  v[4] = bf_lo(q.z); v[5] = bf_hi(q.z);
  v[6] = bf_lo(q.w); v[7] = bf_hi(q.w);
}

// ---------------------------------------------------------------- atomics
__device__ __forceinline__ void atomic_max_f32_nonneg(uint32_t* p, float v) {
  __hip_atomic_fetch_max(p, __float_as_uint(v), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Last-workgroup election: every workgroup calls this once from thread 0 after
// its atomics; returns true in exactly one workgroup, which then sees all of
// them. The counter is returned to zero by that workgroup.
__device__ __forceinline__ bool arrive_last(uint32_t* count, uint32_t nwg) {
  uint32_t prev = __hip_atomic_fetch_add(count, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
  if (prev == nwg - 1) {
    __hip_atomic_store(count, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return true;
  }
  return false;
}

__device__ __forceinline__ float load_amax(uint32_t* p) {
  return __uint_as_float(__hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
}

}  // namespace nvfp4q
