// Measurement probes (built into libnvfp4q_ceilings.so, not part of the C ABI
// in include/): plain kernels with the memory traffic of the library's passes
// and none of their arithmetic, so that the bandwidth a pass of that shape can
// reach on this GPU is measured rather than assumed, plus the two ways of
// putting a grid-wide maximum between reading x and writing codes in one
// launch. Only bench.py --ceilings calls them.
//
//  * read: a wave reads one contiguous span of 64 lanes x U 16-byte loads
//    (U = 8: one 4096-element bf16 row, the amax pass's pattern), grid-stride
//    over spans.
//  * mix: one thread per 16-element block: two adjacent 16-byte loads, an
//    8-byte non-temporal code store and a 1-byte non-temporal scale store
//    (the rowwise encode's traffic), grid-stride over blocks.
//  * rowmix: the same traffic in the rowwise encode pass's layout: rows of
//    4096 bf16, one row per wave, lane l holding block l of each 1024-column
//    superchunk (all eight loads in flight at once), then its 4 code and 4
//    scale stores.
//  * fused: rows of 4096 bf16, one row per wave held in registers: read, a
//    grid-wide maximum through epoch-tagged per-workgroup slots (relaxed
//    device-scope atomics; every wait is bounded), then the mix pass's stores
//    from registers. Only launched when the whole grid is resident at once.
//  * fused_count: the fused probe with other forms of the grid-wide maximum
//    (an arrival counter and an atomic maximum, with or without release and
//    acquire; slots polled all at once; slots read by one workgroup that
//    then raises per-group flags), and with no wait at all (each workgroup's
//    own maximum: the one-launch shape without a barrier).
//  * empty: an empty kernel, launched plainly or as a cooperative launch, for
//    the launch cost of each.
//  * rate: the issue cost of single VALU instructions the encodes lean on:
//    every lane runs eight independent chains of one instruction (inline
//    assembly, so it is exactly that instruction), registers only; the time
//    per wave-instruction and SIMD compares the kinds.
//
// "CuTeDSL at Perplexity", Grid synchronization (an amax before any code is
// written: a kernel boundary or an in-kernel grid barrier).
#include <hip/hip_runtime.h>

#include <cstdint>

namespace {

constexpr int kT = 256;  // threads per workgroup
constexpr int kWaves = kT / 64;

template <int U>
__global__ __launch_bounds__(kT) void k_read(const uint4* __restrict__ x, uint64_t nspans, uint32_t* out) {
  const uint32_t lane = threadIdx.x & 63;
  const uint64_t nw = (uint64_t)gridDim.x * kWaves;
  uint32_t acc = 0;
  for (uint64_t s = (uint64_t)blockIdx.x * kWaves + (threadIdx.x >> 6); s < nspans; s += nw) {
    const uint4* p = x + s * (64 * U) + lane;
    uint4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = p[64 * u];
#pragma unroll
    for (int u = 0; u < U; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  // keeps the loads live; the store happens only for this one value of acc
  if (acc == 0x9E3779B9u) out[blockIdx.x] = acc;
}

__global__ __launch_bounds__(kT) void k_mix(const uint4* __restrict__ x, uint64_t* __restrict__ codes,
                                            uint8_t* __restrict__ scales, uint64_t nblocks) {
  const uint64_t stride = (uint64_t)gridDim.x * kT;
  for (uint64_t b = (uint64_t)blockIdx.x * kT + threadIdx.x; b < nblocks; b += stride) {
    const uint4 a = x[2 * b], c = x[2 * b + 1];
    const uint64_t w = ((uint64_t)(a.x ^ a.y ^ c.x ^ c.y) << 32) | (a.z ^ a.w ^ c.z ^ c.w);
    __builtin_nontemporal_store(w, codes + b);
    __builtin_nontemporal_store((uint8_t)(w ^ (w >> 29)), scales + b);
  }
}

struct BarrierWs {
  uint32_t epoch;  // calls completed; every workgroup of a call reads it before any changes it
  uint32_t err;    // set when a wait gave up
  uint32_t pad[30];
  uint64_t slot[4096];  // (epoch + 1) << 32 | the workgroup's maximum
};

constexpr uint32_t kRowU4 = 512;  // one 4096-element bf16 row in 16-byte units

__device__ __forceinline__ void load_row(const uint4* __restrict__ x, uint32_t row, uint32_t lane, uint4 (&q)[8]) {
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    q[2 * s] = x[(uint64_t)row * kRowU4 + s * 128 + 2 * lane];
    q[2 * s + 1] = x[(uint64_t)row * kRowU4 + s * 128 + 2 * lane + 1];
  }
}

__device__ __forceinline__ void store_row(uint64_t* __restrict__ codes, uint8_t* __restrict__ scales, uint32_t row,
                                          uint32_t lane, const uint4 (&q)[8], uint32_t g) {
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const uint4 a = q[2 * s], c = q[2 * s + 1];
    const uint64_t w = ((uint64_t)(a.x ^ a.y ^ c.x ^ c.y ^ g) << 32) | (a.z ^ a.w ^ c.z ^ c.w);
    const uint64_t b = (uint64_t)row * 256 + s * 64 + lane;  // block index: 256 blocks per row
    __builtin_nontemporal_store(w, codes + b);
    __builtin_nontemporal_store((uint8_t)(w ^ (w >> 29)), scales + b);
  }
}

__global__ __launch_bounds__(kT) void k_rowmix(const uint4* __restrict__ x, uint64_t* __restrict__ codes,
                                               uint8_t* __restrict__ scales) {
  const uint32_t lane = threadIdx.x & 63;
  const uint32_t row = blockIdx.x * kWaves + (threadIdx.x >> 6);
  uint4 q[8];
  load_row(x, row, lane, q);
  store_row(codes, scales, row, lane, q, 0u);
}

__global__ __launch_bounds__(kT) void k_fused(const uint4* __restrict__ x, uint64_t* __restrict__ codes,
                                              uint8_t* __restrict__ scales, BarrierWs* ws, uint32_t spin_limit) {
  const uint32_t lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const uint32_t row = blockIdx.x * kWaves + wid;
  // lane l holds block l of each 1024-column superchunk s (two adjacent 16-byte loads)
  uint4 q[8];
  load_row(x, row, lane, q);
  const uint32_t epoch = __hip_atomic_load(&ws->epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  uint32_t m = 0;  // the largest bf16 magnitude pattern (its integer order is the order of |x|)
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const uint32_t w[4] = {q[k].x, q[k].y, q[k].z, q[k].w};
#pragma unroll
    for (int i = 0; i < 4; ++i) m = max(m, max(w[i] & 0x7FFFu, (w[i] >> 16) & 0x7FFFu));
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) m = max(m, (uint32_t)__shfl_xor((int)m, o, 64));
  __shared__ uint32_t red[kWaves];
  __shared__ uint32_t gmax;
  if (lane == 0) red[wid] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t t = red[0];
#pragma unroll
    for (int i = 1; i < kWaves; ++i) t = max(t, red[i]);
    __hip_atomic_store(&ws->slot[blockIdx.x], ((uint64_t)(epoch + 1) << 32) | t, __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
  }
  if (wid == 0) {
    // wave 0 polls every workgroup's slot, 64 at a time, each wait bounded
    uint32_t g = 0, spins = 0;
    for (uint32_t s0 = 0; s0 < gridDim.x; s0 += 64) {
      const uint32_t s = s0 + lane;
      bool done = s >= gridDim.x;
      uint64_t v = 0;
      while (true) {
        if (!done) {
          v = __hip_atomic_load(&ws->slot[s], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          done = (uint32_t)(v >> 32) == epoch + 1;
        }
        if (__all(done)) break;
        if (++spins > spin_limit) {
          if (lane == 0) __hip_atomic_store(&ws->err, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          break;
        }
        __builtin_amdgcn_s_sleep(2);
      }
      if (s < gridDim.x) g = max(g, (uint32_t)v);
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) g = max(g, (uint32_t)__shfl_xor((int)g, o, 64));
    if (lane == 0) gmax = g;
  }
  __syncthreads();
  const uint32_t g = gmax;
  // every workgroup has read the epoch before any slot could hold epoch + 1
  if (blockIdx.x == 0 && threadIdx.x == 0)
    __hip_atomic_store(&ws->epoch, epoch + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  store_row(codes, scales, row, lane, q, g);
}

// Other forms of the grid-wide maximum, by mode:
//  0: one arrival counter and one atomic maximum per call (set p = epoch & 1;
//     each call clears the set the next call uses), release on the arrival
//     and acquire after the wait;
//  1: no wait (each workgroup's own maximum): the one-launch shape's floor;
//  2: as 0 with relaxed atomics only: the maximum's atomic returns before the
//     arrival is issued, and the final maximum is read by an atomic;
//  3: per-workgroup slots as in k_fused, wave 0 polling all of them at once
//     (every slot load of a round in flight together);
//  4: per-workgroup slots read by workgroup 0 only, which then writes the
//     maximum to one flag per 64 workgroups (each on its own 128-byte line);
//     the others poll their group's flag.
struct CountWs {
  uint32_t epoch;  // calls completed; read by every workgroup before any changes it
  uint32_t err;    // set when a wait gave up
  uint32_t pad[30];
  uint32_t count[2][32];  // arrivals of the call using the set (one 128-byte line each)
  uint32_t maxv[2][32];   // that call's maximum (bf16 magnitude pattern)
  uint64_t flag[64][16];  // modes 4: (epoch + 1) << 32 | maximum, one line per 64 workgroups
  uint64_t slot[4096];    // modes 3, 4: (epoch + 1) << 32 | the workgroup's maximum
};

__device__ __forceinline__ void give_up(CountWs* ws) {
  __hip_atomic_store(&ws->err, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__global__ __launch_bounds__(kT) void k_fused_count(const uint4* __restrict__ x, uint64_t* __restrict__ codes,
                                                    uint8_t* __restrict__ scales, CountWs* ws, uint32_t spin_limit,
                                                    int mode) {
  const uint32_t lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const uint32_t row = blockIdx.x * kWaves + wid;
  uint4 q[8];
  load_row(x, row, lane, q);
  uint32_t m = 0;
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const uint32_t w[4] = {q[k].x, q[k].y, q[k].z, q[k].w};
#pragma unroll
    for (int i = 0; i < 4; ++i) m = max(m, max(w[i] & 0x7FFFu, (w[i] >> 16) & 0x7FFFu));
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) m = max(m, (uint32_t)__shfl_xor((int)m, o, 64));
  __shared__ uint32_t red[kWaves];
  __shared__ uint32_t gmax;
  if (lane == 0) red[wid] = m;
  __syncthreads();
  uint32_t t = red[0];
#pragma unroll
  for (int i = 1; i < kWaves; ++i) t = max(t, red[i]);
  uint32_t g = t;
  if (mode != 1) {
    if (wid == 0) {
      const uint32_t epoch = __hip_atomic_load(&ws->epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      const uint32_t p = epoch & 1u, tag = epoch + 1u;
      if (mode == 0 || mode == 2) {
        if (lane == 0) {
          if (mode == 0) {
            __hip_atomic_fetch_max(&ws->maxv[p][0], t, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_fetch_add(&ws->count[p][0], 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
          } else {
            // the arrival depends on the maximum's returned value: it is issued after that atomic is done
            const uint32_t o = __hip_atomic_fetch_max(&ws->maxv[p][0], t, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_fetch_add(&ws->count[p][0], 1u + (o == 0xFFFFFFFFu), __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
          }
        }
        for (uint32_t spins = 0;; ++spins) {
          const uint32_t c = __hip_atomic_load(&ws->count[p][0], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          if (c >= gridDim.x) break;
          if (spins >= spin_limit) {
            if (lane == 0) give_up(ws);
            break;
          }
          __builtin_amdgcn_s_sleep(1);
        }
        if (mode == 0) {
          __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
          g = __hip_atomic_load(&ws->maxv[p][0], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        } else {
          g = __hip_atomic_fetch_or(&ws->maxv[p][0], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        // every workgroup has read the epoch and arrived: clear the next call's set
        if (blockIdx.x == 0 && lane == 0) {
          __hip_atomic_store(&ws->count[p ^ 1u][0], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          __hip_atomic_store(&ws->maxv[p ^ 1u][0], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          __hip_atomic_store(&ws->epoch, tag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
      } else {
        if (lane == 0)
          __hip_atomic_store(&ws->slot[blockIdx.x], ((uint64_t)tag << 32) | t, __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
        if (mode == 3 || blockIdx.x == 0) {
          // all of the grid's slots (at most 64 per lane) in flight at once, each round
          const uint32_t per = (gridDim.x + 63) / 64;
          for (uint32_t spins = 0;; ++spins) {
            bool done = true;
            uint32_t mm = 0;
            for (uint32_t k = 0; k < per; ++k) {
              const uint32_t s = k * 64 + lane;
              if (s < gridDim.x) {
                const uint64_t v = __hip_atomic_load(&ws->slot[s], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                done = done && (uint32_t)(v >> 32) == tag;
                mm = max(mm, (uint32_t)v);
              }
            }
            g = mm;
            if (__all(done)) break;
            if (spins >= spin_limit) {
              if (lane == 0) give_up(ws);
              break;
            }
            __builtin_amdgcn_s_sleep(1);
          }
#pragma unroll
          for (int o = 32; o >= 1; o >>= 1) g = max(g, (uint32_t)__shfl_xor((int)g, o, 64));
          if (mode == 4) {
            const uint32_t ngroups = (gridDim.x + 63) / 64;
            if (lane < ngroups)
              __hip_atomic_store(&ws->flag[lane][0], ((uint64_t)tag << 32) | g, __ATOMIC_RELAXED,
                                 __HIP_MEMORY_SCOPE_AGENT);
          }
          // every slot carries this call's tag: every workgroup has read the epoch
          if (blockIdx.x == 0 && lane == 0)
            __hip_atomic_store(&ws->epoch, tag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        } else {
          for (uint32_t spins = 0;; ++spins) {
            const uint64_t v =
                __hip_atomic_load(&ws->flag[blockIdx.x / 64][0], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            g = (uint32_t)v;
            if ((uint32_t)(v >> 32) == tag) break;
            if (spins >= spin_limit) {
              if (lane == 0) give_up(ws);
              break;
            }
            __builtin_amdgcn_s_sleep(1);
          }
        }
      }
      if (lane == 0) gmax = g;
    }
    __syncthreads();
    g = gmax;
  }
  store_row(codes, scales, row, lane, q, g);
}

__global__ void k_empty() {}

// ---------------------------------------------------------------- issue rate
constexpr int kRateKinds = 16;
const char* const kRateNames[kRateKinds] = {
    "v_add_u32", "v_bitop3_b32", "v_mad_u64_u32", "v_mul_hi_u32", "v_mul_lo_u32", "v_mul_f32", "v_fma_f32",
    "v_max3_f32", "v_lshlrev_b32", "v_perm_b32", "v_dot2c_f32_bf16", "v_add_f32_dpp", "v_cvt_pk_bf16_f32",
    "v_cvt_pk_fp8_f32", "v_cvt_scalef32_pk_fp4_f32", "v_cvt_scalef32_sr_pk_fp4_f32"};

#define RATE8(S) S(0) S(1) S(2) S(3) S(4) S(5) S(6) S(7)
template <int K>
__global__ __launch_bounds__(kT) void k_rate(uint32_t seed, uint32_t iters, uint32_t* out) {
  uint32_t a[8];
  uint64_t w[8];
  float f[8];
  const uint32_t t = threadIdx.x + blockIdx.x * kT + seed;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = t * (i + 3) + i;
    w[i] = (uint64_t)a[i] << 7;
    f[i] = (float)a[i] * 1e-3f;
  }
  const uint32_t M = 0xD2511F53u ^ seed, N = 0x9E3779B9u + seed;
  for (uint32_t it = 0; it < iters; ++it) {
#define R0(i) asm volatile("v_add_u32 %0, %0, %1" : "+v"(a[i]) : "v"(N));
#define R1(i) asm volatile("v_bitop3_b32 %0, %0, %1, %2 bitop3:0x96" : "+v"(a[i]) : "v"(N), "v"(M));
#define R2(i) asm volatile("v_mad_u64_u32 %0, vcc, %1, %2, %0" : "+v"(w[i]) : "v"(a[i]), "v"(M) : "vcc");
#define R3(i) asm volatile("v_mul_hi_u32 %0, %0, %1" : "+v"(a[i]) : "v"(M));
#define R4(i) asm volatile("v_mul_lo_u32 %0, %0, %1" : "+v"(a[i]) : "v"(M));
#define R5(i) asm volatile("v_mul_f32 %0, %0, %1" : "+v"(f[i]) : "v"(f[(i + 1) & 7]));
#define R6(i) asm volatile("v_fma_f32 %0, %0, %1, %2" : "+v"(f[i]) : "v"(f[(i + 1) & 7]), "v"(f[(i + 2) & 7]));
#define R7(i) asm volatile("v_max3_f32 %0, %0, %1, %2" : "+v"(f[i]) : "v"(f[(i + 1) & 7]), "v"(f[(i + 2) & 7]));
#define R8(i) asm volatile("v_lshlrev_b32 %0, 16, %0" : "+v"(a[i]));
#define R9(i) asm volatile("v_perm_b32 %0, %0, %1, %2" : "+v"(a[i]) : "v"(N), "v"(M));
#define R10(i) asm volatile("v_dot2c_f32_bf16 %0, %1, %2" : "+v"(f[i]) : "v"(a[i]), "v"(N));
#define R11(i) asm volatile("v_add_f32_dpp %0, %0, %0 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf" : "+v"(f[i]));
#define R12(i) asm volatile("v_cvt_pk_bf16_f32 %0, %1, %2" : "=v"(a[i]) : "v"(f[i]), "v"(f[(i + 1) & 7]));
#define R13(i) asm volatile("v_cvt_pk_fp8_f32 %0, %1, %2" : "+v"(a[i]) : "v"(f[i]), "v"(f[(i + 1) & 7]));
#define R14(i) asm volatile("v_cvt_scalef32_pk_fp4_f32 %0, %1, %2, %3" : "+v"(a[i]) : "v"(f[i]), "v"(f[(i + 1) & 7]), "v"(1.0f));
#define R15(i) asm volatile("v_cvt_scalef32_sr_pk_fp4_f32 %0, %1, %2, %3" : "+v"(a[i]) : "v"(w[i]), "v"(N), "v"(1.0f));
    if constexpr (K == 0) { RATE8(R0) }
    if constexpr (K == 1) { RATE8(R1) }
    if constexpr (K == 2) { RATE8(R2) }
    if constexpr (K == 3) { RATE8(R3) }
    if constexpr (K == 4) { RATE8(R4) }
    if constexpr (K == 5) { RATE8(R5) }
    if constexpr (K == 6) { RATE8(R6) }
    if constexpr (K == 7) { RATE8(R7) }
    if constexpr (K == 8) { RATE8(R8) }
    if constexpr (K == 9) { RATE8(R9) }
    if constexpr (K == 10) { RATE8(R10) }
    if constexpr (K == 11) { RATE8(R11) }
    if constexpr (K == 12) { RATE8(R12) }
    if constexpr (K == 13) { RATE8(R13) }
    if constexpr (K == 14) { RATE8(R14) }
    if constexpr (K == 15) { RATE8(R15) }
  }
  uint32_t r = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) r ^= a[i] ^ (uint32_t)w[i] ^ (uint32_t)(w[i] >> 32) ^ __float_as_uint(f[i]);
  out[blockIdx.x * kT + threadIdx.x] = r;
}

template <int K>
void launch_rate(uint32_t grid, uint32_t iters, uint32_t* out, hipStream_t s) {
  hipLaunchKernelGGL(k_rate<K>, dim3(grid), dim3(kT), 0, s, 1u, iters, out);
}
typedef void (*RateLaunch)(uint32_t, uint32_t, uint32_t*, hipStream_t);
const RateLaunch kRateLaunch[kRateKinds] = {
    launch_rate<0>, launch_rate<1>, launch_rate<2>,  launch_rate<3>,  launch_rate<4>,  launch_rate<5>,
    launch_rate<6>, launch_rate<7>, launch_rate<8>,  launch_rate<9>,  launch_rate<10>, launch_rate<11>,
    launch_rate<12>, launch_rate<13>, launch_rate<14>, launch_rate<15>};

uint32_t grid_for(uint64_t items, uint64_t per_wg, uint32_t cap) {
  uint64_t g = (items + per_wg - 1) / per_wg;
  if (g > cap) g = cap;
  return g ? (uint32_t)g : 1u;
}

}  // namespace

extern "C" {

// Read `bytes` (a multiple of 8 KiB) at x; out: one word per workgroup (at
// most 4096), written only for one particular value. Returns a hipError_t.
int ceil_read(const void* x, uint64_t bytes, void* out, void* stream) {
  const uint64_t nspans = bytes / (64 * 8 * 16);
  if (nspans == 0 || bytes % (64 * 8 * 16)) return (int)hipErrorInvalidValue;
  const uint32_t grid = grid_for(nspans, kWaves, 4096);
  hipLaunchKernelGGL((k_read<8>), dim3(grid), dim3(kT), 0, (hipStream_t)stream, (const uint4*)x, nspans,
                     (uint32_t*)out);
  return (int)hipGetLastError();
}

// The rowwise encode's traffic for `nblocks` 16-element bf16 blocks at x:
// codes [nblocks] x 8 bytes, scales [nblocks] bytes.
int ceil_mix(const void* x, uint64_t nblocks, void* codes, void* scales, void* stream) {
  if (nblocks == 0) return (int)hipErrorInvalidValue;
  const uint32_t grid = grid_for(nblocks, kT, 65536);
  hipLaunchKernelGGL(k_mix, dim3(grid), dim3(kT), 0, (hipStream_t)stream, (const uint4*)x, (uint64_t*)codes,
                     (uint8_t*)scales, nblocks);
  return (int)hipGetLastError();
}

// The rowwise encode pass's layout of the same traffic: rows x 4096 bf16 (rows a
// multiple of 4), one row per wave; codes [rows * 256] x 8 bytes, scales
// [rows * 256] bytes.
int ceil_rowmix(const void* x, uint32_t rows, void* codes, void* scales, void* stream) {
  if (rows == 0 || rows % kWaves) return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(k_rowmix, dim3(rows / kWaves), dim3(kT), 0, (hipStream_t)stream, (const uint4*)x,
                     (uint64_t*)codes, (uint8_t*)scales);
  return (int)hipGetLastError();
}

// Bytes of the barrier workspace of ceil_fused (zero-filled before its first use).
uint64_t ceil_fused_ws_bytes(void) { return sizeof(BarrierWs); }

// One launch: read rows x 4096 bf16, grid-wide maximum, then the mix stores
// (codes [rows * 256] x 8 bytes, scales [rows * 256] bytes). rows must be a
// multiple of 4 with rows / 4 workgroups all resident at once (checked from
// the occupancy of the kernel; hipErrorCooperativeLaunchTooLarge otherwise)
// and at most 4 * 4096. A wait that exceeds spin_limit polls sets the
// workspace's err word and gives up.
int ceil_fused(const void* x, uint32_t rows, void* codes, void* scales, void* ws, uint32_t spin_limit,
               void* stream) {
  if (rows == 0 || rows % kWaves || rows / kWaves > 4096) return (int)hipErrorInvalidValue;
  const uint32_t grid = rows / kWaves;
  int dev = 0, per_cu = 0, cus = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e == hipSuccess) e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, k_fused, kT, 0);
  if (e != hipSuccess) return (int)e;
  if ((uint64_t)per_cu * cus < grid) return (int)hipErrorCooperativeLaunchTooLarge;
  hipLaunchKernelGGL(k_fused, dim3(grid), dim3(kT), 0, (hipStream_t)stream, (const uint4*)x, (uint64_t*)codes,
                     (uint8_t*)scales, (BarrierWs*)ws, spin_limit);
  return (int)hipGetLastError();
}

// Bytes of the workspace of ceil_fused_count (zero-filled before its first use).
uint64_t ceil_fused_count_ws_bytes(void) { return sizeof(CountWs); }

// ceil_fused with another form of the grid-wide maximum (mode 0, 2, 3, 4 as
// listed at k_fused_count), or with no wait at all (mode 1: each workgroup's
// own maximum). Same limits.
int ceil_fused_count(const void* x, uint32_t rows, void* codes, void* scales, void* ws, uint32_t spin_limit,
                     int mode, void* stream) {
  if (rows == 0 || rows % kWaves || rows / kWaves > 4096 || mode < 0 || mode > 4)
    return (int)hipErrorInvalidValue;
  const uint32_t grid = rows / kWaves;
  int dev = 0, per_cu = 0, cus = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e == hipSuccess) e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, k_fused_count, kT, 0);
  if (e != hipSuccess) return (int)e;
  if ((uint64_t)per_cu * cus < grid) return (int)hipErrorCooperativeLaunchTooLarge;
  hipLaunchKernelGGL(k_fused_count, dim3(grid), dim3(kT), 0, (hipStream_t)stream, (const uint4*)x,
                     (uint64_t*)codes, (uint8_t*)scales, (CountWs*)ws, spin_limit, mode);
  return (int)hipGetLastError();
}

// Issue-rate probe: the number of instruction kinds, each kind's name, and
// one launch of kind `kind` (grid x 256 threads, `iters` iterations of 8
// instructions per lane; out: grid * 256 words).
int ceil_rate_kinds(void) { return kRateKinds; }
const char* ceil_rate_name(int kind) { return kind >= 0 && kind < kRateKinds ? kRateNames[kind] : nullptr; }
int ceil_rate(int kind, uint32_t grid, uint32_t iters, void* out, void* stream) {
  if (kind < 0 || kind >= kRateKinds || grid == 0) return (int)hipErrorInvalidValue;
  kRateLaunch[kind](grid, iters, (uint32_t*)out, (hipStream_t)stream);
  return (int)hipGetLastError();
}

// n launches of an empty kernel of `grid` x 256 threads, plain (coop 0) or
// cooperative (coop 1), back to back on `stream`.
int ceil_empty(uint32_t n, uint32_t grid, int coop, void* stream) {
  for (uint32_t i = 0; i < n; ++i) {
    hipError_t e;
    if (coop) {
      e = hipLaunchCooperativeKernel((const void*)k_empty, dim3(grid), dim3(kT), nullptr, 0, (hipStream_t)stream);
    } else {
      hipLaunchKernelGGL(k_empty, dim3(grid), dim3(kT), 0, (hipStream_t)stream);
      e = hipGetLastError();
    }
    if (e != hipSuccess) return (int)e;
  }
  return (int)hipSuccess;
}

}  // extern "C"
